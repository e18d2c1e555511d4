"""serq_linear's K-split path (few tokens, long K) without allocation.

The skinny kernel splits K across workgroups when the activation rows do not
fit its LDS; the slices' int32 partial sums meet in the library's file-scope
device scratch. These tests call the path through the C ABI: its first call
in a fresh process under HIP graph capture (nothing on it may allocate or
synchronize), and calls in a row whose sizes shrink, so that the second call
runs over scratch still holding the first one's partial sums and counters
that the first one must have returned to zero.
"""

from __future__ import annotations

import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import w4a4_linear_layers_amd as S
from gpu_helpers import check_y, dev, host, sample
from layouts import pack_rq
from oracle import serq_oracle as O
from synth import random_codes

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


def test_split_first_call_under_graph_capture():
    """A fresh process whose first serq_linear call (the 8B down shape at 32
    tokens, a K-split launch) is captured into a HIP graph; three replays
    and eager split calls between them, each bit-exact against the oracle."""
    print("child: split_capture_child.py", flush=True)
    p = subprocess.run([sys.executable, os.path.join(HERE, "split_capture_child.py")], capture_output=True,
                       text=True, timeout=240)
    print(p.stdout[-3000:], p.stderr[-3000:], flush=True)
    assert p.returncode == 0 and p.stdout.strip().endswith("OK")


def _layer(M, K, N, r, bits, seed):
    rng = np.random.default_rng(seed)
    Xc = random_codes(rng, (M, K), bits)
    Wc = random_codes(rng, (K, N), 4)
    Rc = random_codes(rng, (r, N), 4)
    sx = rng.uniform(0.01, 2.0, M).astype(np.float32)
    sw = rng.uniform(0.001, 0.1, N).astype(np.float32)
    sr = rng.uniform(0.0001, 0.01, N).astype(np.float32) if r else np.zeros(N, np.float32)
    Xq = O.pack_int4(Xc) if bits == 4 else Xc.view(np.uint8)
    layer = S.DeviceLayer(K=K, N=N, r=r, perm=None, s_hat_inv=None, Wq=dev(O.pack_int4(Wc.T)), sw=dev(sw),
                          Rq=dev(pack_rq(Rc)), sr=dev(sr))
    return Xc, Wc, Rc, sx, sw, sr, dev(Xq), layer


@pytest.mark.parametrize("bits", [4, 8])
def test_split_calls_in_a_row_shrinking(bits):
    """The 70B down shape at 32 tokens (the largest split: the most partial
    sums), then the 8B down shape at 20 tokens, then a narrow layer at 5
    tokens, back to back on one stream with no synchronization between
    them; every call checked against the oracle (sampled columns of the
    large ones, with the first and last)."""
    shapes = [(32, 28672, 8192, 256), (20, 14336, 4096, 128), (5, 28672 if bits == 4 else 40960, 96, 64)]
    runs = []
    for i, (M, K, N, r) in enumerate(shapes):
        print(f"split call {i}: M={M} K={K} N={N} r={r} a_bits={bits}", flush=True)
        name = S.kernel_name(M, K, N, r, bits)
        assert name in ("decode16", "decode32", "decode16_ksplit", "decode32_ksplit"), name
        assert i == 1 or name.endswith("_ksplit"), name
        Xc, Wc, Rc, sx, sw, sr, xq, layer = _layer(M, K, N, r, bits, seed=100 * i + bits)
        y, am, ar = S.linear(xq, dev(sx), layer, a_bits=bits, out_dtype=torch.float32, debug=True)
        runs.append((Xc, Wc, Rc, sx, sw, sr, r, y, am, ar))
    torch.cuda.synchronize()
    for i, (Xc, Wc, Rc, sx, sw, sr, r, y, am, ar) in enumerate(runs):
        cols = sample(Wc.shape[1], 256, i)
        am_ref, ar_ref = O.linear_int(Xc, Wc[:, cols], Rc[:, cols], r)
        assert np.array_equal(host(am)[:, cols], am_ref), f"call {i}: acc_main"
        assert np.array_equal(host(ar)[:, cols], ar_ref), f"call {i}: acc_res"
        check_y(host(y)[:, cols], am_ref, ar_ref, sx, sw[cols], sr[cols], "f32")
