"""Child process of test_gpu_split.py (run as a script, not collected).

The first serq_linear call of this process takes the skinny kernel's K split
(LLaMA-3-8B down shape, 14336 -> 4096, r = 128, 32 tokens: the activation
rows exceed the kernel's LDS) and is made while torch captures a HIP graph,
so nothing on that path may allocate or synchronize. The graph is then
replayed three times, with eager work in between (the outputs overwritten,
another split-path call of a different shape), and every replay's
accumulators and output are compared with the oracle bit for bit (Y within
the derived tolerance). Prints one line per step; exits non-zero on failure.
"""

from __future__ import annotations

import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import w4a4_linear_layers_amd as S  # noqa: E402
from gpu_helpers import check_y, dev, host  # noqa: E402
from layouts import pack_rq  # noqa: E402
from oracle import serq_oracle as O  # noqa: E402
from synth import random_codes  # noqa: E402


def case(M, K, N, r, seed):
    rng = np.random.default_rng(seed)
    Xc = random_codes(rng, (M, K), 4)
    Wc = random_codes(rng, (K, N), 4)
    Rc = random_codes(rng, (r, N), 4)
    sx = rng.uniform(0.01, 2.0, M).astype(np.float32)
    sw = rng.uniform(0.001, 0.1, N).astype(np.float32)
    sr = rng.uniform(0.0001, 0.01, N).astype(np.float32)
    layer = S.DeviceLayer(K=K, N=N, r=r, perm=None, s_hat_inv=None, Wq=dev(O.pack_int4(Wc.T)), sw=dev(sw),
                          Rq=dev(pack_rq(Rc)), sr=dev(sr))
    am_ref, ar_ref = O.linear_int(Xc, Wc, Rc, r)
    return dict(xq=dev(O.pack_int4(Xc)), sx_h=sx, sx=dev(sx), sw=sw, sr=sr, layer=layer, am=am_ref, ar=ar_ref)


def check(tag, y, am, ar, c):
    assert np.array_equal(host(am), c["am"]), f"{tag}: acc_main differs"
    assert np.array_equal(host(ar), c["ar"]), f"{tag}: acc_res differs"
    check_y(host(y), c["am"], c["ar"], c["sx_h"], c["sw"], c["sr"], "f32")
    print(f"{tag}: bit-exact", flush=True)


def main() -> int:
    M, K, N, r = 32, 14336, 4096, 128
    assert S.kernel_name(M, K, N, r, 4) == "decode32_ksplit", S.kernel_name(M, K, N, r, 4)
    big = case(M, K, N, r, seed=1)
    # a second split-path shape for the eager calls between replays
    M2, K2, N2, r2 = 16, 28672, 200, 64
    assert S.kernel_name(M2, K2, N2, r2, 4) == "decode16_ksplit"
    small = case(M2, K2, N2, r2, seed=2)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    am = torch.empty((M, N), dtype=torch.int32, device="cuda")
    ar = torch.empty((M, N), dtype=torch.int32, device="cuda")
    f = S.lib.serq_linear
    L = big["layer"]

    def call(stream):
        return f(big["xq"].data_ptr(), big["sx"].data_ptr(), 4, L.Wq.data_ptr(), L.sw.data_ptr(),
                 L.Rq.data_ptr(), L.sr.data_ptr(), M, K, N, r, y.data_ptr(), S._lib.SERQ_F32,
                 am.data_ptr(), ar.data_ptr(), stream)

    torch.cuda.synchronize()
    print("capturing the first serq_linear call of the process", flush=True)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        status = call(torch.cuda.current_stream().cuda_stream)
    assert status == 0, S.lib.serq_strerror(status).decode()
    torch.cuda.synchronize()
    for i in range(3):
        y.fill_(float("nan"))
        am.fill_(-1)
        ar.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        check(f"replay {i}", y, am, ar, big)
        ys, ams, ars = S.linear(small["xq"], small["sx"], small["layer"], a_bits=4, out_dtype=torch.float32,
                                debug=True)
        torch.cuda.synchronize()
        check(f"eager split call after replay {i}", ys, ams, ars, small)
    print("OK", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
