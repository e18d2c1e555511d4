"""GPU parity of the MXFP4 layer: serq_quant_act_mx and serq_linear_mx
against the oracle.

Bit-exact: the FP4 codes and E8M0 bytes of the activations. The fp32
accumulators: bit-exact where every block of a row pair shares one scale
(E2M1 products are multiples of 1/4 and the partial sums stay far below
2^24 quarters, so no sum can round), and otherwise within the summation
bound |err| <= (K/32 + 64) 2^-24 sum |terms| (one rounding per accumulation
step of the fp32 matrix instruction, with room for rounded partial sums
inside a step). Y = fl(acc_main + acc_res) within that bound plus one
rounding of the sum (and one bf16 spacing for bf16 output).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import w4a4_linear_layers_amd as S
from gpu_helpers import bf16_bits_to_f32, bf16_spacing, bf16_tensor, dev, host, sample
from oracle import serq_oracle as O
from synth import make_layer, round_to_bf16_bits, workload_layer

pytestmark = pytest.mark.gpu


def _sync():
    torch.cuda.synchronize()


def _mx_input(M, K, dtype, seed):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K)).astype(np.float32)
    X[:, rng.choice(K, max(1, K // 100), replace=False)] *= 50
    if M > 1:
        X[1] = 0.0                                    # zero row: exponent -127, zero codes
    if M > 2:
        X[2, :32] = 0.0                               # one zero block
        X[2, 32:64] *= np.float32(1e30)               # a block of huge values
        X[2, 64:96] *= np.float32(1e-30)              # and one of tiny ones
    if M > 3:
        # exact ties: E2M1 midpoints times a power of two (amax 7.5 -> e = 0)
        mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.5], np.float32)
        X[3] = np.resize(np.concatenate([mids, -mids]), K)
    sinv = np.exp2(rng.integers(-3, 3, K)).astype(np.float32)      # powers of two keep the ties exact
    sinv[rng.choice(K, K // 4, replace=False)] = np.exp(rng.uniform(-2, 1, K // 4)).astype(np.float32)
    if M > 3:
        sinv[:] = np.where(np.arange(K) < 32, np.float32(1.0), sinv)
    if dtype == "bf16":
        bits = round_to_bf16_bits(X).reshape(M, K)
        return bf16_bits_to_f32(bits), bf16_tensor(bits), sinv
    return X, dev(X), sinv


@pytest.mark.parametrize("M,K", [(1, 32), (5, 64), (33, 4096), (128, 14336), (7, 28672), (300, 1024), (4, 96)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quant_act_mx_bit_exact(M, K, dtype):
    X, Xt, sinv = _mx_input(M, K, dtype, seed=M + K)
    xq, xsc = S.quant_act_mx(Xt, dev(sinv))
    _sync()
    ref = O.quant_act_mx(X, sinv)
    assert np.array_equal(host(xsc), ref["sc"])
    got = host(xq)
    assert np.array_equal(got, ref["packed"]), np.argwhere(got != ref["packed"])[:5]


def _random_mx(rng, rows, k, e_lo, e_hi):
    codes = rng.integers(0, 16, (rows, k)).astype(np.uint8)
    e = rng.integers(e_lo, e_hi + 1, (rows, k // 32)).astype(np.int64)
    return codes, e


def _check_acc(got, want, mag, K):
    tol = (K / 32 + 64) * 2.0 ** -24 * mag
    err = np.abs(got.astype(np.float64) - want)
    assert (err <= tol).all(), (float((err / np.maximum(tol, 1e-300)).max()), np.unravel_index(np.argmax(err - tol), err.shape))


def _check_y(y, out, mag, K, dt):
    y64 = out["y64"]
    tol = (K / 32 + 64) * 2.0 ** -24 * mag + 2.0 ** -24 * np.abs(y64)
    if dt == "bf16":
        yf = bf16_bits_to_f32(y).astype(np.float64)
        tol = tol + bf16_spacing(yf.astype(np.float32))
    else:
        yf = y.astype(np.float64)
    assert (np.abs(yf - y64) <= tol).all()


@pytest.mark.parametrize("M,K,N,r,uniform", [
    (128, 4096, 128, 64, True), (200, 1024, 300, 32, True),          # one shared scale: exact sums
    (4096, 256, 4096, 96, True),                                     # the 256 x 256 pipelined tile
    (1, 64, 32, 32, False), (37, 320, 200, 96, False), (130, 1024, 260, 0, False),   # K % 128: plain kernel
    (256, 4096, 512, 256, False), (300, 2048, 1000, 2048, False), (64, 96, 130, 64, False),
    (4100, 384, 4104, 128, False), (3, 128, 8, 32, False),         # ragged 256 tiles; one k-tile
    # one or two tokens: the GEMV
    (1, 4096, 256, 64, True),                                        # one shared scale: exact sums
    (2, 384, 100, 96, False),        # a half line at the rows' end, N % 8 != 0, three residual blocks
    (2, 1024, 72, 1024, False),      # r = K: four residual lines
    (1, 28672, 24, 256, False),      # long rows
    (2, 512, 8200, 32, False),       # four-wave workgroups (many row octets), ragged N
    (1, 2048, 4104, 0, False),       # r = 0
    # three to sixteen tokens on layers narrower than 16384 channels: the skinny kernel
    (4, 1024, 72, 1024, False),      # r = K: eight residual chunks
    (3, 28672, 24, 256, False),      # long rows
    (8, 1024, 300, 96, False),       # eight tokens
    (6, 4096, 64, 64, True),         # six tokens, one shared scale: exact sums
    (16, 4096, 4096, 64, True),      # one shared scale: exact sums
    (13, 1152, 300, 96, False),      # nine chunks, a partial residual chunk, ragged N
    (16, 384, 50, 384, False),       # r = K: three residual chunks
    (10, 128, 40, 0, False),         # one chunk (most waves idle), r = 0
    (7, 14336, 100, 128, False),     # fourteen chunks per wave (several rounds of loads in flight)
    (2, 256, 16400, 32, False),      # two tokens on a wide layer: the tile kernel
])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_linear_mx_vs_oracle(M, K, N, r, uniform, out):
    """Random FP4 codes and exponents (ragged M and N, r = 0, an odd number
    of residual blocks, r = K)."""
    rng = np.random.default_rng(M * 7 + K + N + r)
    lo, hi = (0, 0) if uniform else (-20, 20)
    Xc, Xe = _random_mx(rng, M, K, lo, hi)
    Wc, We = _random_mx(rng, N, K, lo, hi)
    Rc, Re = _random_mx(rng, N, r, lo - 4, hi - 4) if r else (np.zeros((N, 0), np.uint8), np.zeros((N, 0), np.int64))
    layer = dict(N=N, r=r, Wq_codes=Wc, We=We, Rq_codes=Rc, Re=Re)
    q = dict(codes=Xc, e=Xe)
    ref = O.linear_mx(q, layer)
    L = S.MxLayer(K=K, N=N, r=r, perm=None, s_hat_inv=None, Wq=dev(O.pack_fp4(Wc)), Wsc=dev((We + 127).astype(np.uint8)),
                  Rq=dev(O.pack_fp4(Rc)), Rsc=dev((Re + 127).astype(np.uint8)))
    odt = torch.float32 if out == "f32" else torch.bfloat16
    y, am, ar = S.linear_mx(dev(O.pack_fp4(Xc)), dev((Xe + 127).astype(np.uint8)), L, out_dtype=odt, debug=True)
    y2 = S.linear_mx(dev(O.pack_fp4(Xc)), dev((Xe + 127).astype(np.uint8)), L, out_dtype=odt)
    _sync()
    if uniform:
        assert np.array_equal(host(am).astype(np.float64), ref["acc_main"])
        assert np.array_equal(host(ar).astype(np.float64), ref["acc_res"])
    else:
        mag_main = np.abs(O.linear_mx(dict(codes=Xc, e=Xe), dict(layer, r=0))["mag"])
        _check_acc(host(am), ref["acc_main"], mag_main, K)
        _check_acc(host(ar), ref["acc_res"], ref["mag"], r)
    _check_y(host(y), ref, ref["mag"], K, out)
    assert np.array_equal(host(y), host(y2))                     # the debug outputs change nothing


@pytest.mark.slow
@pytest.mark.parametrize("M", [16, 300, 2048])
def test_workload_q_proj_mx(M):
    """The q_proj-shaped layer in MXFP4 end to end: host calibration bit for
    bit against the oracle, GPU activation codes and exponents bit for bit on
    every row, accumulators and Y within the bound on every output."""
    li = workload_layer("q_proj", "q_proj")
    r = 64
    L = S.calibrate_mx(li.W_bits, li.act_absmax, r=r)
    R = O.calibrate_mx(li.W, li.act_absmax, r=r)
    for k in ("Wq", "Wsc", "Rq", "Rsc"):
        assert np.array_equal(getattr(L, k), R[k]), k
    D = L.to("cuda")
    xq, xsc = S.quant_act_mx(bf16_tensor(li.X_bits[:M][:, L.perm]), D)
    y, am, ar = S.linear_mx(xq, xsc, D, debug=True)
    _sync()
    q = O.quant_act_mx(li.X[:M][:, L.perm], L.s_hat_inv)
    assert np.array_equal(host(xq), q["packed"]) and np.array_equal(host(xsc), q["sc"])
    ref = O.linear_mx(q, R)
    mag_main = O.linear_mx(q, dict(R, r=0))["mag"]
    _check_acc(host(am), ref["acc_main"], mag_main, li.K)
    _check_y(host(y), ref, ref["mag"], li.K, "bf16")
    # the method's point on outlier data: the compensated MX layer is closer
    # to the exact product than MX without the residual
    exact = li.X[:M].astype(np.float64) @ li.W.astype(np.float64)
    e_with = np.linalg.norm(ref["y64"] - exact)
    e_without = np.linalg.norm(ref["acc_main"] - exact)
    assert e_with < e_without


def test_linear_mx_unaligned_exponents():
    """Exponent arrays at an odd address take the plain kernel: same results."""
    rng = np.random.default_rng(5)
    M, K, N = 64, 512, 96
    Xc, Xe = _random_mx(rng, M, K, -3, 3)
    Wc, We = _random_mx(rng, N, K, -3, 3)
    wsc = torch.zeros(N * K // 32 + 1, dtype=torch.uint8, device="cuda")
    wsc[1:] = dev((We + 127).astype(np.uint8).ravel())
    xsc = torch.zeros(M * K // 32 + 1, dtype=torch.uint8, device="cuda")
    xsc[1:] = dev((Xe + 127).astype(np.uint8).ravel())
    L = S.MxLayer(K=K, N=N, r=0, perm=None, s_hat_inv=None, Wq=dev(O.pack_fp4(Wc)), Wsc=wsc[1:].view(N, K // 32),
                  Rq=None, Rsc=None)
    xq = dev(O.pack_fp4(Xc))
    y = S.linear_mx(xq, xsc[1:].view(M, K // 32), L, out_dtype=torch.float32)
    L2 = S.MxLayer(K=K, N=N, r=0, perm=None, s_hat_inv=None, Wq=L.Wq, Wsc=dev((We + 127).astype(np.uint8)),
                   Rq=None, Rsc=None)
    y2 = S.linear_mx(xq, dev((Xe + 127).astype(np.uint8)), L2, out_dtype=torch.float32)
    _sync()
    ref = O.linear_mx(dict(codes=Xc, e=Xe), dict(N=N, r=0, Wq_codes=Wc, We=We))
    _check_y(host(y), ref, ref["mag"], K, "f32")
    _check_y(host(y2), ref, ref["mag"], K, "f32")


def test_linear_mx_empty_and_side_stream():
    rng = np.random.default_rng(3)
    Xc, Xe = _random_mx(rng, 40, 256, -3, 3)
    Wc, We = _random_mx(rng, 64, 256, -3, 3)
    L = S.MxLayer(K=256, N=64, r=0, perm=None, s_hat_inv=None, Wq=dev(O.pack_fp4(Wc)),
                  Wsc=dev((We + 127).astype(np.uint8)), Rq=None, Rsc=None)
    xq, xsc = dev(O.pack_fp4(Xc)), dev((Xe + 127).astype(np.uint8))
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y = S.linear_mx(xq, xsc, L, out_dtype=torch.float32)
    s.synchronize()
    ref = O.linear_mx(dict(codes=Xc, e=Xe), dict(N=64, r=0, Wq_codes=Wc, We=We))
    _check_y(host(y), ref, ref["mag"], 256, "f32")
    y0 = S.linear_mx(xq[:0], xsc[:0], L)
    _sync()
    assert y0.shape == (0, 64)
