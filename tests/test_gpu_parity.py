"""GPU parity: the HIP kernels against the CPU oracle, element by element.

Bit-exact: activation codes and per-token scales (serq_quant_act), the int32
accumulators acc_main and acc_res (serq_linear's debug outputs). Within the
tolerance derived in gpu_helpers.py: the dequantized output Y.

Shapes cover every kernel the library dispatches to (decode16, decode32, the
four macro tiles, the generic kernel), W4A4 and W4A8, fp32 and bf16, ragged M,
N and K tails, r = 0, r not a multiple of the MFMA depth, zero rows, and the
five layer workloads at their full sizes (checked on sampled rows/columns).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import w4a4_linear_layers_amd as S
from gpu_helpers import bf16_tensor, check_y, dev, host, sample
from layouts import bf6_decode, pack_rq, pad_rq, rq_row_bytes
from oracle import serq_oracle as O
from synth import random_codes, round_to_bf16_bits, workload_layer

pytestmark = pytest.mark.gpu


def _sync():
    torch.cuda.synchronize()


# ----------------------------------------------------------------- quant_act

def _act_input(M, K, dtype, seed):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K)).astype(np.float32)
    outl = rng.choice(K, max(1, K // 100), replace=False)
    X[:, outl] *= 50
    if M > 2:
        X[1] = 0.0                      # all-zero row -> scale 0, zero codes
        X[2, :] = 0.0
        X[2, K // 3] = -3.5             # single non-zero element
    if M > 3:
        X[3] = np.round(X[3] * 2) / 2   # half-integer values: rounding ties
    sinv = (np.exp(rng.uniform(-2, 1, K))).astype(np.float32)
    if M > 3:
        sinv[:] = np.where(np.arange(K) % 2 == 0, sinv, np.float32(1.0))
    if dtype == "bf16":
        bits = round_to_bf16_bits(X).reshape(M, K)
        Xf = (bits.astype(np.uint32) << 16).view(np.float32)
        return Xf, bf16_tensor(bits), sinv
    return X, dev(X), sinv


@pytest.mark.parametrize("M,K", [(16, 256), (7, 4096), (33, 14336), (5, 28672), (9, 1000), (4, 1002), (11, 8192), (6, 2048),
                                 (3, 40000), (1, 2), (64, 8),
                                 (600, 1000), (1030, 4096), (520, 8192),     # several rows per workgroup
                                 (2, 70000), (128, 14336), (129, 14336),     # chunked rows (few rows, long K)
                                 (520, 40000), (513, 4096), (512, 4104),     # 1024, 256 or 512 lanes per row
                                 (600, 20000)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("bits", [4, 8])
def test_quant_act_bit_exact(M, K, dtype, bits):
    X, Xt, sinv = _act_input(M, K, dtype, seed=M * 7 + K)
    xq, sx = S.quant_act(Xt, dev(sinv), a_bits=bits)
    _sync()
    ref = O.quant_act(X, sinv, bits)
    assert np.array_equal(host(sx).view(np.uint32), ref["sx"].view(np.uint32))
    got = host(xq).view(np.uint8)
    assert np.array_equal(got, ref["packed"].view(np.uint8)), np.argwhere(got != ref["packed"].view(np.uint8))[:5]


def test_quant_act_empty_is_noop():
    xq = torch.full((0, 32), 7, dtype=torch.uint8, device="cuda")
    sx = torch.empty(0, device="cuda")
    S.quant_act(torch.empty((0, 64), device="cuda"), torch.ones(64, device="cuda"), a_bits=4, out=(xq, sx))
    _sync()


# ------------------------------------------------- silu(g) * u -> quant_act

def _gate_up_input(M, K, dtype, layout, seed):
    """Gate and up outputs in down's order: g of a few units spread, u with
    a few outlier channels, planted values at the exp clamp, the saturation
    of silu, zero, and a zero row; returned as host fp32 arrays (the values
    the device holds) and as device views of the requested layout."""
    rng = np.random.default_rng(seed)
    G = (rng.standard_normal((M, K)) * 3).astype(np.float32)
    U = rng.standard_normal((M, K)).astype(np.float32)
    U[:, rng.choice(K, max(1, K // 64), replace=False)] *= 30
    planted = np.array([-200.0, -88.7, -80.0, -79.9, -30.0, -0.0, 0.0, 1e-3, 20.0, 37.5, 90.0, 1e4], np.float32)
    G[0, :min(K, planted.size)] = planted[:K]
    if M > 1:
        U[1] = 0.0                              # h = 0 row -> scale 0, zero codes
    if M > 2:
        G[2] = -60.0                            # h tiny (silu(-60) ~ -5e-25), codes still full range
    if dtype == "bf16":
        gb = round_to_bf16_bits(G).reshape(M, K)
        ub = round_to_bf16_bits(U).reshape(M, K)
        G = (gb.astype(np.uint32) << 16).view(np.float32)
        U = (ub.astype(np.uint32) << 16).view(np.float32)
        pack = lambda a: bf16_tensor(a)         # noqa: E731
        raw_g, raw_u = gb, ub
    else:
        pack = dev
        raw_g, raw_u = G, U
    if layout == "split":
        return G, U, pack(raw_g), pack(raw_u)
    pad = 0 if layout == "cat" else 24
    Y = np.zeros((M, 2 * K + pad), raw_g.dtype)
    Y[:, :K] = raw_g
    Y[:, K + pad:] = raw_u
    Yt = pack(Y)
    return G, U, Yt[:, :K], Yt[:, K + pad:]


@pytest.mark.parametrize("M,K,layout", [(16, 14336, "cat"), (5, 28672, "cat"), (33, 4096, "split"),
                                        (3, 1000, "split"), (4, 1002, "cat"), (2, 40000, "split"),
                                        (9, 2048, "padded"), (1, 2, "split"), (600, 1000, "padded"),
                                        (1030, 4096, "cat"), (2, 70000, "split"), (128, 14336, "padded"),
                                        (129, 8200, "padded"), (7, 4104, "cat"), (513, 36000, "split"),
                                        (100, 28672, "cat"), (65, 14336, "split")])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("bits", [4, 8])
def test_silu_mul_quant_act_bit_exact(M, K, layout, dtype, bits):
    G, U, g, u = _gate_up_input(M, K, dtype, layout, seed=M * 13 + K)
    rng = np.random.default_rng(K)
    sinv = np.exp(rng.uniform(-2, 1, K)).astype(np.float32)
    xq, sx = S.silu_mul_quant_act(g, u, dev(sinv), a_bits=bits)
    _sync()
    ref = O.silu_mul_quant_act(G, U, sinv, bits)
    assert np.array_equal(host(sx).view(np.uint32), ref["sx"].view(np.uint32))
    got = host(xq).view(np.uint8)
    assert np.array_equal(got, ref["packed"].view(np.uint8)), np.argwhere(got != ref["packed"].view(np.uint8))[:5]


@pytest.mark.slow
@pytest.mark.parametrize("M,K", [(4096, 14336), (16, 28672)])
def test_silu_mul_quant_act_full_size(M, K):
    """The benchmark's launch configuration (a bf16 gate/up output M x 2K read
    in place), codes and scales of sampled rows (always the first and last;
    rows are independent) against the oracle."""
    G, U, g, u = _gate_up_input(M, K, "bf16", "cat", seed=K + M)
    sinv = np.exp(np.random.default_rng(5).uniform(-2, 1, K)).astype(np.float32)
    xq, sx = S.silu_mul_quant_act(g, u, dev(sinv), a_bits=4)
    _sync()
    rows = sample(M, 48, 7)
    ref = O.silu_mul_quant_act(G[rows], U[rows], sinv, 4)
    assert np.array_equal(host(sx)[rows].view(np.uint32), ref["sx"].view(np.uint32))
    assert np.array_equal(host(xq)[rows].view(np.uint8), ref["packed"].view(np.uint8))


def test_silu_mul_quant_act_empty_and_bad_arguments():
    sinv = torch.ones(64, device="cuda")
    xq = torch.full((0, 32), 7, dtype=torch.uint8, device="cuda")
    sx = torch.empty(0, device="cuda")
    z = torch.empty((0, 64), device="cuda")
    S.silu_mul_quant_act(z, z, sinv, a_bits=4, out=(xq, sx))
    g = torch.zeros((4, 64), device="cuda")
    vp = lambda t: t.data_ptr()                 # noqa: E731
    xq = torch.empty((4, 32), dtype=torch.uint8, device="cuda")
    sx = torch.empty(4, device="cuda")
    f = S.lib.serq_silu_mul_quant_act
    st = torch.cuda.current_stream().cuda_stream
    assert f(vp(g), vp(g), 32, S._lib.SERQ_F32, 4, 64, vp(sinv), 4, vp(xq), vp(sx), st) == S._lib.SERQ_EINVAL   # ld < K
    assert f(vp(g), vp(g), 64, S._lib.SERQ_F32, 4, 63, vp(sinv), 4, vp(xq), vp(sx), st) == S._lib.SERQ_EINVAL   # odd K
    assert f(vp(g), vp(g), 64, S._lib.SERQ_F32, 4, 64, vp(sinv), 5, vp(xq), vp(sx), st) == S._lib.SERQ_EINVAL   # a_bits
    assert f(vp(g) + 2, vp(g), 64, S._lib.SERQ_F32, 4, 62, vp(sinv), 4, vp(xq), vp(sx), st) == S._lib.SERQ_EALIGN
    _sync()


def test_binding_rejects_wrong_buffer_sizes():
    """The binding checks caller-supplied buffers against the sizes the
    kernels write or read (the C ABI cannot), before anything is launched."""
    x = torch.zeros((4, 64), device="cuda")
    sinv = torch.ones(64, device="cuda")
    with pytest.raises(ValueError):
        S.quant_act(x, sinv, out=(torch.empty((4, 16), dtype=torch.uint8, device="cuda"),
                                  torch.empty(4, device="cuda")))
    with pytest.raises(ValueError):
        S.quant_act(x, sinv, out=(torch.empty((4, 32), dtype=torch.uint8, device="cuda"),
                                  torch.empty(3, device="cuda")))
    with pytest.raises(ValueError):
        S.quant_act(x, torch.ones(32, device="cuda"))
    with pytest.raises(ValueError):
        S.silu_mul_quant_act(x, x, sinv, a_bits=8, out=(torch.empty((4, 32), dtype=torch.int8, device="cuda"),
                                                        torch.empty(4, device="cuda")))
    li = workload_layer("tiny", "tiny")
    D = S.calibrate(li.W, li.act_absmax, r=8).to("cuda")
    xq, sx = S.quant_act(torch.zeros((4, 256), device="cuda"), D)
    with pytest.raises(ValueError):
        S.linear(xq[:, :64], sx, D)
    with pytest.raises(ValueError):
        S.linear(xq, sx, D, out=torch.empty((4, 255), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        S.linear(xq, sx, D, out_dtype=torch.float32, out=torch.empty((4, 256), dtype=torch.bfloat16, device="cuda"))
    _sync()


# ------------------------------------------------------- linear on raw codes

def _codes_case(M, K, N, r, bits, seed, zero_scales=True):
    rng = np.random.default_rng(seed)
    Xc = random_codes(rng, (M, K), bits)
    Wc = random_codes(rng, (K, N), 4)
    Rc = random_codes(rng, (r, N), 4)
    sx = rng.uniform(0.01, 2.0, M).astype(np.float32)
    sw = rng.uniform(0.001, 0.1, N).astype(np.float32)
    sr = rng.uniform(0.0001, 0.01, N).astype(np.float32) if r else np.zeros(N, np.float32)
    if zero_scales and M > 1:
        sx[M // 2] = 0.0
    if zero_scales and N > 1:
        sw[N // 3] = 0.0
    Xq = O.pack_int4(Xc) if bits == 4 else Xc.view(np.uint8)
    layer = S.DeviceLayer(K=K, N=N, r=r, perm=None, s_hat_inv=None, Wq=dev(O.pack_int4(Wc.T)), sw=dev(sw),
                          Rq=dev(pack_rq(Rc)), sr=dev(sr))
    return Xc, Wc, Rc, sx, sw, sr, Xq, layer


def _run_codes(M, K, N, r, bits, out, seed, col_sample=None):
    Xc, Wc, Rc, sx, sw, sr, Xq, layer = _codes_case(M, K, N, r, bits, seed)
    odt = torch.float32 if out == "f32" else torch.bfloat16
    y, am, ar = S.linear(dev(Xq), dev(sx), layer, a_bits=bits, out_dtype=odt, debug=True)
    # without the debug outputs some kernels take other store paths: same Y
    y_plain = S.linear(dev(Xq), dev(sx), layer, a_bits=bits, out_dtype=odt)
    _sync()
    assert torch.equal(y_plain.view(torch.int16 if out == "bf16" else torch.int32),
                       y.view(torch.int16 if out == "bf16" else torch.int32))
    cols = np.arange(N) if col_sample is None else sample(N, col_sample, seed)
    am_ref, ar_ref = O.linear_int(Xc, Wc[:, cols], Rc[:, cols], r)
    am_g, ar_g = host(am)[:, cols], host(ar)[:, cols]
    assert np.array_equal(am_g, am_ref), np.argwhere(am_g != am_ref)[:5]
    assert np.array_equal(ar_g, ar_ref), np.argwhere(ar_g != ar_ref)[:5]
    check_y(host(y)[:, cols], am_ref, ar_ref, sx, sw[cols], sr[cols], out)


LINEAR_CASES = [
    # M, K, N, r, expected kernel
    (1, 4096, 256, 64, "gemv"),
    (2, 1056, 100, 40, "gemv"),           # K % 2048 != 0: partial 1 KB slice; N % 16 != 0
    (3, 96, 40, 96, "gemv"),              # K < one slice, r = K
    (3, 14336, 4096, 128, "gemv"),
    (4, 14336, 4096, 128, "decode16"),
    (1, 2080, 1000, 0, "gemv"),           # r = 0
    (5, 1024, 100, 40, "decode16"),       # N % 16 and N % 4 ragged, r % 64 != 0
    (16, 2080, 64, 0, "decode16"),        # K % 128 != 0, r = 0
    (16, 512, 48, 256, "decode16"),
    (17, 1024, 50, 24, "decode32"),
    (32, 512, 64, 256, "decode32"),
    (16, 1056, 4112, 72, "decode16"),     # K % 256 == 32: the last chunk holds one 16-byte piece per row
    (24, 2080, 8200, 0, "decode32"),      # four waves per group, r = 0
    (8, 32, 64, 8, "decode16"),           # one chunk and the residual: most waves have no item
    (12, 28672, 48, 256, "decode16"),     # long rows: several rounds of loads per wave
    (32, 28672, 40, 32, "decode32"),      # long rows, two token blocks, r <= 32 (16-byte Q(R) rows)
    (20, 4128, 80, 16, "decode32"),
    (40, 1056, 130, 72, "tile32x64k4"),
    (64, 96, 256, 96, "tile32x64k4"),       # K shorter than one k-tile, r = K
    (100, 512, 300, 64, "tile32x64k4"),
    (129, 800, 258, 8, "tile32x64k4"),
    (128, 4096, 4096, 64, "tile32x64k4"),       # deep pipeline, 32-token tiles
    (256, 4096, 4096, 64, "tile64x64k2"),     # two k-groups of two 32 x 64 waves, one workgroup per CU
    (256, 8192, 4096, 64, "tile64x64k4"),     # four k-groups of two 32 x 64 waves
    (200, 8224, 2600, 72, "tile64x64k4"),     # ragged M, N and K
    (200, 1056, 2600, 72, "tile64x64k2"),     # ragged M and N, a ragged last stage
    (150, 1184, 3001, 256, "tile64x64k2"),    # N % 4 != 0, two residual k-tiles, an odd stage count
    (256, 1024, 4096, 0, "tile64x64k2"),      # r = 0, eight k-tiles
    (300, 544, 4000, 40, "tile64x64"),        # ragged M, N and K
    (60, 1056, 32800, 72, "tile64x128"),      # ragged M and N
    (100, 288, 16400, 128, "tile64x128"),
    (100, 288, 24600, 128, "tile128x128k2"),  # two k-groups of 128 x 128, a ragged stage
    (130, 4160, 12400, 256, "tile128x128k2"), # an odd number of k-tiles, two residual k-tiles
    (200, 256, 32768, 64, "tile128x128"),     # many workgroups
    (300, 288, 32768, 128, "tile256x256"),    # K not a multiple of the k-tile, ragged M
    (520, 1056, 16400, 72, "tile256x256"),    # ragged M and N, r % 32 != 0
    (2048, 1056, 28672, 72, "tile128x128"),   # seven full rounds of 128 x 128 tiles
    # W4A4 256 x 256 tiles (W4A8 takes 128 x 128 tiles on these)
    (512, 384, 32768, 64, "tile256x256"),     # 256 tiles, fewer k-tiles than stages
    (500, 992, 32700, 72, "tile256x256"),     # ragged M, N and K
    (500, 992, 32702, 72, "tile256x256"),     # N % 4 != 0: element stores
    (480, 4160, 65536, 256, "tile256x256"),   # two residual k-tiles, ragged M
    (1024, 256, 16384, 0, "tile256x256"),     # r = 0
    # more 256 x 256 tiles than CUs (several rounds of workgroups)
    (760, 1024, 65536, 128, "tile256x256"),   # 768 tiles, ragged M
    (500, 2048, 65536, 0, "tile256x256"),     # 512 tiles, r = 0
    (600, 1536, 40960, 72, "tile256x256"),    # 480 tiles, a zero-filled residual k-tile
    (7, 100, 30, 6, "generic"),           # K % 32 != 0, r % 8 != 0
    (3, 384, 10, 320, "generic"),         # r > 256
]


@pytest.mark.parametrize("M,K,N,r,kern", LINEAR_CASES, ids=[c[4] + f"-{c[0]}x{c[1]}x{c[2]}r{c[3]}" for c in LINEAR_CASES])
@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_linear_codes_bit_exact(M, K, N, r, kern, bits, out):
    if kern == "gemv" and bits == 8:
        kern = "decode16"                 # the int4 dot-product kernel is W4A4 only
    if kern == "tile256x256" and bits == 8:
        kern = "tile128x128"
    if kern == "tile64x64k2" and bits == 8:
        kern = "tile64x64"
    assert S.kernel_name(M, K, N, r, bits).removesuffix("_ksplit") == kern
    _run_codes(M, K, N, r, bits, out, seed=M + K + N + r + bits, col_sample=512 if N > 2048 else None)


# W4A4 shapes whose tile choice differs from W4A8's: 64 x 64 tiles with two
# k-groups where they make one round of two per CU (W4A8: 64 x 128 tiles),
# and the two-k-group 128 x 128 tile where exactly one such tile falls on
# each CU and K is long (W4A8: one k-group).
W4A4_ROUTE_CASES = [
    (512, 1056, 4096, 72, "tile64x64k2"),     # 512 tiles of 64 x 64, eight k-tiles and a ragged stage
    (256, 1056, 8192, 0, "tile64x64k2"),      # r = 0
    (500, 1184, 4000, 256, "tile64x64k2"),    # ragged M and N, two residual k-tiles
    (128, 8192, 32768, 64, "tile128x128k2"),  # 256 tiles of 128 x 128, K = 8192
    (200, 8224, 16300, 72, "tile128x128k2"),  # ragged M, N and K
]


@pytest.mark.parametrize("M,K,N,r,kern", W4A4_ROUTE_CASES,
                         ids=[c[4] + f"-{c[0]}x{c[1]}x{c[2]}r{c[3]}" for c in W4A4_ROUTE_CASES])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_linear_w4a4_routes_bit_exact(M, K, N, r, kern, out):
    assert S.kernel_name(M, K, N, r, 4) == kern
    _run_codes(M, K, N, r, 4, out, seed=M + K + N + r, col_sample=512)


def test_linear_extreme_codes():
    """All codes at the int4/int8 extremes: the largest accumulators."""
    for bits in (4, 8):
        M, K, N, r = 48, 4096, 64, 256
        lo = -8 if bits == 4 else -128
        Xc = np.full((M, K), lo, np.int8)
        Wc = np.full((K, N), -8, np.int8)
        Rc = np.full((r, N), -8, np.int8)
        Xq = O.pack_int4(Xc) if bits == 4 else Xc.view(np.uint8)
        sx = np.ones(M, np.float32)
        sw = np.full(N, 2.0 ** -10, np.float32)
        sr = np.full(N, 2.0 ** -12, np.float32)
        layer = S.DeviceLayer(K=K, N=N, r=r, perm=None, s_hat_inv=None, Wq=dev(O.pack_int4(Wc.T)), sw=dev(sw),
                              Rq=dev(pack_rq(Rc)), sr=dev(sr))
        y, am, ar = S.linear(dev(Xq), dev(sx), layer, a_bits=bits, out_dtype=torch.float32, debug=True)
        _sync()
        am_ref, ar_ref = O.linear_int(Xc, Wc, Rc, r)
        assert np.array_equal(host(am), am_ref) and np.array_equal(host(ar), ar_ref)
        check_y(host(y), am_ref, ar_ref, sx, sw, sr, "f32")


@pytest.mark.parametrize("M,K,N,kern", [(40, 131040, 64, "tile32x64k4"), (20, 131040, 48, "decode32_ksplit"),
                                        (4, 131072, 40, "generic"), (1, 131072, 40, "gemv")])
def test_linear_longest_rows_extreme_codes(M, K, N, kern):
    """The longest rows at the int4 extremes: just below 2^17, where the
    widened sums of the MFMA kernels (256 x the products) reach 2^31 - 2^15,
    and from 2^17 on (generic kernel, int4 dot products). The expected
    accumulators are the closed forms 64 (K - 1) + x0 w0 over all K and
    64 (r - 1) + x0 r0 over the r salient columns, with the first code of
    every row and column varied over [-8, 7]."""
    r = 64
    assert S.kernel_name(M, K, N, r, 4) == kern
    x0 = (np.arange(M) % 16 - 8).astype(np.int8)
    w0 = ((np.arange(N) * 5) % 16 - 8).astype(np.int8)
    r0 = ((np.arange(N) * 3 + 1) % 16 - 8).astype(np.int8)
    Xc = np.full((M, K), -8, np.int8)
    Xc[:, 0] = x0
    Wc = np.full((K, N), -8, np.int8)
    Wc[0] = w0
    Rc = np.full((r, N), -8, np.int8)
    Rc[0] = r0
    sx = np.ones(M, np.float32)
    sw = np.full(N, 2.0 ** -16, np.float32)
    sr = np.full(N, 2.0 ** -12, np.float32)
    layer = S.DeviceLayer(K=K, N=N, r=r, perm=None, s_hat_inv=None, Wq=dev(O.pack_int4(Wc.T)), sw=dev(sw),
                          Rq=dev(pack_rq(Rc)), sr=dev(sr))
    y, am, ar = S.linear(dev(O.pack_int4(Xc)), dev(sx), layer, a_bits=4, out_dtype=torch.float32, debug=True)
    _sync()
    am_ref = 64 * (K - 1) + x0.astype(np.int64)[:, None] * w0.astype(np.int64)[None, :]
    ar_ref = 64 * (r - 1) + x0.astype(np.int64)[:, None] * r0.astype(np.int64)[None, :]
    assert np.array_equal(host(am), am_ref) and np.array_equal(host(ar), ar_ref)
    check_y(host(y), am_ref, ar_ref, sx, sw, sr, "f32")


def test_linear_on_side_stream_and_empty():
    Xc, Wc, Rc, sx, sw, sr, Xq, layer = _codes_case(64, 512, 96, 64, 4, seed=5)
    s = torch.cuda.Stream()
    xq_d, sx_d = dev(Xq), dev(sx)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        y, am, ar = S.linear(xq_d, sx_d, layer, a_bits=4, out_dtype=torch.float32, debug=True)
    s.synchronize()
    am_ref, ar_ref = O.linear_int(Xc, Wc, Rc, 64)
    assert np.array_equal(host(am), am_ref)
    y0 = S.linear(xq_d[:0], sx_d[:0], layer, a_bits=4)
    _sync()
    assert y0.shape == (0, 96)


# ------------------------------------------------ the layer workloads, end to end

def _end_to_end(li, r, bits, out, Ms, *, row_sample=48, col_sample=192, seed=0, W=None, W_in=None):
    """Library calibration + GPU quant_act + GPU linear vs the oracle.

    Bit-exact on full tensors: perm, s_hat_inv, Q(W^), Q(R) and their scales
    for every output column (oracle calibrate on the whole layer), and the
    activation codes and scales of every token row. The accumulators and Y
    on sampled rows x columns (always the first and last of each). ``W`` /
    ``W_in`` replace the layer's weight (fp32 values / the library's input,
    bf16 bit patterns for bf16 workloads), e.g. gate and up side by side."""
    W = li.W if W is None else W
    if W_in is None:
        W_in = li.W_bits if li.dtype == "bf16" else li.W
    N = W.shape[1]
    print(f"calibrate {W.shape[0]} x {N}, r = {r}", flush=True)
    L = S.calibrate(W_in, li.act_absmax, r=r)
    R = O.calibrate(W, li.act_absmax, r=r)
    assert np.array_equal(L.perm, R["perm"])
    assert np.array_equal(L.s_hat_inv.view(np.uint32), R["s_hat_inv"].view(np.uint32))
    assert np.array_equal(L.Wq, R["Wq"])
    assert np.array_equal(L.sw.view(np.uint32), R["sw"].view(np.uint32))
    assert np.array_equal(L.Rq, pad_rq(R["Rq"], r))
    assert np.array_equal(L.sr.view(np.uint32), R["sr"].view(np.uint32))
    D = L.to("cuda")
    cols = sample(N, col_sample, seed + 1)
    Wc, Rc = R["Wq_codes"][:, cols], R["Rq_codes"][:, cols]
    sw, sr = R["sw"][cols], R["sr"][cols]
    del R
    odt = torch.float32 if out == "f32" else torch.bfloat16
    for M in Ms:
        print(f"M = {M}: {S.kernel_name(M, W.shape[0], N, r, bits)}", flush=True)
        if li.dtype == "bf16":
            xt = bf16_tensor(li.X_bits[:M][:, L.perm])
        else:
            xt = dev(li.X[:M][:, L.perm])
        xq, sx = S.quant_act(xt, D, a_bits=bits)
        y, am, ar = S.linear(xq, sx, D, a_bits=bits, out_dtype=odt, debug=True)
        _sync()
        q = O.quant_act(li.X[:M][:, L.perm], L.s_hat_inv, bits)
        assert np.array_equal(host(xq).view(np.uint8), q["packed"].view(np.uint8))
        assert np.array_equal(host(sx).view(np.uint32), q["sx"].view(np.uint32))
        rows = sample(M, row_sample, seed + M)
        am_ref, ar_ref = O.linear_int(q["codes"][rows], Wc, Rc, r)
        assert np.array_equal(host(am)[np.ix_(rows, cols)], am_ref)
        assert np.array_equal(host(ar)[np.ix_(rows, cols)], ar_ref)
        check_y(host(y)[np.ix_(rows, cols)], am_ref, ar_ref, q["sx"][rows], sw, sr, out)
        del xt, xq, sx, y, am, ar, q
    return L


def _gate_up_cat(li):
    """Gate and up side by side, K x 2N: the layer the two share one input
    as (calibrated together, one s and P for both)."""
    W = np.concatenate([li.W, li.meta["W_up"]], axis=1)
    W_in = np.concatenate([li.W_bits, li.meta["W_up_bits"]], axis=1)
    return W, W_in


def test_gptq_layer_end_to_end():
    """SERQ(GPTQ): a layer calibrated with GPTQ codes (library host code, bit
    for bit against the oracle's GPTQ), then GPU quant_act + serq_linear on
    it at 16 and 300 tokens: codes, scales and accumulators bit-exact, Y
    within tolerance, on every row and column. The kernels are the same;
    only the weight codes change."""
    from synth import make_layer
    li = make_layer(1024, 1536, 300, n_out=10, factor=50.0, seed=0, tag=20, dtype="bf16")
    r = 64
    X_cal_bits = round_to_bf16_bits(li.X_cal).reshape(li.X_cal.shape)
    L = S.calibrate_gptq(li.W_bits, li.act_absmax, X_cal_bits, r=r)
    R = O.calibrate_gptq(li.W, li.act_absmax, li.X_cal, r=r)
    assert np.array_equal(L.Wq, R["Wq"]) and np.array_equal(L.perm, R["perm"])
    assert np.array_equal(L.Rq, pad_rq(R["Rq"], r)) and np.array_equal(L.sw.view(np.uint32), R["sw"].view(np.uint32))
    assert not np.array_equal(L.Wq, S.calibrate(li.W_bits, li.act_absmax, r=r).Wq)
    D = L.to("cuda")
    for M in (16, 300):
        print(f"M = {M}: {S.kernel_name(M, 1024, 1536, r, 4)}", flush=True)
        xq, sx = S.quant_act(bf16_tensor(li.X_bits[:M][:, L.perm]), D, a_bits=4)
        y, am, ar = S.linear(xq, sx, D, a_bits=4, out_dtype=torch.bfloat16, debug=True)
        _sync()
        q = O.quant_act(li.X[:M][:, L.perm], L.s_hat_inv, 4)
        assert np.array_equal(host(xq).view(np.uint8), q["packed"]) and np.array_equal(host(sx), q["sx"])
        am_ref, ar_ref = O.linear_int(q["codes"], R["Wq_codes"], R["Rq_codes"], r)
        assert np.array_equal(host(am), am_ref) and np.array_equal(host(ar), ar_ref)
        check_y(host(y), am_ref, ar_ref, q["sx"], R["sw"], R["sr"], "bf16")


def test_workload_tiny_full():
    """256 -> 256, r = 8, M = 16, fp32 in and out: every output checked."""
    li = workload_layer("tiny", "tiny")
    _end_to_end(li, 8, 4, "f32", [16], row_sample=16, col_sample=256)


@pytest.mark.slow
def test_workload_q_proj():
    li = workload_layer("q_proj", "q_proj")
    _end_to_end(li, 64, 4, "bf16", [1, 16, 256, 2048])


@pytest.mark.slow
@pytest.mark.parametrize("layer", ["gate_up", "down"])
def test_workload_mlp8b(layer):
    """gate/up as the one 4096 -> 2 x 14336 layer (gate and up share their
    input, so they are calibrated together), down 14336 -> 4096."""
    li = workload_layer("mlp8b", layer)
    W, W_in = _gate_up_cat(li) if layer == "gate_up" else (None, None)
    _end_to_end(li, 128, 4, "bf16", [1, 32, 4096], W=W, W_in=W_in)


@pytest.mark.slow
@pytest.mark.parametrize("layer", ["gate_up", "down"])
def test_workload_mlp8b_w4a8(layer):
    li = workload_layer("mlp8b_w4a8", layer)
    W, W_in = _gate_up_cat(li) if layer == "gate_up" else (None, None)
    _end_to_end(li, 128, 8, "bf16", [2048], W=W, W_in=W_in)


@pytest.mark.slow
@pytest.mark.parametrize("layer", ["up70", "down70"])
def test_workload_l70b(layer):
    li = workload_layer("l70b", layer)
    _end_to_end(li, 256, 4, "bf16", [1, 8192], row_sample=32, col_sample=128)


@pytest.mark.slow
def test_mlp8b_p4_propagation():
    """The down projection's order P4 pushed into the gate/up output channels
    (serq_permute_outputs): gate/up then produce their outputs already in P4
    order, bit for bit the permuted outputs, and down consumes
    h = silu(g) * u with no gather."""
    M = 32
    gu = workload_layer("mlp8b", "gate_up", M_max=M)
    dn = workload_layer("mlp8b", "down", M_max=1, draw_x=False)
    N = gu.N
    Wcat = np.concatenate([gu.W_bits, gu.meta["W_up_bits"]], axis=1)
    Lgu = S.calibrate(Wcat, gu.act_absmax, r=128)
    Ld = S.calibrate(dn.W_bits, dn.act_absmax, r=128)
    p4 = Ld.perm

    def part(lo, hi):
        return S.SerqLayer(K=Lgu.K, N=N, r=128, perm=Lgu.perm, s_hat_inv=Lgu.s_hat_inv,
                           Wq=Lgu.Wq[lo:hi].copy(), sw=Lgu.sw[lo:hi].copy(), Rq=Lgu.Rq[lo:hi].copy(),
                           sr=Lgu.sr[lo:hi].copy())

    gate, up = part(0, N), part(N, 2 * N)
    gate_p = S.permute_outputs(part(0, N), p4)
    up_p = S.permute_outputs(part(N, 2 * N), p4)
    xq, sx = S.quant_act(bf16_tensor(gu.X_bits[:, Lgu.perm]), dev(Lgu.s_hat_inv), a_bits=4)
    outs = {}
    for name, L in (("g", gate), ("u", up), ("gp", gate_p), ("up", up_p)):
        outs[name] = S.linear(xq, sx, L.to("cuda"), a_bits=4, out_dtype=torch.bfloat16, debug=True)
    _sync()
    for a, b in (("g", "gp"), ("u", "up")):
        y0, am0, ar0 = (host(t) for t in outs[a])
        y1, am1, ar1 = (host(t) for t in outs[b])
        assert np.array_equal(am1, am0[:, p4]) and np.array_equal(ar1, ar0[:, p4])
        assert np.array_equal(y1, y0[:, p4])

    def silu_mul(g_bits, u_bits):      # glue between the layers (host, not timed)
        g = (g_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        u = (u_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        return round_to_bf16_bits((g / (1.0 + np.exp(-g)) * u).astype(np.float32)).reshape(g_bits.shape)

    h = silu_mul(host(outs["g"][0]), host(outs["u"][0]))
    h_p4 = silu_mul(host(outs["gp"][0]), host(outs["up"][0]))
    assert np.array_equal(h_p4, h[:, p4])          # arrives in P4 order, no gather needed
    D = Ld.to("cuda")
    xq_d, sx_d = S.quant_act(bf16_tensor(h_p4), D, a_bits=4)
    y, am, ar = S.linear(xq_d, sx_d, D, a_bits=4, out_dtype=torch.bfloat16, debug=True)
    _sync()
    cols = sample(dn.N, 192, 3)
    R = O.calibrate_columns(dn.W, dn.act_absmax, cols, r=128)
    hf = (h.astype(np.uint32) << 16).view(np.float32)
    q = O.quant_act(hf[:, R["perm"]], R["s_hat_inv"], 4)
    assert np.array_equal(host(xq_d).view(np.uint8), q["packed"])
    am_ref, ar_ref = O.linear_int(q["codes"], R["Wq_codes"], R["Rq_codes"], 128)
    assert np.array_equal(host(am)[:, cols], am_ref) and np.array_equal(host(ar)[:, cols], ar_ref)
    check_y(host(y)[:, cols], am_ref, ar_ref, q["sx"], R["sw"], R["sr"], "bf16")


@pytest.mark.slow
def test_mlp8b_fused_activation_chain():
    """gate and up as one layer of 2 x 14336 outputs whose channels carry
    down's order P4 (serq_permute_outputs), its bf16 output M x 28672 read
    in place by serq_silu_mul_quant_act (g = left half, u = right half,
    ld = 28672), then down: codes, scales and accumulators against the
    oracle's silu_mul_quant_act and linear."""
    M = 32
    gu = workload_layer("mlp8b", "gate_up", M_max=M)
    dn = workload_layer("mlp8b", "down", M_max=1, draw_x=False)
    N = gu.N
    Wcat = np.concatenate([gu.W_bits, gu.meta["W_up_bits"]], axis=1)
    Lgu = S.calibrate(Wcat, gu.act_absmax, r=128)
    Ld = S.calibrate(dn.W_bits, dn.act_absmax, r=128)
    p4 = Ld.perm
    Lp = S.permute_outputs(S.SerqLayer(K=Lgu.K, N=2 * N, r=128, perm=Lgu.perm, s_hat_inv=Lgu.s_hat_inv,
                                       Wq=Lgu.Wq.copy(), sw=Lgu.sw.copy(), Rq=Lgu.Rq.copy(), sr=Lgu.sr.copy()),
                           np.concatenate([p4, N + p4]))
    xq, sx = S.quant_act(bf16_tensor(gu.X_bits[:, Lgu.perm]), dev(Lgu.s_hat_inv), a_bits=4)
    y0 = S.linear(xq, sx, Lgu.to("cuda"), a_bits=4, out_dtype=torch.bfloat16)
    y = S.linear(xq, sx, Lp.to("cuda"), a_bits=4, out_dtype=torch.bfloat16)
    D = Ld.to("cuda")
    xq_d, sx_d = S.silu_mul_quant_act(y[:, :N], y[:, N:], D, a_bits=4)
    yd, am, ar = S.linear(xq_d, sx_d, D, a_bits=4, out_dtype=torch.bfloat16, debug=True)
    _sync()
    yb, y0b = host(y), host(y0)
    assert np.array_equal(yb[:, :N], y0b[:, :N][:, p4]) and np.array_equal(yb[:, N:], y0b[:, N:][:, p4])
    f32 = lambda b: (b.astype(np.uint32) << 16).view(np.float32)     # noqa: E731
    cols = sample(dn.N, 192, 5)
    R = O.calibrate_columns(dn.W, dn.act_absmax, cols, r=128)
    assert np.array_equal(R["perm"], p4)
    q = O.silu_mul_quant_act(f32(yb[:, :N]), f32(yb[:, N:]), R["s_hat_inv"], 4)
    # the same codes from the unpermuted outputs, gathered on the host
    q0 = O.silu_mul_quant_act(f32(y0b[:, :N])[:, p4], f32(y0b[:, N:])[:, p4], R["s_hat_inv"], 4)
    assert np.array_equal(q["packed"], q0["packed"]) and np.array_equal(q["sx"], q0["sx"])
    assert np.array_equal(host(xq_d).view(np.uint8), q["packed"].view(np.uint8))
    assert np.array_equal(host(sx_d).view(np.uint32), q["sx"].view(np.uint32))
    am_ref, ar_ref = O.linear_int(q["codes"], R["Wq_codes"], R["Rq_codes"], 128)
    assert np.array_equal(host(am)[:, cols], am_ref) and np.array_equal(host(ar)[:, cols], ar_ref)
    check_y(host(yd)[:, cols], am_ref, ar_ref, q["sx"], R["sw"], R["sr"], "bf16")


# ------------------------------------------------------------- the bf6 route

@pytest.mark.parametrize("M,K", [(1, 2), (5, 30), (37, 320), (130, 1000), (129, 256), (300, 4096), (64, 96)])
def test_act_bf6_layout(M, K):
    """serq_act_bf6 against the header's layout (independent reader) and
    against the host prepack of the same codes, byte for byte."""
    rng = np.random.default_rng(M * 3 + K)
    c = random_codes(rng, (M, K), 4)
    c.flat[:16] = np.arange(-8, 8)[: min(16, c.size)]
    packed = O.pack_int4(c)
    x6 = S.act_bf6(dev(packed), K)
    _sync()
    got = host(x6)
    assert got.size == S.bf6_bytes(M, K)
    assert np.array_equal(got, S._prepack(packed, M, K, K // 2))
    full, codes = bf6_decode(got, M, K)
    assert np.array_equal(codes, c)
    full[:M, :K] = 0
    assert not full.any()


def _bf6_layer(Wc, Rc, sw, sr, K, N, r):
    W6 = S._prepack(O.pack_int4(Wc.T), N, K, K // 2)
    R6 = S._prepack(pack_rq(Rc), N, r, rq_row_bytes(r)) if r else np.zeros(0, np.uint8)
    return S.Bf6Layer(K=K, N=N, r=r, W6=dev(W6), sw=dev(sw), R6=dev(R6), sr=dev(sr))


def _bf6_tile(M, N):
    """The tile rule stated with serq_linear_bf6's host code: a 256 side only
    where the 128-row padding is a multiple of 256, and only with a tile for
    every CU."""
    mp, np_ = -(-M // 128) * 128, -(-N // 128) * 128
    if mp % 256 == 0 and np_ % 256 == 0 and (mp // 256) * (np_ // 256) >= 256:
        return "bf6_tile256x256"
    return "bf6_tile128x128"


BF6_CASES = [
    # M, K, N, r
    (1, 256, 128, 64),
    (37, 320, 200, 72),        # K % 128 != 0, ragged M and N, r % 32 != 0
    (130, 1000, 260, 40),      # K % 32 != 0 (the element-wise activation path)
    (64, 96, 256, 96),         # K shorter than one k-tile, r = K
    (200, 4160, 1000, 256),    # an odd number of k-tiles, two residual k-tiles
    (256, 1056, 300, 0),       # r = 0
    (513, 2048, 640, 130),     # two residual k-tiles, the second nearly empty
    (128, 4096, 4096, 64),
    (300, 8192, 1000, 128),
    (1024, 256, 16384, 64),    # 256 x 256 tiles
    (1000, 300, 16284, 130),   # 256 x 256 tiles, ragged M, N and K, two residual k-tiles
    (2048, 1024, 8192, 0),     # 256 x 256 tiles, r = 0
    (2048, 1024, 4096, 64),    # 128 x 128 tiles, 512 of them
    (2000, 520, 4000, 200),    # 128 x 128 tiles, ragged M, N and K, two residual k-tiles
]


@pytest.mark.parametrize("M,K,N,r", BF6_CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}r{c[3]}" for c in BF6_CASES])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_linear_bf6_bit_exact(M, K, N, r, out):
    """The bf6 route: exact integer accumulators against the oracle, Y within
    the epilogue tolerance, and Y bit-identical to serq_linear's."""
    assert S.bf6_kernel_name(M, N, r) == _bf6_tile(M, N)
    Xc, Wc, Rc, sx, sw, sr, Xq, layer = _codes_case(M, K, N, r, 4, seed=M + K + N + r + 6)
    L6 = _bf6_layer(Wc, Rc, sw, sr, K, N, r)
    odt = torch.float32 if out == "f32" else torch.bfloat16
    xq_d, sx_d = dev(Xq), dev(sx)
    x6 = S.act_bf6(xq_d, K)
    y, am, ar = S.linear_bf6(x6, sx_d, L6, out_dtype=odt, debug=True)
    y_fast = S.linear_bf6(x6, sx_d, L6, out_dtype=odt)            # the epilogue without debug outputs
    y_int = S.linear(xq_d, sx_d, layer, a_bits=4, out_dtype=odt)
    _sync()
    assert np.array_equal(host(y_fast), host(y_int))
    cols = np.arange(N) if N <= 2048 else sample(N, 512, M)
    am_ref, ar_ref = O.linear_int(Xc, Wc[:, cols], Rc[:, cols], r)
    am_g, ar_g = host(am)[:, cols], host(ar)[:, cols]
    assert np.array_equal(am_g, am_ref), np.argwhere(am_g != am_ref)[:5]
    assert np.array_equal(ar_g, ar_ref), np.argwhere(ar_g != ar_ref)[:5]
    check_y(host(y)[:, cols], am_ref, ar_ref, sx, sw[cols], sr[cols], out)
    assert np.array_equal(host(y), host(y_int))


def test_linear_bf6_extreme_codes_and_empty():
    """All codes -8 over K = 4096 (+ r = 256): the largest sums, exact in fp32."""
    M, K, N, r = 48, 4096, 64, 256
    Xc = np.full((M, K), -8, np.int8)
    Wc = np.full((K, N), -8, np.int8)
    Rc = np.full((r, N), -8, np.int8)
    sx = np.ones(M, np.float32)
    sw = np.full(N, 2.0 ** -10, np.float32)
    sr = np.full(N, 2.0 ** -12, np.float32)
    L6 = _bf6_layer(Wc, Rc, sw, sr, K, N, r)
    x6 = S.act_bf6(dev(O.pack_int4(Xc)), K)
    y, am, ar = S.linear_bf6(x6, dev(sx), L6, out_dtype=torch.float32, debug=True)
    _sync()
    am_ref, ar_ref = O.linear_int(Xc, Wc, Rc, r)
    assert np.array_equal(host(am), am_ref) and np.array_equal(host(ar), ar_ref)
    check_y(host(y), am_ref, ar_ref, sx, sw, sr, "f32")
    assert np.array_equal(host(S.linear_bf6(x6, dev(sx), L6, out_dtype=torch.float32)), host(y))
    e6 = S.act_bf6(torch.empty((0, K // 2), dtype=torch.uint8, device="cuda"), K)
    y0 = S.linear_bf6(e6, torch.empty(0, dtype=torch.float32, device="cuda"), L6)
    _sync()
    assert e6.numel() == 0 and y0.shape == (0, N)


@pytest.mark.parametrize("K", [28672, 1 << 18])
def test_linear_bf6_sums_to_2_24(K):
    """fp32 accumulation on the FP6 instruction is exact up to 2^24: every
    code -8 except the first of each row and column (varied over [-8, 7]),
    so the partial sums are odd or even integers climbing to
    64 (K - 1) + x0 w0 <= 2^24 (K = 2^18: 24 significant bits in the last
    steps). Expected values in closed form; K = 28672 is the 70B down
    layer's length."""
    M, N, r = 40, 96, 256
    x0 = (np.arange(M) % 16 - 8).astype(np.int8)
    w0 = ((np.arange(N) * 5) % 16 - 8).astype(np.int8)
    r0 = ((np.arange(N) * 3 + 1) % 16 - 8).astype(np.int8)
    Xc = np.full((M, K), -8, np.int8)
    Xc[:, 0] = x0
    Wc = np.full((K, N), -8, np.int8)
    Wc[0] = w0
    Rc = np.full((r, N), -8, np.int8)
    Rc[0] = r0
    sx = np.ones(M, np.float32)
    sw = np.full(N, 2.0 ** -20, np.float32)
    sr = np.full(N, 2.0 ** -12, np.float32)
    L6 = _bf6_layer(Wc, Rc, sw, sr, K, N, r)
    x6 = S.act_bf6(dev(O.pack_int4(Xc)), K)
    y, am, ar = S.linear_bf6(x6, dev(sx), L6, out_dtype=torch.float32, debug=True)
    _sync()
    am_ref = 64 * (K - 1) + x0.astype(np.int64)[:, None] * w0.astype(np.int64)[None, :]
    ar_ref = 64 * (r - 1) + x0.astype(np.int64)[:, None] * r0.astype(np.int64)[None, :]
    assert am_ref.max() <= 2 ** 24
    assert np.array_equal(host(am), am_ref), np.argwhere(host(am) != am_ref)[:5]
    assert np.array_equal(host(ar), ar_ref)
    check_y(host(y), am_ref, ar_ref, sx, sw, sr, "f32")


@pytest.mark.slow
def test_workload_q_proj_bf6():
    """q_proj at 2048 tokens (the benchmark's launch): calibrated layer, GPU
    quant_act, then the bf6 route against serq_linear bit for bit and the
    oracle's accumulators on sampled columns."""
    li = workload_layer("q_proj", "q_proj")
    L = S.calibrate(li.W_bits, li.act_absmax, r=64)
    D = L.to("cuda")
    B = S.prepack_bf6(L).to("cuda")
    M = 2048
    xq, sx = S.quant_act(bf16_tensor(li.X_bits[:M][:, L.perm]), D, a_bits=4)
    x6 = S.act_bf6(xq, L.K)
    y6, am, ar = S.linear_bf6(x6, sx, B, debug=True)
    y6f = S.linear_bf6(x6, sx, B)
    y = S.linear(xq, sx, D, a_bits=4)
    _sync()
    assert np.array_equal(host(y6), host(y)) and np.array_equal(host(y6f), host(y))
    cols = sample(L.N, 128, 3)
    Xc = O.unpack_int4(host(xq))
    Wc = O.unpack_int4(L.Wq[cols]).T
    Rc = O.unpack_int4(np.ascontiguousarray(L.Rq[cols, : L.r // 2])).T
    am_ref, ar_ref = O.linear_int(Xc, Wc, Rc, L.r)
    assert np.array_equal(host(am)[:, cols], am_ref) and np.array_equal(host(ar)[:, cols], ar_ref)
