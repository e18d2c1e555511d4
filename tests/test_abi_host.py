"""Host-side checks of the C ABI (no GPU needed).

* the library loads and exports every function include/serq.h declares;
* argument errors are reported before anything is launched;
* the offline calls (serq_calibrate, serq_permute_outputs) match the oracle
  bit for bit on packed tensors, scales and the permutation.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import w4a4_linear_layers_amd as S
from w4a4_linear_layers_amd import _lib
from layouts import bf6_decode, pad_rq, rq_row_bytes
from oracle import serq_oracle as O
from synth import bf16_bits_to_f32, make_layer, round_to_bf16_bits, workload_layer

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "serq.h")


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(serq_[a-z0-9_]+)\s*\(", txt)))


def test_header_declarations_are_exported():
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS), names
    for n in names:
        assert hasattr(_lib.lib, n), n
        assert ctypes.cast(getattr(_lib.lib, n), ctypes.c_void_p).value


def test_strerror_and_version():
    assert _lib.lib.serq_abi_version() == 300
    for code in (0, -1, -2, -3, -4, 7):
        assert _lib.lib.serq_strerror(code)


def test_rq_row_bytes():
    """Q(R) rows are padded to 32 codes (16 bytes); calibration writes zero
    codes into the padding."""
    assert _lib.lib.serq_rq_row_bytes(-2) == -1
    for r in range(0, 300, 2):
        assert _lib.lib.serq_rq_row_bytes(r) == rq_row_bytes(r) == S.rq_row_bytes(r)
    li = make_layer(96, 40, 1, n_out=2, factor=20.0, seed=3, tag=7)
    L = S.calibrate(li.W, li.act_absmax, r=10)
    assert L.Rq.shape == (40, 16) and not L.Rq[:, 5:].any() and L.Rq[:, :5].any()


# ---------------------------------------------------------------- argument errors
# Only rejected calls (and M == 0 no-ops) are made here: the fake addresses
# below are never dereferenced because validation happens first.

A16 = 0x10000          # an aligned fake device address
A_BAD = 0x10004        # a misaligned one


def quant(X=A16, dt=_lib.SERQ_BF16, M=4, K=64, sinv=A16, bits=4, xq=A16, sx=A16):
    return _lib.lib.serq_quant_act(X, dt, M, K, sinv, bits, xq, sx, None)


def act(G=A16, U=A16 + 128, ld=64, dt=_lib.SERQ_BF16, M=4, K=64, sinv=A16, bits=4, xq=A16, sx=A16):
    return _lib.lib.serq_silu_mul_quant_act(G, U, ld, dt, M, K, sinv, bits, xq, sx, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=5), _lib.SERQ_EINVAL), (dict(bits=2), _lib.SERQ_EINVAL), (dict(M=-1), _lib.SERQ_EINVAL),
    (dict(K=0), _lib.SERQ_EINVAL), (dict(K=63, ld=64), _lib.SERQ_EINVAL), (dict(ld=62), _lib.SERQ_EINVAL),
    (dict(G=None), _lib.SERQ_EINVAL), (dict(U=None), _lib.SERQ_EINVAL), (dict(sinv=None), _lib.SERQ_EINVAL),
    (dict(xq=None), _lib.SERQ_EINVAL), (dict(sx=None), _lib.SERQ_EINVAL),
    (dict(G=A16 + 1), _lib.SERQ_EALIGN), (dict(U=A16 + 3), _lib.SERQ_EALIGN),
    (dict(dt=_lib.SERQ_F32, U=A16 + 2), _lib.SERQ_EALIGN), (dict(sinv=A_BAD), _lib.SERQ_EALIGN),
    (dict(xq=A_BAD), _lib.SERQ_EALIGN), (dict(sx=A_BAD), _lib.SERQ_EALIGN),
    (dict(M=0), _lib.SERQ_OK), (dict(M=0, G=None, U=None, xq=None, sx=None), _lib.SERQ_OK),
    (dict(M=0, sinv=None), _lib.SERQ_EINVAL),
])
def test_silu_mul_quant_act_argument_errors(kw, code):
    """G and U need only element alignment (U = G + K for a gate/up output);
    Xq, sx and s_hat_inv 16 bytes; ld >= K."""
    assert act(**kw) == code


def lin(xq=A16, sx=A16, bits=4, wq=A16, sw=A16, rq=A16, sr=A16, M=4, K=64, N=32, r=8, y=A16,
        dt=_lib.SERQ_BF16, dm=None, dr=None):
    return _lib.lib.serq_linear(xq, sx, bits, wq, sw, rq, sr, M, K, N, r, y, dt, dm, dr, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=5), _lib.SERQ_EINVAL), (dict(bits=2), _lib.SERQ_EINVAL), (dict(M=-1), _lib.SERQ_EINVAL),
    (dict(K=0), _lib.SERQ_EINVAL), (dict(K=63), _lib.SERQ_EINVAL), (dict(X=None), _lib.SERQ_EINVAL),
    (dict(sinv=None), _lib.SERQ_EINVAL), (dict(xq=None), _lib.SERQ_EINVAL), (dict(sx=None), _lib.SERQ_EINVAL),
    (dict(X=A_BAD), _lib.SERQ_EALIGN), (dict(xq=A_BAD), _lib.SERQ_EALIGN), (dict(sx=A_BAD), _lib.SERQ_EALIGN),
    (dict(M=0), _lib.SERQ_OK), (dict(M=0, X=None, xq=None, sx=None), _lib.SERQ_OK),
    (dict(M=0, sinv=None), _lib.SERQ_EINVAL),
])
def test_quant_act_argument_errors(kw, code):
    assert quant(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(bits=3), _lib.SERQ_EINVAL), (dict(dt=9), _lib.SERQ_EINVAL), (dict(M=-2), _lib.SERQ_EINVAL),
    (dict(K=0), _lib.SERQ_EINVAL), (dict(K=33), _lib.SERQ_EINVAL), (dict(N=0), _lib.SERQ_EINVAL),
    (dict(r=-2), _lib.SERQ_EINVAL), (dict(r=7), _lib.SERQ_EINVAL), (dict(r=66), _lib.SERQ_EINVAL),
    (dict(xq=None), _lib.SERQ_EINVAL), (dict(wq=None), _lib.SERQ_EINVAL), (dict(y=None), _lib.SERQ_EINVAL),
    (dict(rq=None), _lib.SERQ_EINVAL), (dict(sr=None), _lib.SERQ_EINVAL),
    (dict(dm=A16), _lib.SERQ_EINVAL), (dict(dr=A16), _lib.SERQ_EINVAL),
    (dict(wq=A_BAD), _lib.SERQ_EALIGN), (dict(y=A_BAD), _lib.SERQ_EALIGN), (dict(sw=A_BAD), _lib.SERQ_EALIGN),
    (dict(rq=A_BAD), _lib.SERQ_EALIGN), (dict(dm=A16, dr=A_BAD), _lib.SERQ_EALIGN),
    (dict(M=0), _lib.SERQ_OK), (dict(M=0, r=0, rq=None, sr=None), _lib.SERQ_OK),
    (dict(M=0, xq=None, sx=None, y=None), _lib.SERQ_OK), (dict(M=0, wq=None), _lib.SERQ_EINVAL),
])
def test_linear_argument_errors(kw, code):
    assert lin(**kw) == code


def lin6(x6=A16, sx=A16, w6=A16, sw=A16, r6=A16, sr=A16, M=4, K=256, N=32, r=8, y=A16, dt=_lib.SERQ_BF16,
         dm=None, dr=None):
    return _lib.lib.serq_linear_bf6(x6, sx, w6, sw, r6, sr, M, K, N, r, y, dt, dm, dr, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=4), _lib.SERQ_EINVAL), (dict(M=-1), _lib.SERQ_EINVAL), (dict(K=0), _lib.SERQ_EINVAL),
    (dict(K=255), _lib.SERQ_EINVAL), (dict(K=(1 << 18) + 2), _lib.SERQ_EINVAL), (dict(N=0), _lib.SERQ_EINVAL),
    (dict(r=258, K=512), _lib.SERQ_EINVAL), (dict(r=5), _lib.SERQ_EINVAL), (dict(r=260, K=256), _lib.SERQ_EINVAL),
    (dict(x6=None), _lib.SERQ_EINVAL), (dict(w6=None), _lib.SERQ_EINVAL), (dict(r6=None), _lib.SERQ_EINVAL),
    (dict(sx=None), _lib.SERQ_EINVAL), (dict(y=None), _lib.SERQ_EINVAL), (dict(dm=A16), _lib.SERQ_EINVAL),
    (dict(x6=A_BAD), _lib.SERQ_EALIGN), (dict(w6=A_BAD), _lib.SERQ_EALIGN), (dict(r6=A_BAD), _lib.SERQ_EALIGN),
    (dict(y=A_BAD), _lib.SERQ_EALIGN), (dict(dm=A16, dr=A_BAD), _lib.SERQ_EALIGN),
    (dict(M=0), _lib.SERQ_OK), (dict(M=0, x6=None, sx=None, y=None), _lib.SERQ_OK),
    (dict(M=0, r=0, r6=None, sr=None), _lib.SERQ_OK), (dict(M=0, w6=None), _lib.SERQ_EINVAL),
])
def test_linear_bf6_argument_errors(kw, code):
    """The bf6 linear takes W4A4 sizes with K <= 2^18 (exact fp32 sums) and
    r <= 256."""
    assert lin6(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), _lib.SERQ_EINVAL), (dict(K=0), _lib.SERQ_EINVAL), (dict(K=7), _lib.SERQ_EINVAL),
    (dict(K=(1 << 18) + 2), _lib.SERQ_EINVAL), (dict(xq=None), _lib.SERQ_EINVAL), (dict(x6=None), _lib.SERQ_EINVAL),
    (dict(xq=A_BAD), _lib.SERQ_EALIGN), (dict(x6=A_BAD), _lib.SERQ_EALIGN),
    (dict(M=0), _lib.SERQ_OK), (dict(M=0, xq=None, x6=None), _lib.SERQ_OK),
])
def test_act_bf6_argument_errors(kw, code):
    args = dict(xq=A16, M=4, K=256, x6=A16)
    args.update(kw)
    assert _lib.lib.serq_act_bf6(args["xq"], args["M"], args["K"], args["x6"], None) == code


def test_bf6_bytes_and_prepack_errors():
    assert _lib.lib.serq_bf6_bytes(-1, 4) == -1 and _lib.lib.serq_bf6_bytes(4, -2) == -1
    for rows, k in [(1, 2), (128, 128), (129, 128), (128, 130), (4096, 4096), (28672, 8192)]:
        assert S.bf6_bytes(rows, k) == -(-rows // 128) * -(-k // 128) * 128 * 96
    buf = np.zeros((4, 8), np.uint8)
    out = np.zeros(S.bf6_bytes(4, 16), np.uint8)
    pre = _lib.lib.serq_prepack_bf6
    assert pre(buf.ctypes.data, 4, 16, 8, out.ctypes.data) == _lib.SERQ_OK
    assert pre(None, 4, 16, 8, out.ctypes.data) == _lib.SERQ_EINVAL
    assert pre(buf.ctypes.data, 4, 16, 8, None) == _lib.SERQ_EINVAL
    assert pre(buf.ctypes.data, 0, 16, 8, out.ctypes.data) == _lib.SERQ_EINVAL
    assert pre(buf.ctypes.data, 4, 18, 8, out.ctypes.data) == _lib.SERQ_EINVAL    # k > 2 pitch
    assert pre(buf.ctypes.data, 4, 15, 8, out.ctypes.data) == _lib.SERQ_EINVAL    # odd k


@pytest.mark.parametrize("rows,k,pitch", [(1, 2, 1), (5, 30, 16), (130, 300, 150), (128, 256, 128),
                                          (33, 72, 48), (256, 1024, 512)])
def test_prepack_bf6_layout(rows, k, pitch):
    """serq_prepack_bf6 against a reader written from the header's statement
    of the layout and of E3M2: every field decodes to its int4 code, every
    code of [-8, 7] occurs, the padding is zero, and bytes of the pitch past
    k are ignored."""
    rng = np.random.default_rng(rows * 7 + k)
    c = rng.integers(-8, 8, (rows, k)).astype(np.int8)
    c.flat[:16] = np.arange(-8, 8)[: min(16, c.size)]
    packed = np.zeros((rows, pitch), np.uint8)
    packed[:, : k // 2] = O.pack_int4(c)
    packed[:, k // 2:] = 0xA5                      # junk beyond the k codes
    out = S._prepack(packed, rows, k, pitch)
    full, codes = bf6_decode(out, rows, k)
    assert np.array_equal(codes, c)
    pad = full.copy()
    pad[:rows, :k] = 0
    assert not pad.any()


def test_prepack_bf6_of_a_calibrated_layer():
    """Q(W^) and Q(R) of a calibrated layer survive the re-encoding."""
    li = make_layer(384, 200, 1, n_out=3, factor=20.0, seed=11, tag=2)
    L = S.calibrate(li.W, li.act_absmax, r=72)
    B = S.prepack_bf6(L)
    _, wc = bf6_decode(B.W6, L.N, L.K)
    _, rc = bf6_decode(B.R6, L.N, L.r)
    assert np.array_equal(wc, O.unpack_int4(L.Wq))
    assert np.array_equal(rc, O.unpack_int4(np.ascontiguousarray(L.Rq[:, : L.r // 2])))


def test_bf6_tile_choice():
    """serq_linear_bf6 takes 256 x 256 tiles only where the 128-row padding
    of both operands is a multiple of 256 and the tiles give every one of the
    256 CUs one; else 128 x 128."""
    assert _lib.lib.serq_linear_bf6_kernel_name(0, 4096, 0) is None
    assert _lib.lib.serq_linear_bf6_kernel_name(16, -1, 0) is None
    assert _lib.lib.serq_linear_bf6_kernel_name(16, 16, -2) is None
    for M, N in [(2048, 4096), (4096, 4096), (4000, 4096), (3900, 4096), (4096, 4000), (4096, 3800),
                 (8192, 28672), (1024, 16384), (1000, 16284), (512, 4096), (1, 1), (2048, 8192)]:
        mp, np_ = -(-M // 128) * 128, -(-N // 128) * 128
        wide = mp % 256 == 0 and np_ % 256 == 0 and (mp // 256) * (np_ // 256) >= 256
        assert S.bf6_kernel_name(M, N, 64) == ("bf6_tile256x256" if wide else "bf6_tile128x128"), (M, N)


def test_python_wrapper_raises():
    with pytest.raises(S.SerqError):
        S.calibrate(np.zeros((5, 4), np.float32), np.ones(5, np.float32), r=2)   # odd K
    with pytest.raises(S.SerqError):
        S.calibrate(np.zeros((4, 4), np.float32), np.ones(4, np.float32), r=6)   # r > K


def test_calibrate_argument_errors():
    W = np.zeros((8, 4), np.float32)
    a = np.ones(8, np.float32)
    out = [np.zeros(8, np.int32), np.zeros(8, np.float32), np.zeros((4, 4), np.uint8), np.zeros(4, np.float32),
           np.zeros((4, rq_row_bytes(2)), np.uint8), np.zeros(4, np.float32)]
    p = [o.ctypes.data for o in out]
    c = _lib.lib.serq_calibrate
    assert c(W.ctypes.data, 0, 8, 4, a.ctypes.data, 0.5, 2, *p) == _lib.SERQ_OK
    assert c(W.ctypes.data, 0, 8, 4, a.ctypes.data, 1.5, 2, *p) == _lib.SERQ_EINVAL
    assert c(W.ctypes.data, 3, 8, 4, a.ctypes.data, 0.5, 2, *p) == _lib.SERQ_EINVAL
    assert c(W.ctypes.data, 0, 8, 4, a.ctypes.data, 0.5, 3, *p) == _lib.SERQ_EINVAL
    assert c(None, 0, 8, 4, a.ctypes.data, 0.5, 2, *p) == _lib.SERQ_EINVAL
    assert c(W.ctypes.data, 0, 8, 4, a.ctypes.data, 0.5, 2, *p[:4], None, None) == _lib.SERQ_EINVAL
    # an all-zero weight: every column quantizes to zero codes with scale 0
    assert np.all(out[3] == 0) and np.all(out[2] == 0)


# ---------------------------------------------------------------- calibration parity

def assert_layer_equal(L, R, cols=None):
    sel = slice(None) if cols is None else np.asarray(cols)
    assert np.array_equal(L.perm, R["perm"])
    assert np.array_equal(L.s_hat_inv.view(np.uint32), np.asarray(R["s_hat_inv"], np.float32).view(np.uint32))
    assert np.array_equal(L.Wq[sel], R["Wq"])
    assert np.array_equal(L.sw[sel].view(np.uint32), R["sw"].view(np.uint32))
    assert np.array_equal(L.Rq[sel], pad_rq(R["Rq"], L.r))
    assert np.array_equal(L.sr[sel].view(np.uint32), R["sr"].view(np.uint32))


@pytest.mark.parametrize("K,N,r,dtype,alpha,seed", [
    (256, 256, 8, "f32", 0.5, 0), (64, 40, 0, "f32", 0.5, 1), (96, 33, 96, "bf16", 0.5, 2),
    (130, 17, 6, "bf16", 0.5, 3), (512, 64, 64, "f32", 0.3, 4), (512, 64, 128, "bf16", 0.8, 5),
    (2, 1, 2, "f32", 0.5, 6),
])
def test_calibrate_matches_oracle(K, N, r, dtype, alpha, seed):
    li = make_layer(K, N, 1, n_out=max(1, K // 100), factor=50.0, seed=seed, tag=7, dtype=dtype)
    W = li.W_bits if dtype == "bf16" else li.W
    L = S.calibrate(W, li.act_absmax, r=r, alpha=alpha)
    R = O.calibrate(li.W, li.act_absmax, r=r, alpha=alpha)
    assert_layer_equal(L, R)


def test_calibrate_ties_and_dead_channels():
    # equal smoothing factors (ties), dead activation channels, zero weight rows/columns
    K, N = 64, 24
    rng = np.random.default_rng(3)
    W = (0.02 * rng.standard_normal((K, N))).astype(np.float32)
    W[5] = 0.0
    W[:, 7] = 0.0
    amax = np.ones(K, np.float32)
    amax[[1, 9, 33]] = 0.0
    W[[2, 3, 4]] = W[2]     # identical rows -> identical s
    L = S.calibrate(W, amax, r=16)
    R = O.calibrate(W, amax, r=16)
    assert_layer_equal(L, R)
    assert L.sw[7] == 0 and not L.Wq[7].any()


@pytest.mark.slow
@pytest.mark.parametrize("workload,layer", [
    ("q_proj", "q_proj"), ("mlp8b", "down"), ("l70b", "up70"), ("l70b", "down70"),
])
def test_calibrate_full_size_sampled_columns(workload, layer):
    li = workload_layer(workload, layer, M_max=1, draw_x=False)
    r = li.meta["r"]
    L = S.calibrate(li.W_bits, li.act_absmax, r=r)
    cols = np.random.default_rng(0).choice(li.N, 48, replace=False)
    R = O.calibrate_columns(li.W, li.act_absmax, cols, r=r)
    assert_layer_equal(L, R, cols)


@pytest.mark.slow
def test_calibrate_gate_up_shared_input():
    """gate and up share their input, hence s and P: calibrated on [W_g | W_u]."""
    li = workload_layer("mlp8b", "gate_up", M_max=1, draw_x=False)
    Wcat = np.concatenate([li.W_bits, li.meta["W_up_bits"]], axis=1)
    L = S.calibrate(Wcat, li.act_absmax, r=128)
    Wf = np.concatenate([li.W, li.meta["W_up"]], axis=1)
    cols = np.random.default_rng(1).choice(Wf.shape[1], 48, replace=False)
    R = O.calibrate_columns(Wf, li.act_absmax, cols, r=128)
    assert_layer_equal(L, R, cols)


# ---------------------------------------------------------------- GPTQ calibration parity

def _gptq_inputs(K, N, T, seed, corr=0.4):
    rng = np.random.default_rng(seed)
    A = (rng.standard_normal((K, K)) * corr + np.eye(K)).astype(np.float32)
    Xc = (rng.standard_normal((T, K)).astype(np.float32) @ A).astype(np.float32)
    Xc[:, rng.choice(K, max(1, K // 50), replace=False)] *= np.float32(30.0)
    W = (0.02 * rng.standard_normal((K, N))).astype(np.float32)
    return W, Xc


@pytest.mark.parametrize("K,N,T,r,wdt,xdt,damp,seed", [
    (64, 40, 128, 8, "f32", "f32", 0.01, 0), (128, 96, 256, 0, "f32", "f32", 0.01, 1),
    (96, 33, 50, 96, "bf16", "f32", 0.01, 2), (256, 130, 256, 32, "bf16", "bf16", 0.1, 3),
    (40, 24, 64, 6, "f32", "bf16", 0.0, 4), (512, 70, 300, 64, "f32", "f32", 0.01, 5),
    (2, 1, 3, 0, "f32", "f32", 0.01, 6),
])
def test_calibrate_gptq_matches_oracle(K, N, T, r, wdt, xdt, damp, seed):
    """serq_calibrate_gptq bit for bit against the oracle's GPTQ (every output
    buffer), f32 and bf16 weights and calibration inputs, r = 0 and r = K,
    with and without dampening."""
    W, Xc = _gptq_inputs(K, N, T, seed)
    if wdt == "bf16":
        Wb = round_to_bf16_bits(W).reshape(K, N)
        W, W_in = bf16_bits_to_f32(Wb).reshape(K, N), Wb
    else:
        W_in = W
    if xdt == "bf16":
        Xb = round_to_bf16_bits(Xc).reshape(T, K)
        Xc, X_in = bf16_bits_to_f32(Xb).reshape(T, K), Xb
    else:
        X_in = Xc
    a = np.abs(Xc).max(axis=0).astype(np.float32)
    L = S.calibrate_gptq(W_in, a, X_in, r=r, damp=damp)
    R = O.calibrate_gptq(W, a, Xc, r=r, damp=damp)
    assert_layer_equal(L, R)


def test_calibrate_gptq_dead_channels_and_zero_inputs():
    """A channel that is zero in every calibration token (zero activation
    maximum, an all-zero Hessian row, kept positive definite by the
    dampening), an all-zero weight row, and all-zero calibration inputs (the
    identity Hessian: RTN's codes)."""
    W, Xc = _gptq_inputs(48, 20, 96, 9)
    Xc[:, 7] = 0.0
    W[11] = 0.0
    a = np.abs(Xc).max(axis=0).astype(np.float32)
    assert_layer_equal(S.calibrate_gptq(W, a, Xc, r=6), O.calibrate_gptq(W, a, Xc, r=6))
    Z = np.zeros_like(Xc)
    L = S.calibrate_gptq(W, a, Z, r=6)
    assert_layer_equal(L, O.calibrate_gptq(W, a, Z, r=6))
    assert_layer_equal(L, O.calibrate(W, a, r=6))


def test_calibrate_gptq_argument_errors():
    W, Xc = _gptq_inputs(8, 4, 16, 1)
    a = np.abs(Xc).max(axis=0).astype(np.float32)
    out = [np.zeros(8, np.int32), np.zeros(8, np.float32), np.zeros((4, 4), np.uint8), np.zeros(4, np.float32),
           np.zeros((4, rq_row_bytes(2)), np.uint8), np.zeros(4, np.float32)]
    p = [o.ctypes.data for o in out]
    g = _lib.lib.serq_calibrate_gptq
    ok = (W.ctypes.data, 0, 8, 4, a.ctypes.data, 0.5, 2, Xc.ctypes.data, 0, 16, 0.01)
    assert g(*ok, *p) == _lib.SERQ_OK
    for i, bad in ((7, None), (8, 5), (9, 0), (9, -1), (10, -0.5), (10, float("nan")), (10, float("inf")),
                   (6, 3), (1, 7)):
        args = list(ok)
        args[i] = bad
        assert g(*args, *p) == _lib.SERQ_EINVAL, (i, bad)
    # fewer tokens than channels and no dampening: H is singular
    assert g(W.ctypes.data, 0, 8, 4, a.ctypes.data, 0.5, 2, Xc.ctypes.data, 0, 3, 0.0, *p) == _lib.SERQ_EINVAL
    with pytest.raises(ValueError):
        O.calibrate_gptq(W, a, Xc[:3], r=2, damp=0.0)
    with pytest.raises(ValueError):
        S.calibrate_gptq(W, a, Xc[:, :6], r=2)


# ---------------------------------------------------------------- MXFP4 calibration parity

@pytest.mark.parametrize("K,N,r,dtype,seed", [
    (256, 40, 64, "f32", 0), (128, 33, 0, "bf16", 1), (96, 17, 96, "f32", 2), (512, 64, 128, "bf16", 3),
    (32, 1, 32, "f32", 4), (1024, 100, 256, "bf16", 5),
])
def test_calibrate_mx_matches_oracle(K, N, r, dtype, seed):
    """serq_calibrate_mx bit for bit against the oracle's MXFP4 calibration:
    perm, s_hat_inv, FP4 codes and E8M0 bytes of Q(W^) and Q(R), with an
    all-zero column, a column of huge values and one of tiny values."""
    li = make_layer(K, N, 1, n_out=2, factor=30.0, seed=seed, tag=31, dtype=dtype)
    W = li.W.copy()
    if N > 3:
        W[:, 1] = 0.0
        W[:, 2] *= np.float32(1e30)
        W[:, 3] *= np.float32(1e-30)
    W_in = round_to_bf16_bits(W).reshape(K, N) if dtype == "bf16" else W
    if dtype == "bf16":
        W = bf16_bits_to_f32(W_in).reshape(K, N)
    L = S.calibrate_mx(W_in, li.act_absmax, r=r)
    R = O.calibrate_mx(W, li.act_absmax, r=r)
    assert np.array_equal(L.perm, R["perm"])
    assert np.array_equal(L.s_hat_inv.view(np.uint32), R["s_hat_inv"].view(np.uint32))
    for k in ("Wq", "Wsc", "Rq", "Rsc"):
        assert np.array_equal(getattr(L, k), R[k]), k


def test_mx_argument_errors():
    W = np.ones((64, 4), np.float32)
    a = np.ones(64, np.float32)
    out = [np.zeros(64, np.int32), np.zeros(64, np.float32), np.zeros((4, 32), np.uint8), np.zeros((4, 2), np.uint8),
           np.zeros((4, 16), np.uint8), np.zeros((4, 1), np.uint8)]
    p = [o.ctypes.data for o in out]
    c = _lib.lib.serq_calibrate_mx
    assert c(W.ctypes.data, 0, 64, 4, a.ctypes.data, 0.5, 32, *p) == _lib.SERQ_OK
    assert c(W.ctypes.data, 0, 48, 4, a.ctypes.data, 0.5, 32, *p) == _lib.SERQ_EINVAL      # K % 32
    assert c(W.ctypes.data, 0, 64, 4, a.ctypes.data, 0.5, 16, *p) == _lib.SERQ_EINVAL      # r % 32
    assert c(W.ctypes.data, 0, 64, 4, a.ctypes.data, 0.5, 96, *p) == _lib.SERQ_EINVAL      # r > K
    assert c(W.ctypes.data, 0, 64, 4, a.ctypes.data, 0.5, 32, *p[:4], None, None) == _lib.SERQ_EINVAL
    q = _lib.lib.serq_quant_act_mx
    assert q(A16, _lib.SERQ_BF16, 4, 48, A16, A16, A16, None) == _lib.SERQ_EINVAL           # K % 32
    assert q(A16, 5, 4, 64, A16, A16, A16, None) == _lib.SERQ_EINVAL                        # dtype
    assert q(A16, _lib.SERQ_BF16, -1, 64, A16, A16, A16, None) == _lib.SERQ_EINVAL
    assert q(A16 + 2, _lib.SERQ_BF16, 4, 64, A16, A16, A16, None) == _lib.SERQ_EALIGN
    assert q(None, _lib.SERQ_BF16, 0, 64, A16, None, None, None) == _lib.SERQ_OK            # M = 0: no-op
    f = _lib.lib.serq_linear_mx
    ok = [A16, A16, A16, A16, A16, A16, 4, 64, 32, 32, A16, _lib.SERQ_BF16, None, None, None]
    for i, bad, code in ((7, 48, _lib.SERQ_EINVAL), (9, 16, _lib.SERQ_EINVAL), (9, 96, _lib.SERQ_EINVAL),
                         (8, 0, _lib.SERQ_EINVAL), (11, 7, _lib.SERQ_EINVAL), (2, A16 + 4, _lib.SERQ_EALIGN),
                         (0, A16 + 8, _lib.SERQ_EALIGN), (10, A16 + 2, _lib.SERQ_EALIGN), (4, None, _lib.SERQ_EINVAL),
                         (12, A16, _lib.SERQ_EINVAL)):
        args = list(ok)
        args[i] = bad
        assert f(*args) == code, (i, bad)
    args = list(ok)
    args[6] = 0
    assert f(*args) == _lib.SERQ_OK                                                           # M = 0: no-op


def test_permute_outputs_matches_oracle():
    li = make_layer(64, 40, 1, n_out=2, factor=30.0, seed=9, tag=1, dtype="f32")
    L = S.calibrate(li.W, li.act_absmax, r=16)
    R = O.calibrate(li.W, li.act_absmax, r=16)
    p = np.random.default_rng(4).permutation(40).astype(np.int32)
    S.permute_outputs(L, p)
    assert_layer_equal(L, O.permute_outputs(R, p))


def test_permute_outputs_rejects_non_permutation():
    li = make_layer(16, 8, 1, n_out=1, factor=30.0, seed=9, tag=1, dtype="f32")
    L = S.calibrate(li.W, li.act_absmax, r=4)
    before = L.Wq.copy()
    with pytest.raises(S.SerqError):
        S.permute_outputs(L, np.array([0, 1, 2, 3, 4, 5, 6, 6], np.int32))
    with pytest.raises(S.SerqError):
        S.permute_outputs(L, np.array([0, 1, 2, 3, 4, 5, 6, 8], np.int32))
    assert np.array_equal(before, L.Wq)


def test_layer_save_load_roundtrip(tmp_path):
    li = make_layer(64, 24, 1, n_out=2, factor=30.0, seed=2, tag=1, dtype="bf16")
    L = S.calibrate(li.W_bits, li.act_absmax, r=8)
    L.save(str(tmp_path / "layer.npz"))
    L2 = S.SerqLayer.load(str(tmp_path / "layer.npz"))
    for k in ("perm", "s_hat_inv", "Wq", "sw", "Rq", "sr"):
        assert np.array_equal(getattr(L, k), getattr(L2, k))


def test_kernel_dispatch_rules():
    assert S.kernel_name(1, 4096, 4096, 64) == "gemv"
    assert S.kernel_name(3, 4096, 4096, 64) == "gemv"
    assert S.kernel_name(4, 4096, 4096, 64) == "decode16"
    assert S.kernel_name(4, 4096, 4096, 64, 8) == "decode16"     # W4A8: no int4 dot products
    assert S.kernel_name(4, 65536, 4096, 64) == "decode16"       # activation rows beyond the GEMV's LDS budget
    assert S.kernel_name(5, 4096, 4096, 64) == "decode16"
    assert S.kernel_name(16, 4096, 4096, 64) == "decode16"
    assert S.kernel_name(32, 4096, 14336, 128) == "decode32"
    # 256 x 256 tiles where their rounds (256 tiles each) take less time than
    # the rounds of 128 x 128 tiles (512 each, half the work)
    assert S.kernel_name(4096, 4096, 28672, 128) == "tile256x256"      # 7 rounds against 14
    assert S.kernel_name(4096, 4096, 28672, 128, 8) == "tile128x128"   # W4A8: 128 x 128 tiles
    assert S.kernel_name(4096, 14336, 4096, 128) == "tile256x256"      # 1 round against 2
    assert S.kernel_name(4096, 4096, 14336, 128) == "tile128x128"      # 3.5 rounds (4) against 7
    assert S.kernel_name(2048, 4096, 28672, 128) == "tile128x128"      # 3.5 rounds (4) against 7
    assert S.kernel_name(300, 4096, 32768, 64) == "tile256x256"        # 1 round against 1.5 (2)
    assert S.kernel_name(2048, 4096, 4096, 64) == "tile128x128"        # 1 round against 1
    assert S.kernel_name(65, 4096, 4096, 64) == "tile32x64k4"          # 128 tiles of 64 x 64: half the CUs
    assert S.kernel_name(128, 14336, 4096, 128) == "tile32x64k4"
    assert S.kernel_name(129, 14336, 4096, 64) == "tile64x64k4"      # 192 tiles of 64 x 64, long K
    assert S.kernel_name(256, 14336, 4096, 64) == "tile64x64k4"      # 256 tiles of 64 x 64, long K
    assert S.kernel_name(256, 4096, 4096, 64) == "tile64x64k2"       # 32 k-tiles: two groups
    assert S.kernel_name(256, 4096, 4096, 64, 8) == "tile64x64"      # W4A8: one group
    assert S.kernel_name(384, 4096, 4096, 64) == "tile64x64k2"       # 384 tiles of 64 x 64
    assert S.kernel_name(40, 4096, 28672, 128) == "tile64x64k2"      # 448 tiles of 64 x 64
    assert S.kernel_name(256, 1024, 4096, 64) == "tile64x64k2"       # eight k-tiles
    assert S.kernel_name(256, 992, 4096, 64) == "tile64x64"          # under eight k-tiles: one group
    assert S.kernel_name(64, 4096, 32768, 64) == "tile64x128"        # 256 tiles of 64 x 128
    # W4A4 from 256 tokens: 64 x 64 tiles with two k-groups where they are one round of two per CU
    assert S.kernel_name(512, 4096, 4096, 64) == "tile64x64k2"
    assert S.kernel_name(512, 14336, 4096, 128) == "tile64x64k2"
    assert S.kernel_name(256, 28672, 8192, 256) == "tile64x64k2"
    assert S.kernel_name(512, 4096, 4096, 64, 8) == "tile64x128"      # W4A8 unchanged
    assert S.kernel_name(640, 4096, 4096, 64) == "tile64x128"        # 640 tiles of 64 x 64: more than a round
    assert S.kernel_name(512, 992, 4096, 64) == "tile64x128"         # under eight k-tiles
    # exactly one 128 x 128 tile per CU and K >= 8192 (W4A4): two k-groups
    assert S.kernel_name(1024, 14336, 4096, 128) == "tile128x128k2"
    assert S.kernel_name(512, 28672, 8192, 256) == "tile128x128k2"
    assert S.kernel_name(1024, 14336, 4096, 128, 8) == "tile128x128"
    assert S.kernel_name(1024, 28672, 8192, 256) == "tile128x128"    # 512 tiles
    assert S.kernel_name(768, 4096, 4096, 64) == "tile128x128k2"     # 192 tiles of 128 x 128: two k-groups
    assert S.kernel_name(1024, 4096, 4096, 64) == "tile128x128"
    assert S.kernel_name(64, 4096, 4096, 64) == "tile32x64k4"
    assert S.kernel_name(16, 4100, 64, 8) == "generic"      # K % 32 != 0
    assert S.kernel_name(16, 4096, 64, 6) == "generic"      # r % 8 != 0
    assert S.kernel_name(16, 4096, 64, 512) == "generic"    # r > 256
    assert S.kernel_name(16, 63, 64, 8) is None


def test_kernel_dispatch_long_rows():
    """The MFMA kernels sum widened codes (256x the products for W4A4, 16x for
    W4A8), exact in int32 for K < 2^17; from 2^17 on only the int4
    dot-product GEMV (unscaled sums) and the generic kernel serve."""
    assert S.kernel_name(64, 131040, 64, 8) == "tile32x64k4"
    assert S.kernel_name(64, 131072, 64, 8) == "generic"
    assert S.kernel_name(8, 131072, 64, 8, 8) == "generic"
    assert S.kernel_name(1, 131072, 64, 8) == "gemv"


def test_kernel_dispatch_split_scratch_bound():
    """The K split's partial sums live in 16 MiB of file-scope device scratch:
    shapes whose split would need more take a tile kernel instead (nothing is
    allocated and no size is refused). A 32-token split keeps 2 x 32 x 16 x 4
    bytes per 16 output channels and K slice."""
    assert S.kernel_name(32, 14336, 4096, 128) == "decode32_ksplit"      # 8B down: 256 groups x 2 slices
    assert S.kernel_name(32, 28672, 8192, 256) == "decode32_ksplit"      # 70B down: 512 groups x 4 slices
    assert S.kernel_name(32, 28672, 8192, 256, 8) == "decode32_ksplit"   # W4A8: 512 groups x 8 slices (16 MiB)
    assert S.kernel_name(20, 14336, 4096, 128) == "decode32"             # fits in LDS: one slice
    # 2048 groups x 8 slices x 4 KB = 64 MiB of partial sums: no split, no skinny kernel
    name = S.kernel_name(32, 65536, 32768, 64)
    assert name.startswith("tile"), name
    # W4A8 at 16 tokens: 1024 groups x 14 slices x 2 KB = 28 MiB
    assert S.kernel_name(16, 131040, 16384, 64, 4) == "decode16_ksplit"   # 7 slices: 14 MiB
    name = S.kernel_name(16, 131040, 16384, 64, 8)
    assert name.startswith("tile"), name


def test_single_hip_runtime_in_process():
    """Importing the package before torch must not load a second HIP runtime
    next to the one PyTorch ships (they would not share streams or memory)."""
    import subprocess
    import sys
    code = ("import re, w4a4_linear_layers_amd, torch\n"
            "m = open('/proc/self/maps').read()\n"
            "print(len(set(re.findall(r'/\\S*libamdhip64\\S*', m))))\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "1", out.stdout
