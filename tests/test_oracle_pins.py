"""The oracle against its pins, and planted mistakes against the pins.

Every pin in oracle_pins.py must pass on the oracle. Each mutant below plants
one plausible mistake in the oracle (on the CPU, through monkeypatch) and at
least one pin must then fail: a dropped term, a wrong sign, a wrong index, a
transposed or inverted permutation, a wrong rounding rule or a wrong scale.
"""

import os

import numpy as np
import pytest

import oracle_pins as P
from oracle import serq_oracle as O


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check(O)


# ------------------------------------------------------------------ mutants

def _mut_compensator_sign(orig):
    return lambda Wh, Wd, r: (Wd[:r] - Wh[:r]).astype(np.float32)


def _mut_saliency_ascending(orig):
    return lambda s: np.argsort(np.asarray(s, np.float64), kind="stable").astype(np.int32)


def _mut_round_half_up(orig):
    def q(v, m, bits):
        lo, hi = O.qrange(bits)
        v = np.asarray(v, np.float32)
        m = np.float32(m)
        if m == 0:
            return np.zeros(v.shape, np.int8), np.float32(0)
        inv = np.float32(np.float32(hi) / m)
        t = (v * inv).astype(np.float32)
        return np.clip(np.floor(t + np.float32(0.5)), lo, hi).astype(np.int8), np.float32(m / np.float32(hi))
    return q


def _mut_scale_over_8(orig):
    def q(v, m, bits):
        lo, hi = O.qrange(bits)
        v = np.asarray(v, np.float32)
        m = np.float32(m)
        if m == 0:
            return np.zeros(v.shape, np.int8), np.float32(0)
        inv = np.float32(np.float32(-lo) / m)
        t = (v * inv).astype(np.float32)
        return np.clip(np.rint(t), lo, hi).astype(np.int8), np.float32(m / np.float32(-lo))
    return q


def _mut_drop_residual(orig):
    def f(Xc, Wc, Rc, r):
        am, ar = orig(Xc, Wc, Rc, r)
        return am, np.zeros_like(ar)
    return f


def _mut_residual_last_columns(orig):
    def f(Xc, Wc, Rc, r):
        am, _ = orig(Xc, Wc, Rc, 0)
        Xc = np.asarray(Xc, np.int64)
        ar = Xc[:, Xc.shape[1] - r:] @ np.asarray(Rc, np.int64) if r else np.zeros_like(am)
        return am, ar
    return f


def _mut_inverse_perm_fold(orig):
    def f(W, s, perm):
        inv = np.argsort(perm)
        return orig(W, s, inv)
    return f


def _mut_quant_act_ignores_sinv(orig):
    return lambda X, s_hat_inv, a_bits: orig(X, np.ones_like(s_hat_inv), a_bits)


def _mut_pack_swapped(orig):
    def f(codes):
        c = np.asarray(codes, np.int64)
        return ((c[..., 1::2] & 0xF) | ((c[..., 0::2] & 0xF) << 4)).astype(np.uint8)
    return f


def _mut_epilogue_sw_for_both(orig):
    return lambda am, ar, sx, sw, sr: orig(am, ar, sx, sw, sw)


def _mut_per_tensor_weights(orig):
    def f(A, bits):
        A = np.asarray(A, np.float32)
        codes = np.zeros(A.shape, np.int8)
        scales = np.zeros(A.shape[1], np.float32)
        if A.size:
            codes, sc = O.quantize_group(A, np.abs(A).max(), bits)
            scales[:] = sc
        return codes, scales
    return f


def _mut_alpha_swapped(orig):
    return lambda a, w, alpha=0.5: orig(w, a, alpha)


def _mut_bf16_via_f32(orig):
    def f(y):
        y32 = np.asarray(y, np.float64).astype(np.float32)
        u = y32.view(np.uint32).astype(np.uint64)
        lsb = (u >> np.uint64(16)) & np.uint64(1)
        u = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
        return u.astype(np.uint32).view(np.float32)
    return f


def _mut_exp_drops_ln2_lo(orig):
    def f(x):
        x = np.clip(np.asarray(x, np.float32), -O.EXP_ARG_CLAMP, O.EXP_ARG_CLAMP).astype(np.float32)
        n = np.rint((x * O.LOG2E_F32).astype(np.float32)).astype(np.float32)
        r = O.fma32(-n, O.LN2_HI_F32, x)
        p = np.full(x.shape, O.EXP_TAYLOR_F32[7], np.float32)
        for k in range(6, -1, -1):
            p = O.fma32(p, r, O.EXP_TAYLOR_F32[k])
        return np.ldexp(p, n.astype(np.int32)).astype(np.float32)
    return f


def _mut_fma_double_rounding(orig):
    def f(a, b, c):
        a64, b64, c64 = (np.asarray(v, np.float32).astype(np.float64) for v in (a, b, c))
        return (a64 * b64 + c64).astype(np.float32)
    return f


def _mut_silu_sign(orig):
    def f(G, U):
        g = np.asarray(G, np.float32)
        s = (np.float32(1.0) + O.exp32(g)).astype(np.float32)
        return ((g / s).astype(np.float32) * np.asarray(U, np.float32)).astype(np.float32)
    return f


def _mut_fused_skips_silu(orig):
    return lambda G, U, s_hat_inv, a_bits: O.quant_act((np.asarray(G, np.float32) * np.asarray(U, np.float32)).astype(np.float32), s_hat_inv, a_bits)


def _mut_columns_s_from_sampled(orig):
    """s formed from the sampled columns' row maxima instead of all of W."""
    def f(W, act_absmax, cols, *, alpha=O.ALPHA_DEFAULT, r):
        W = np.asarray(W, np.float32)
        Wc = W[:, cols]
        s, s_inv = O.smoothing_factors(act_absmax, np.abs(Wc).max(axis=1), alpha)
        perm = O.saliency_order(s)
        W_hat = O.fold_and_permute(Wc, s, perm)
        Wq_codes, sw = O.quantize_columns(W_hat, 4)
        R = O.compensator(W_hat, O.dequantize_columns(Wq_codes, sw), r)
        Rq_codes, sr = O.quantize_columns(R, 4)
        return dict(s=s, s_inv=s_inv, perm=perm, s_hat_inv=s_inv[perm], cols=np.asarray(cols),
                    Wq_codes=Wq_codes, sw=sw, Rq_codes=Rq_codes, sr=sr, Wq=O.pack_int4(Wq_codes.T),
                    Rq=O.pack_int4(Rq_codes.T) if r else np.zeros((len(cols), 0), np.uint8))
    return f


def _mut_columns_codes_shifted(orig):
    """An off-by-one in the sampled columns (the next column's codes)."""
    def f(W, act_absmax, cols, **kw):
        W = np.asarray(W, np.float32)
        cols = np.asarray(cols)
        return orig(W, act_absmax, np.minimum(cols + 1, W.shape[1] - 1), **kw)
    return f


def _mut_gptq_propagates_salient(orig):
    """The salient rows' errors moved onto later rows as well (corrected
    twice: once by R, once by GPTQ)."""
    return lambda W_hat, U, r: orig(W_hat, U, 0)


def _mut_gptq_update_sign(orig):
    def f(W_hat, U, r):
        return orig(W_hat, -np.triu(U, 1) + np.diag(np.diag(U)), r)
    return f


def _mut_gptq_no_damping(orig):
    return lambda X_hat, damp=O.GPTQ_DAMP: orig(X_hat, 0.0)


def _mut_gptq_unflattened_inputs(orig):
    """The Hessian from the calibration inputs in their original order,
    without the flattening (not what the layer sees)."""
    def f(W, act_absmax, X_cal, *, alpha=O.ALPHA_DEFAULT, r, damp=O.GPTQ_DAMP):
        base = O.calibrate(W, act_absmax, alpha=alpha, r=r)
        U = O.gptq_inverse_factor(O.gptq_hessian(np.asarray(X_cal, np.float32), damp))
        codes = O.gptq_quantize(base["W_hat"], U, r)
        out = dict(base)
        out.update(Wq_codes=codes, W_deq=O.dequantize_columns(codes, base["sw"]), Wq=O.pack_int4(codes.T),
                   H=None, U=U, X_hat_cal=(np.asarray(X_cal, np.float32)[:, base["perm"]]
                                           * base["s_hat_inv"][None, :]).astype(np.float32))
        return out
    return f


def _mut_e2m1_ties_away(orig):
    """Ties rounded away from zero instead of to the even mantissa."""
    def f(t):
        t = np.asarray(t, np.float64)
        a = np.minimum(np.abs(t), 6.0)
        d = np.abs(a[..., None] - O.E2M1_VALUES)
        best = d.min(axis=-1, keepdims=True)
        cand = d == best
        mag = 7 - np.argmax(cand[..., ::-1], axis=-1)          # the larger of the nearest
        sign = (t < 0) & (mag != 0)
        return (mag | (sign.astype(np.int64) << 3)).astype(np.uint8)
    return f


def _mut_mx_exponent_no_offset(orig):
    """The shared exponent without E2M1's largest exponent subtracted."""
    return lambda amax: np.clip(orig(amax) + 2, -127, 127)


def _mut_mx_blocks_along_n(orig):
    """Weight blocks of 32 output channels (along N) instead of along K."""
    def f(W, act_absmax, *, alpha=O.ALPHA_DEFAULT, r):
        L = orig(W, act_absmax, alpha=alpha, r=r)
        Wh = L["W_hat"]
        K, N = Wh.shape
        pad = (-N) % 32
        Wp = np.concatenate([Wh, np.zeros((K, pad), np.float32)], axis=1)
        c, e = O.mx_quantize_rows(Wp)
        deq = O.mx_dequantize_rows(c, e)[:, :N]
        c2, e2 = O.mx_quantize_rows(deq.T)
        L = dict(L)
        L.update(Wq_codes=c2, We=e2, W_deq=O.mx_dequantize_rows(c2, e2).T, Wq=O.pack_fp4(c2))
        return L
    return f


def _mut_mx_residual_last_blocks(orig):
    def f(Xq, layer):
        out = orig(Xq, layer)
        r = layer["r"]
        if r:
            Xq2 = dict(Xq)
            Xq2["codes"] = np.roll(Xq["codes"], r, axis=1)
            Xq2["e"] = np.roll(Xq["e"], r // 32, axis=1)
            out2 = orig(Xq2, layer)
            out = dict(out)
            out["acc_res"] = out2["acc_res"]
        return out
    return f


MUTANTS = {
    "compensator_sign": ("compensator", _mut_compensator_sign),
    "saliency_ascending": ("saliency_order", _mut_saliency_ascending),
    "round_half_up": ("quantize_group", _mut_round_half_up),
    "scale_over_8": ("quantize_group", _mut_scale_over_8),
    "drop_residual": ("linear_int", _mut_drop_residual),
    "residual_last_columns": ("linear_int", _mut_residual_last_columns),
    "inverse_perm_fold": ("fold_and_permute", _mut_inverse_perm_fold),
    "quant_act_ignores_sinv": ("quant_act", _mut_quant_act_ignores_sinv),
    "pack_swapped": ("pack_int4", _mut_pack_swapped),
    "epilogue_sw_for_both": ("epilogue", _mut_epilogue_sw_for_both),
    "per_tensor_weights": ("quantize_columns", _mut_per_tensor_weights),
    "alpha_swapped": ("smoothing_factors", _mut_alpha_swapped),
    "bf16_double_rounding": ("round_f64_to_bf16", _mut_bf16_via_f32),
    "exp_drops_ln2_lo": ("exp32", _mut_exp_drops_ln2_lo),
    "fma_double_rounding": ("fma32", _mut_fma_double_rounding),
    "silu_sign": ("silu_mul", _mut_silu_sign),
    "fused_skips_silu": ("silu_mul_quant_act", _mut_fused_skips_silu),
    "columns_s_from_sampled": ("calibrate_columns", _mut_columns_s_from_sampled),
    "columns_codes_shifted": ("calibrate_columns", _mut_columns_codes_shifted),
    "gptq_propagates_salient": ("gptq_quantize", _mut_gptq_propagates_salient),
    "gptq_update_sign": ("gptq_quantize", _mut_gptq_update_sign),
    "gptq_no_damping": ("gptq_hessian", _mut_gptq_no_damping),
    "gptq_unflattened_inputs": ("calibrate_gptq", _mut_gptq_unflattened_inputs),
    "e2m1_ties_away": ("e2m1_round", _mut_e2m1_ties_away),
    "mx_exponent_no_offset": ("mx_block_exponent", _mut_mx_exponent_no_offset),
    "mx_blocks_along_n": ("calibrate_mx", _mut_mx_blocks_along_n),
    "mx_residual_last_blocks": ("linear_mx", _mut_mx_residual_last_blocks),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, make = MUTANTS[name]
    orig = getattr(O, attr)
    monkeypatch.setattr(O, attr, make(orig))
    caught = []
    for check in P.ALL_CHECKS:
        try:
            check(O)
        except (AssertionError, ValueError, IndexError):
            caught.append(check.__name__)
    assert caught, f"no pin catches mutant {name}"


def test_worked_layer_fixture_is_the_exact_derivation():
    """The worked 4 x 2 layer fixture equals its exact-rational derivation
    (tests/golden/derive_worked_layer.py, independent of the oracle), value
    for value."""
    import importlib.util
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "derive_worked_layer.py")
    spec = importlib.util.spec_from_file_location("derive_worked_layer", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    fx = mod.load_fixture()
    got = mod.derive(fx["inputs"])

    def flat(v):
        return [float(x) for x in np.ravel(np.array(v, dtype=object))]

    for k, v in got.items():
        assert flat(v) == flat(fx["expected"][k]), k
