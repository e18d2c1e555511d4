"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

Each ``check_*`` takes the oracle module and raises AssertionError when the
oracle disagrees with a closed form, an identity the pages state, brute
force on tiny inputs, or a hand-derived fixture under tests/golden/. They are
run on the real oracle (must pass) and on deliberately broken copies of it
(must fail) by test_oracle_pins.py, which shows that each plausible mistake
is caught by at least one pin.

Page tags: [N] papernotes.org ICLR 2026 notes on SERQ; [GDE]
gist.science/de "Technische Zusammenfassung"; [GJA] gist.science/ja "技術概要";
[RAD] AI Radio episode transcript.
"""

from __future__ import annotations

import json
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name: str) -> dict:
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def f32_ulp(x: float) -> float:
    x = abs(float(np.float32(x)))
    return float(np.spacing(np.float32(x)))


def _small_layer(seed=3, K=64, N=24, M=5, n_out=2, factor=30.0):
    rng = np.random.default_rng(seed)
    outl = rng.choice(K, n_out, replace=False)
    W = (0.02 * rng.standard_normal((K, N))).astype(np.float32)
    Xc = rng.standard_normal((64, K)).astype(np.float32)
    Xc[:, outl] *= factor
    X = rng.standard_normal((M, K)).astype(np.float32)
    X[:, outl] *= factor
    return W, np.abs(Xc).max(axis=0).astype(np.float32), X


# ---------------------------------------------------------------- packing

def check_pack(O):
    g = golden("pack_int4.json")
    for case in g["cases"]:
        codes = np.array(case["codes"], np.int8)[None, :]
        assert O.pack_int4(codes)[0].tolist() == case["bytes"], case
        assert O.unpack_int4(np.array([case["bytes"]], np.uint8))[0].tolist() == case["codes"], case
    allb = np.arange(256, dtype=np.uint8)[None, :]
    assert np.array_equal(O.pack_int4(O.unpack_int4(allb)), allb)
    # brute force: code 2t is byte t's low nibble as 4-bit two's complement
    un = O.unpack_int4(allb)[0]
    for b in range(256):
        lo, hi = b & 15, b >> 4
        assert un[2 * b] == (lo - 16 if lo >= 8 else lo)
        assert un[2 * b + 1] == (hi - 16 if hi >= 8 else hi)


# ---------------------------------------------------------------- quantizer

def check_quantizer_golden(O):
    g = golden("quantizer.json")
    for case in g["cases"]:
        q, sc = O.quantize_group(np.array(case["v"], np.float32), case["m"], case["bits"])
        assert q.tolist() == case["codes"], case
        assert float(sc) == case["scale"], case


def _nearest_even_by_search(t: float, lo: int, hi: int) -> int:
    """Pick the integer in [lo, hi] nearest to t, ties to the even one, by
    exhaustive search (an independent statement of round-half-even + clamp)."""
    best = None
    for q in range(lo, hi + 1):
        d = abs(Fraction(t) - q)
        if best is None or d < best[0] or (d == best[0] and q % 2 == 0):
            best = (d, q)
    return best[1]


def check_quantizer_bruteforce(O):
    rng = np.random.default_rng(11)
    for bits, (lo, hi) in ((4, (-8, 7)), (8, (-128, 127))):
        for trial in range(40):
            n = int(rng.integers(1, 9))
            v = (rng.standard_normal(n) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32)
            if trial % 7 == 0:  # plant exact ties on the grid
                v = (np.array(rng.integers(-2 * hi, 2 * hi + 1, n), np.float32) / 2).astype(np.float32)
            m = np.float32(np.abs(v).max())
            q, sc = O.quantize_group(v, m, bits)
            if m == 0:
                assert sc == 0 and not q.any()
                continue
            inv = np.float32(np.float32(hi) / m)
            assert sc == np.float32(m / np.float32(hi))
            for i in range(n):
                t = float(np.float32(v[i] * inv))
                assert q[i] == _nearest_even_by_search(t, lo, hi), (bits, v, i)
                # absmax scaling never reaches the clamp's negative extreme
                assert -hi <= q[i] <= hi
                # reconstruction error at most half a step (plus reciprocal slack)
                err = abs(Fraction(float(v[i])) - q[i] * Fraction(float(sc)))
                assert err <= Fraction(float(sc)) * (Fraction(1, 2) + Fraction(1, 2 ** 19)), (v[i], q[i], sc)
            # the absolute maximum maps to +-qmax
            j = int(np.argmax(np.abs(v)))
            assert abs(int(q[j])) == hi


# ---------------------------------------------------------------- smoothing

def _exact_s(a: float, w: float, alpha: float) -> Decimal:
    getcontext().prec = 60
    a = max(Decimal(float(np.float32(a))), Decimal(1e-5))
    w = max(Decimal(float(np.float32(w))), Decimal(1e-5))
    if alpha == 0.5:
        return a.sqrt() / w.sqrt()
    al = Decimal(float(np.float32(alpha)))  # the calibration takes alpha as binary32
    return (al * a.ln()).exp() / ((1 - al) * w.ln()).exp()


def check_smoothing(O):
    g = golden("smoothing.json")
    for case in g["cases"]:
        s, s_inv = O.smoothing_factors(np.array([case["a"]], np.float32), np.array([case["w"]], np.float32),
                                       case["alpha"])
        assert abs(float(s[0]) - case["s"]) <= f32_ulp(case["s"]), case
    rng = np.random.default_rng(5)
    a = (np.abs(rng.standard_normal(64)) * 10.0 ** rng.uniform(-4, 3, 64)).astype(np.float32)
    w = (np.abs(rng.standard_normal(64)) * 10.0 ** rng.uniform(-4, 1, 64)).astype(np.float32)
    for alpha in (0.5, 0.3, 0.8):
        s, s_inv = O.smoothing_factors(a, w, alpha)
        for j in range(64):
            ex = float(_exact_s(a[j], w[j], alpha))
            assert abs(float(s[j]) - ex) <= f32_ulp(ex), (alpha, a[j], w[j], s[j], ex)
            # s_inv is the correctly rounded fp32 reciprocal
            exr = Fraction(1) / Fraction(float(s[j]))
            assert abs(Fraction(float(s_inv[j])) - exr) <= Fraction(f32_ulp(float(exr))) / 2
    # SmoothQuant balance at alpha = 0.5: after flattening, channel j's
    # activation maximum a/s equals its folded weight maximum s*w.
    s, _ = O.smoothing_factors(a, w, 0.5)
    af = np.maximum(a.astype(np.float64), 1e-5)
    wf = np.maximum(w.astype(np.float64), 1e-5)
    bal = (af / s) / (s * wf)
    assert np.all(np.abs(bal - 1) < 3e-7), bal


# ---------------------------------------------------------------- permutation

def check_perm(O):
    rng = np.random.default_rng(7)
    s = rng.choice(np.array([0.5, 1.0, 2.0, 3.0, 7.0], np.float32), size=50)
    perm = O.saliency_order(s)
    assert sorted(perm.tolist()) == list(range(50))                  # bijection
    sp = s[perm]
    assert np.all(sp[:-1] >= sp[1:])                                    # descending saliency
    for i in range(49):                                                 # ties: lower index first
        if sp[i] == sp[i + 1]:
            assert perm[i] < perm[i + 1]
    # all equal -> identity
    assert O.saliency_order(np.ones(9, np.float32)).tolist() == list(range(9))


def check_fold_identity(O):
    """[RAD] and [N] 关键设计 1: (X diag(s^-1) P^-1)(P diag(s) W) = XW."""
    W, amax, X = _small_layer()
    L = O.calibrate(W, amax, r=8)
    perm, s = L["perm"], L["s"]
    # exact in fp64 when both factors are formed in fp64 from s and perm
    Xh = X.astype(np.float64)[:, perm] / s.astype(np.float64)[perm][None, :]
    Wh = s.astype(np.float64)[perm][:, None] * W.astype(np.float64)[perm, :]
    Y = X.astype(np.float64) @ W.astype(np.float64)
    assert np.linalg.norm(Xh @ Wh - Y) <= 1e-12 * np.linalg.norm(Y)
    # the oracle's own fp32 folded weight and flattened activations
    q = O.quant_act(X[:, perm], L["s_hat_inv"], 4)
    Yf = q["x_hat"].astype(np.float64) @ L["W_hat"].astype(np.float64)
    assert np.linalg.norm(Yf - Y) <= 1e-5 * np.linalg.norm(Y)
    # the folded rows are in descending-s order: row i is channel perm[i]
    assert np.array_equal(L["W_hat"][0], (s[perm[0]] * W[perm[0]]).astype(np.float32))


# ---------------------------------------------------------------- compensator

def check_compensator(O):
    """[N] 核心 idea: R = W~_s - Q(W~_s) on the r salient rows."""
    W, amax, _ = _small_layer(seed=4, K=96, N=40)
    r = 16
    L = O.calibrate(W, amax, r=r)
    Wh, Wd, R, sw = L["W_hat"][:r], L["W_deq"][:r], L["R"], L["sw"]
    assert R.shape == (r, W.shape[1])                                   # r x d
    recon = (Wd + R).astype(np.float32)
    sterbenz = (L["Wq_codes"][:r] == 0) | ((np.abs(Wh) >= np.abs(Wd) / 2) & (np.abs(Wh) <= 2 * np.abs(Wd))
                                           & (np.sign(Wh) == np.sign(Wd)))
    assert np.array_equal(recon[sterbenz], Wh[sterbenz])
    ulp = np.spacing(np.abs(Wh).astype(np.float32))
    assert np.all(np.abs(recon - Wh)[~sterbenz] <= ulp[~sterbenz])
    # R is a rounding error: at most half a quantization step per column
    assert np.all(np.abs(R.astype(np.float64)) <= sw[None, :].astype(np.float64) * (0.5 + 2 ** -19))
    # R covers exactly the r most salient rows
    assert np.array_equal(L["W_hat"][:r], Wh)
    assert L["Rq_codes"].shape == (r, W.shape[1])


# ---------------------------------------------------------------- integer GEMM

def check_int_gemm(O):
    rng = np.random.default_rng(9)
    for (M, K, N, r) in ((3, 8, 5, 2), (1, 16, 7, 0), (4, 12, 3, 12)):
        Xc = rng.integers(-8, 8, (M, K))
        Wc = rng.integers(-8, 8, (K, N))
        Rc = rng.integers(-8, 8, (r, N))
        am, ar = O.linear_int(Xc.astype(np.int8), Wc.astype(np.int8), Rc.astype(np.int8), r)
        for m in range(M):
            for n in range(N):
                tot = 0
                for k in range(K):
                    tot += int(Xc[m, k]) * int(Wc[k, n])
                assert am[m, n] == tot
                tot = 0
                for k in range(r):
                    tot += int(Xc[m, k]) * int(Rc[k, n])
                assert ar[m, n] == tot


# ---------------------------------------------------------------- dequantized output

def check_dequant_identity(O):
    """[N] 关键设计 2: X^ W^ ~ X^_q W^_q + X~_{s,q} Q(R), with X~_{s,q} the
    first r (salient) quantized activation columns. Summed term by term."""
    W, amax, X = _small_layer(seed=6, K=32, N=6, M=3)
    r = 8
    L = O.calibrate(W, amax, r=r)
    q = O.quant_act(X[:, L["perm"]], L["s_hat_inv"], 4)
    out = O.linear(q, L, out="f32")
    M, K = q["codes"].shape
    N = W.shape[1]
    for m in range(M):
        xs = float(q["sx"][m])
        for n in range(N):
            tot = 0.0
            for k in range(K):
                tot += (q["codes"][m, k] * xs) * (int(L["Wq_codes"][k, n]) * float(L["sw"][n]))
            for k in range(r):
                tot += (q["codes"][m, k] * xs) * (int(L["Rq_codes"][k, n]) * float(L["sr"][n]))
            assert abs(out["y64"][m, n] - tot) <= 1e-12 * max(1.0, abs(tot)), (m, n, out["y64"][m, n], tot)
            assert out["y"][m, n] == np.float32(out["y64"][m, n])


def check_special_cases(O):
    W, amax, X = _small_layer(seed=8, K=48, N=10, M=4)
    K, N = W.shape
    # r = 0: SmoothQuant flattening + RTN W4A4, written as fake quantization
    L = O.calibrate(W, amax, r=0)
    q = O.quant_act(X[:, L["perm"]], L["s_hat_inv"], 4)
    y0 = O.linear(q, L, out="f32")["y64"]
    xf = q["codes"].astype(np.float64) * q["sx"].astype(np.float64)[:, None]
    wf = L["Wq_codes"].astype(np.float64) * L["sw"].astype(np.float64)[None, :]
    assert np.allclose(y0, xf @ wf, rtol=1e-12, atol=1e-12)
    assert not L["Rq"].size
    # s == 1 and r = 0: plain per-token x per-channel W4A4 on the original order
    L1 = O.calibrate(W, amax, r=0, s_override=np.ones(K, np.float32))
    assert L1["perm"].tolist() == list(range(K))
    q1 = O.quant_act(X, L1["s_hat_inv"], 4)
    y1 = O.linear(q1, L1, out="f32")["y64"]
    for m in range(X.shape[0]):
        am = float(np.abs(X[m]).max())
        xc = [_nearest_even_by_search(float(np.float32(X[m, k] * np.float32(7 / np.float32(am)))), -8, 7)
              for k in range(K)]
        for n in range(N):
            wm = float(np.abs(W[:, n]).max())
            winv = np.float32(np.float32(7) / np.float32(wm))
            wc = [_nearest_even_by_search(float(np.float32(W[k, n] * winv)), -8, 7) for k in range(K)]
            ref = float(np.float32(am / np.float32(7))) * float(np.float32(np.float32(wm) / np.float32(7))) * \
                sum(a * b for a, b in zip(xc, wc))
            assert abs(y1[m, n] - ref) <= 1e-12 * max(1.0, abs(ref))
    # r = K with an unquantized R removes the weight error exactly:
    # y = deq(Xq) . W^ (fp64)
    LK = O.calibrate(W, amax, r=K, quantize_R=False)
    qK = O.quant_act(X[:, LK["perm"]], LK["s_hat_inv"], 4)
    yK = O.linear_float_residual(qK, LK)
    xd = qK["codes"].astype(np.float64) * qK["sx"].astype(np.float64)[:, None]
    exact = xd @ LK["W_hat"].astype(np.float64)
    assert np.allclose(yK, exact, rtol=1e-6, atol=1e-9)


# ---------------------------------------------------------------- fixtures

def check_worked_layer(O):
    g = golden("worked_layer_4x2.json")
    inp, ex = g["inputs"], g["expected"]
    W = np.array(inp["W"], np.float32)
    L = O.calibrate(W, np.array(inp["act_absmax"], np.float32), alpha=inp["alpha"], r=inp["r"])
    assert L["s"].tolist() == ex["s"]
    assert L["perm"].tolist() == ex["perm"]
    assert L["s_hat_inv"].tolist() == ex["s_hat_inv"]
    assert L["W_hat"].tolist() == ex["W_hat"]
    assert L["Wq_codes"].tolist() == ex["Wq_codes"]
    assert L["sw"].tolist() == ex["sw"]
    assert L["W_deq"].tolist() == ex["W_deq"]
    assert L["R"].tolist() == ex["R"]
    assert L["Rq_codes"].tolist() == ex["Rq_codes"]
    assert L["sr"].tolist() == ex["sr"]
    assert L["Wq"].tolist() == ex["Wq_packed_N_major"]
    assert L["Rq"].tolist() == ex["Rq_packed_N_major"]
    X = np.array(inp["X"], np.float32)
    q = O.quant_act(X[:, L["perm"]], L["s_hat_inv"], inp["a_bits"])
    assert q["x_hat"].tolist() == ex["x_hat"]
    assert q["codes"].tolist() == ex["Xq_codes"]
    assert q["sx"].tolist() == ex["sx"]
    o = O.linear(q, L, out="f32")
    assert o["acc_main"].tolist() == ex["acc_main"]
    assert o["acc_res"].tolist() == ex["acc_res"]
    assert o["y"].tolist() == ex["y_f32"]
    assert O.linear(q, L, out="bf16")["y"].tolist() == ex["y_bf16"]


def check_bf16(O):
    g = golden("bf16_round.json")
    for case in g["cases"]:
        assert float(O.round_f64_to_bf16(np.array([case["x"]]))[0]) == case["bf16"], case
    # brute force: the result is the nearest bf16 value, ties to an even mantissa
    rng = np.random.default_rng(2)
    xs = rng.standard_normal(300) * 10.0 ** rng.uniform(-5, 5, 300)
    got = O.round_f64_to_bf16(xs)
    for x, g_ in zip(xs, got):
        e = math.floor(math.log2(abs(x)))
        step = 2.0 ** (e - 7)
        lo = math.floor(x / step) * step
        cands = [lo, lo + step]
        d = [abs(Fraction(x) - Fraction(c)) for c in cands]
        if d[0] != d[1]:
            want = cands[0] if d[0] < d[1] else cands[1]
        else:
            want = cands[0] if int(round(cands[0] / step)) % 2 == 0 else cands[1]
        assert float(g_) == want, (x, g_, want)


def check_permute_outputs(O):
    """[N] 关键设计 3: a later layer's order pushed into this layer's output
    columns yields the permuted output with no run-time gather."""
    W, amax, X = _small_layer(seed=12, K=32, N=20, M=3)
    L = O.calibrate(W, amax, r=4)
    q = O.quant_act(X[:, L["perm"]], L["s_hat_inv"], 4)
    base = O.linear(q, L, out="f32")
    p = np.random.default_rng(1).permutation(20).astype(np.int32)
    Lp = O.permute_outputs(L, p)
    got = O.linear(q, Lp, out="f32")
    assert np.array_equal(got["acc_main"], base["acc_main"][:, p])
    assert np.array_equal(got["acc_res"], base["acc_res"][:, p])
    assert np.array_equal(got["y"], base["y"][:, p])
    assert np.array_equal(O.unpack_int4(Lp["Wq"]).T, L["Wq_codes"][:, p])


def check_rank_trend(O):
    """[N] 消融实验 / 关键发现: error falls as the rank grows and saturates.
    Statistical sanity on a synthetic outlier layer (not parity)."""
    rng = np.random.default_rng(0)
    K, N, M = 256, 128, 64
    outl = rng.choice(K, 3, replace=False)
    W = (0.02 * rng.standard_normal((K, N))).astype(np.float32)
    Xc = rng.standard_normal((128, K)).astype(np.float32)
    Xc[:, outl] *= 40
    X = rng.standard_normal((M, K)).astype(np.float32)
    X[:, outl] *= 40
    amax = np.abs(Xc).max(axis=0)
    Y = X.astype(np.float64) @ W.astype(np.float64)
    errs = []
    for r in (0, 16, 64, 128):
        L = O.calibrate(W, amax, r=r)
        q = O.quant_act(X[:, L["perm"]], L["s_hat_inv"], 4)
        errs.append(np.linalg.norm(O.linear(q, L, out="f32")["y64"] - Y))
    assert errs[0] > errs[1] > errs[2] > errs[3], errs
    # flattening helps against channel outliers compared with plain W4A4
    L1 = O.calibrate(W, amax, r=0, s_override=np.ones(K, np.float32))
    q1 = O.quant_act(X, L1["s_hat_inv"], 4)
    assert np.linalg.norm(O.linear(q1, L1, out="f32")["y64"] - Y) > errs[0]


# ------------------------------------------------- MLP activation (silu * up)
# Closed forms only: the oracle's fp32 recipe for e^x and silu(g) * u against
# the fp64 definitions, a special value, the clamp, an odd-symmetry identity
# and the composition with the per-token quantizer the step is defined as.

def _f32_nearest(q: Fraction) -> np.float32:
    """The binary32 value nearest to the rational q (ties to even), for q
    zero or in the normal range: exact integer arithmetic throughout."""
    if q == 0:
        return np.float32(0.0)
    neg, q = q < 0, abs(q)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    elif Fraction(2) ** (e + 1) <= q:
        e += 1
    m = q / Fraction(2) ** (e - 23)              # in [2^23, 2^24)
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = math.ldexp(float(fl), e - 23)            # exact: fl has at most 25 bits
    return np.float32(-v if neg else v)


def check_fma32(O):
    """fma32 against exact rational arithmetic rounded once, including the
    double-rounding cases a plain binary64 sum gets wrong."""
    rng = np.random.default_rng(17)
    n = 3000
    a = (rng.standard_normal(n) * np.exp2(rng.integers(-20, 20, n))).astype(np.float32)
    b = (rng.standard_normal(n) * np.exp2(rng.integers(-20, 20, n))).astype(np.float32)
    c = (rng.standard_normal(n) * np.exp2(rng.integers(-40, 40, n))).astype(np.float32)
    c[: n // 3] = -(a[: n // 3] * b[: n // 3]).astype(np.float32)            # cancellation
    c[n // 3: n // 2] = np.nextafter(c[: n // 6], np.float32(np.inf))
    # a * b exactly halfway between two binary32 values, then nudged by a c
    # far below the binary64 spacing: only a single rounding gets these right
    h = np.float32(1.0 + 2.0 ** -12)
    hard_a = np.array([h, h, h, -h, np.float32(3.0 * (1.0 + 2.0 ** -12))], np.float32)
    hard_b = np.array([h, h, h, h, h], np.float32)
    hard_c = np.array([0.0, 2.0 ** -60, -2.0 ** -60, 2.0 ** -70, -2.0 ** -58], np.float32)
    A, B, C = (np.concatenate([x, y]) for x, y in ((a, hard_a), (b, hard_b), (c, hard_c)))
    got = O.fma32(A, B, C)
    for i in range(A.size):
        want = _f32_nearest(Fraction(float(A[i])) * Fraction(float(B[i])) + Fraction(float(C[i])))
        if abs(float(want)) >= 2.0 ** -126 or want == 0:
            assert got[i].view(np.uint32) == want.view(np.uint32), (i, A[i], B[i], C[i], got[i], want)
    # the tie itself rounds to even, and the nudges decide it
    assert O.fma32(h, h, np.float32(0.0)) == np.float32(1.0 + 2.0 ** -11)
    assert O.fma32(h, h, np.float32(2.0 ** -60)) == np.float32(1.0 + 2.0 ** -11 + 2.0 ** -23)
    # no addend: the binary32 product; unit factor: the binary32 sum
    assert np.array_equal(O.fma32(a, b, np.zeros_like(a)), (a * b).astype(np.float32))
    assert np.array_equal(O.fma32(a, np.ones_like(a), c), (a + c).astype(np.float32))


def check_exp32(O):
    x = np.linspace(-80.0, 80.0, 400001).astype(np.float32)
    truth = np.exp(x.astype(np.float64))
    got = O.exp32(x).astype(np.float64)
    ulp = np.spacing(truth.astype(np.float32)).astype(np.float64)
    assert (np.abs(got - truth) <= 1.0 * ulp).all(), float((np.abs(got - truth) / ulp).max())
    assert O.exp32(np.float32(0.0)) == np.float32(1.0)
    assert O.exp32(np.float32(500.0)) == O.exp32(np.float32(80.0))
    assert O.exp32(np.float32(-500.0)) == O.exp32(np.float32(-80.0))


def check_silu_mul(O):
    rng = np.random.default_rng(11)
    g = np.concatenate([rng.standard_normal(20000) * 4.0, np.linspace(-30.0, 30.0, 6001)]).astype(np.float32)
    u = (rng.standard_normal(g.size) * 2.0).astype(np.float32)
    h = O.silu_mul(g, u).astype(np.float64)
    g64, u64 = g.astype(np.float64), u.astype(np.float64)
    truth = g64 * u64 / (1.0 + np.exp(-g64))
    tol = 4.0 * np.spacing(np.abs(truth).astype(np.float32)).astype(np.float64) + 1e-30
    assert (np.abs(h - truth) <= tol).all(), float((np.abs(h - truth) / tol).max())
    # silu(0) = 0; for g >= 20, e^-g < 2^-25 so 1 + e rounds to 1: h = fl32(g u)
    assert (O.silu_mul(np.zeros(5, np.float32), u[:5]) == 0).all()
    big = np.float32([20.0, 33.5, 79.0])
    assert np.array_equal(O.silu_mul(big, u[:3]), (big * u[:3]).astype(np.float32))
    # odd symmetry: silu(g) - silu(-g) = g (sigma(g) + sigma(-g) = 1)
    gs = np.linspace(-12.0, 12.0, 2001).astype(np.float32)
    one = np.ones_like(gs)
    d = O.silu_mul(gs, one).astype(np.float64) - O.silu_mul(-gs, one).astype(np.float64)
    assert np.allclose(d, gs.astype(np.float64), rtol=0, atol=8 * np.spacing(np.float32(12.0)))
    # the fused step is the quantizer applied to silu(G) * U (same codes and scales)
    G = (rng.standard_normal((5, 96)) * 3).astype(np.float32)
    U = rng.standard_normal((5, 96)).astype(np.float32)
    sinv = (rng.random(96) + 0.5).astype(np.float32)
    for bits in (4, 8):
        a = O.silu_mul_quant_act(G, U, sinv, bits)
        hh = (G.astype(np.float64) * U / (1.0 + np.exp(-G.astype(np.float64)))).astype(np.float32)
        b = O.quant_act(hh, sinv, bits)
        # codes agree except where the fp64 and fp32-recipe values straddle a rounding edge
        assert (np.abs(a["codes"].astype(int) - b["codes"].astype(int)) <= 1).all()
        assert np.mean(a["codes"] == b["codes"]) > 0.99
        assert np.allclose(a["sx"], b["sx"], rtol=1e-6, atol=0)


# ---------------------------------------------------------------- sampled columns

def check_calibrate_columns(O):
    """calibrate_columns (the expected values of full-size checks on sampled
    output columns) equals calibrate restricted to those columns, bit for
    bit. [N] 关键设计 1: s is per input channel, over the whole weight row,
    so it (and P) must not depend on which columns are sampled; [N] 关键设计 2
    and [GDE] 3: the weight and R quantizers are per output column, so a
    column's codes and scales depend only on that column once s, P are fixed."""
    rng = np.random.default_rng(21)
    cases = []
    # ties and dead channels: equal s on several channels, an all-zero
    # weight row and a zero activation maximum
    K, N = 32, 40
    W = (0.02 * rng.standard_normal((K, N))).astype(np.float32)
    a = (rng.random(K) * 3 + 0.5).astype(np.float32)
    W[5] = W[9]
    a[5] = a[9]
    W[12] = W[20]
    a[12] = a[20]
    W[17] = 0.0
    a[3] = 0.0
    cases.append((W, a, 8, 0.5))
    W2, a2, _ = _small_layer(seed=7, K=48, N=36)
    cases.append((W2, a2, 0, 0.5))           # r = 0
    cases.append((W2, a2, 48, 0.5))          # r = K
    cases.append((W2, a2, 12, 0.3))          # another alpha
    for W, a, r, alpha in cases:
        full = O.calibrate(W, a, alpha=alpha, r=r)
        N = W.shape[1]
        for cols in (np.array([0, N - 1]), np.sort(rng.choice(N, N // 3, replace=False)), np.arange(N)):
            part = O.calibrate_columns(W, a, cols, alpha=alpha, r=r)
            assert np.array_equal(part["perm"], full["perm"])
            assert np.array_equal(part["s_hat_inv"].view(np.uint32), full["s_hat_inv"].view(np.uint32))
            assert np.array_equal(part["Wq_codes"], full["Wq_codes"][:, cols])
            assert np.array_equal(part["sw"].view(np.uint32), full["sw"][cols].view(np.uint32))
            assert np.array_equal(part["Wq"], full["Wq"][cols])
            assert np.array_equal(part["Rq_codes"], full["Rq_codes"][:, cols])
            assert np.array_equal(part["sr"].view(np.uint32), full["sr"][cols].view(np.uint32))
            assert np.array_equal(part["Rq"], full["Rq"][cols])


def check_exp_split_constant(O):
    """The exponential's reduction constants: c_hi = 22713 * 2^-15 (15
    significant bits), c_hi + c_lo within 2^-40 of ln 2, and n * c_hi exact
    in binary32 for every n the clamp allows (|n| <= 116)."""
    hi = Fraction(float(O.LN2_HI_F32))
    assert hi == Fraction(22713, 2 ** 15)
    assert 22713 % 2 == 1 and 2 ** 14 <= 22713 < 2 ** 15
    lo = Fraction(float(O.LN2_LO_F32))
    assert abs(float(hi + lo) - math.log(2.0)) < 2.0 ** -40
    nmax = int(np.rint(np.float32(O.EXP_ARG_CLAMP) * O.LOG2E_F32))
    assert nmax <= 116
    for n in range(-nmax, nmax + 1):
        assert Fraction(float(np.float32(n) * O.LN2_HI_F32)) == n * hi


# ---------------------------------------------------------------- GPTQ

def _derive_gptq():
    import importlib.util
    spec = importlib.util.spec_from_file_location("derive_gptq", os.path.join(GOLDEN, "derive_gptq.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _gptq_layer(seed, K, N, T, corr=0.4):
    rng = np.random.default_rng(seed)
    A = (rng.standard_normal((K, K)) * corr + np.eye(K)).astype(np.float32)
    Xc = (rng.standard_normal((T, K)).astype(np.float32) @ A).astype(np.float32)
    Xc[:, rng.choice(K, 2, replace=False)] *= np.float32(20.0)
    W = (0.02 * rng.standard_normal((K, N))).astype(np.float32)
    return W, np.abs(Xc).max(axis=0).astype(np.float32), Xc


def check_gptq_exact(O):
    """GPTQ codes against the exact-rational optimal-brain-surgeon derivation
    (tests/golden/derive_gptq.py: trailing-block inverses by Gauss-Jordan, no
    Cholesky factor): the worked 4 x 2 fixture (r = 0, r = 2, no damping,
    all rows salient) and random layers, through calibrate_gptq too (the
    inputs flattened and permuted as the layer sees them). [GDE] 3: SERQ
    works with GPTQ; GPTQ (Frantar et al., ICLR 2023) is the OBS update."""
    D = _derive_gptq()
    fx = golden("gptq_4x2.json")
    Wh = np.array(fx["inputs"]["W_hat"], np.float32)
    Xh = np.array(fx["inputs"]["X_hat"], np.float32)
    for case in fx["inputs"]["cases"]:
        U = O.gptq_inverse_factor(O.gptq_hessian(Xh, case["damp"]))
        got = O.gptq_quantize(Wh, U, case["r"])
        assert got.tolist() == fx["expected"][case["name"]], case["name"]
    for seed in range(6):
        K, N, T = 6, 3, 9
        W, a, Xc = _gptq_layer(100 + seed, K, N, T)
        for r in (0, 2):
            damp = (0.01, 0.3)[seed % 2]
            G = O.calibrate_gptq(W, a, Xc, r=r, damp=damp)
            Xh = (Xc[:, G["perm"]] * G["s_hat_inv"][None, :]).astype(np.float32)
            want = D.gptq_codes(G["W_hat"].tolist(), Xh.tolist(), r, Fraction(float(np.float32(damp))))
            assert G["Wq_codes"].tolist() == want, (seed, r)


def check_gptq_special_cases(O):
    """Where GPTQ has nothing to move, it is RTN bit for bit: a diagonal
    Hessian (orthogonal calibration inputs: no row's error can be absorbed by
    another), all-zero inputs (the identity), and r = K (every row salient).
    The salient rows, R, Q(R) and the permutation are RTN's at any r. The
    inverse factor satisfies U^T U H = I and is upper triangular."""
    W, a, Xc = _gptq_layer(7, 24, 10, 64)
    for r in (0, 8):
        rtn = O.calibrate(W, a, r=r)
        diag_x = np.diag(np.linspace(0.5, 3.0, 24)).astype(np.float32)        # orthogonal columns
        for X in (diag_x, np.zeros((5, 24), np.float32)):
            g = O.calibrate_gptq(W, a, X, r=r)
            assert np.array_equal(g["Wq_codes"], rtn["Wq_codes"])
            assert np.array_equal(g["Wq"], rtn["Wq"])
        g = O.calibrate_gptq(W, a, Xc, r=r)
        assert not np.array_equal(g["Wq_codes"], rtn["Wq_codes"])      # correlated inputs: GPTQ moves codes
        assert np.array_equal(g["Wq_codes"][:r], rtn["Wq_codes"][:r])
        for k in ("perm", "s_hat_inv", "sw", "Rq", "sr", "Rq_codes"):
            assert np.array_equal(g[k], rtn[k]), k
        U, H = g["U"], g["H"]
        assert np.allclose(U.T @ U @ H, np.eye(24), atol=1e-9)
        assert np.array_equal(U, np.triu(U)) and (np.diag(U) > 0).all()
    g = O.calibrate_gptq(W, a, Xc, r=24)
    assert np.array_equal(g["Wq_codes"], O.calibrate(W, a, r=24)["Wq_codes"])


def check_gptq_reduces_error(O):
    """GPTQ's purpose: a smaller output error on the calibration inputs than
    round to nearest, with and without the compensator (the pages' accuracy
    rows use SERQ(GPTQ); [N] 实验关键数据). Statistical, fixed seeds."""
    for seed in (1, 2):
        W, a, Xc = _gptq_layer(seed, 96, 48, 256)
        for r in (0, 16):
            g = O.calibrate_gptq(W, a, Xc, r=r)
            t = O.calibrate(W, a, r=r)
            Xh = g["X_hat_cal"]
            eg = O.weighted_error(Xh, g["W_hat"], g["W_deq"], O.dequantize_columns(g["Rq_codes"], g["sr"]), r)
            et = O.weighted_error(Xh, t["W_hat"], t["W_deq"], O.dequantize_columns(t["Rq_codes"], t["sr"]), r)
            assert eg < 0.9 * et, (seed, r, eg, et)


# ---------------------------------------------------------------- MXFP4

def _e2m1_spec_value(c: int) -> float:
    """E2M1 by its bit fields: sign bit 3, exponent bits 2-1 (bias 1),
    mantissa bit 0; exponent 0 is subnormal (0.m x 2^0)."""
    sgn = -1.0 if c & 8 else 1.0
    e, m = (c >> 1) & 3, c & 1
    mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return sgn * mag


def check_mx_quantizer(O):
    """The MXFP4 quantizer (OCP Microscaling Formats (MX) v1.0; [GDE] 3:
    SERQ works with MXFP4): the hand-worked blocks of mxfp4_blocks.json, the
    E2M1 code table from its bit fields, nearest-value rounding with ties to
    the even mantissa by exhaustive search, saturation at 6, the shared
    exponent's closed form, and lossless blocks."""
    fx = golden("mxfp4_blocks.json")
    for case in fx["cases"]:
        codes, e = O.mx_quantize_rows(np.array(case["v"], np.float32)[None, :])
        assert codes[0].tolist() == case["codes"] and int(e[0, 0]) == case["e"], case["e"]
        assert O.mx_dequantize_rows(codes, e)[0].tolist() == [float(np.float32(v)) for v in case["values"]]
    for c in range(16):
        assert float(O.e2m1_value(np.array([c]))[0]) == _e2m1_spec_value(c) + 0.0
    grid = sorted({abs(_e2m1_spec_value(c)) for c in range(8)})
    mids = [(a + b) / 2 for a, b in zip(grid, grid[1:])]
    ts = np.array(sorted(set(np.linspace(-9, 9, 7201).tolist() + mids + [-m for m in mids]
                              + [m + d for m in mids for d in (1e-9, -1e-9)])))
    got = O.e2m1_value(O.e2m1_round(ts))
    for t, g in zip(ts, got):
        a = min(abs(t), 6.0)
        dist = [abs(a - v) for v in grid]
        best = min(dist)
        near = [v for v, d in zip(grid, dist) if d == best]
        if len(near) == 2:      # a tie: the value whose mantissa bit is 0
            want = [v for v in near if [c for c in range(8) if _e2m1_spec_value(c) == v][0] % 2 == 0][0]
        else:
            want = near[0]
        assert abs(g) == want and (g == 0 or (g < 0) == (t < 0)), (t, g, want)
    rng = np.random.default_rng(4)
    amax = (np.exp2(rng.uniform(-120, 120, 5000)) * rng.uniform(1, 2, 5000)).astype(np.float32)
    e = O.mx_block_exponent(amax).astype(np.float64)
    a = amax.astype(np.float64)
    assert ((np.exp2(e + 2) <= a) & (a < np.exp2(e + 3))).all()
    assert O.mx_block_exponent(np.float32([0.0, 1e-42]))[0] == -127
    # lossless: blocks of E2M1 values times 2^e whose largest magnitude is 4 or 6
    for trial in range(20):
        codes = rng.integers(0, 16, 32)
        codes[rng.integers(0, 32)] = rng.choice([6, 7, 14, 15])
        ee = int(rng.integers(-100, 100))
        v = (O.e2m1_value(codes) * 2.0 ** ee).astype(np.float32)
        c2, e2 = O.mx_quantize_rows(v[None, :])
        assert np.array_equal(O.mx_dequantize_rows(c2, e2)[0], v)


def check_mx_layer(O):
    """The MXFP4 layer: the block dot products against brute force in exact
    rationals; R = fl32(W^ - deq Q(W^)) on the salient rows (the definition,
    [N] 核心 idea) with the exact reconstruction on the Sterbenz set; blocks
    along K per output column (scaling one column of W by 2^j moves only its
    exponents); the residual on the first r channels' blocks."""
    rng = np.random.default_rng(8)
    K, N, M, r = 96, 5, 3, 32
    W = (0.05 * rng.standard_normal((K, N))).astype(np.float32)
    a = (rng.random(K) * 4 + 0.1).astype(np.float32)
    L = O.calibrate_mx(W, a, r=r)
    X = rng.standard_normal((M, K)).astype(np.float32) * 3
    q = O.quant_act_mx(X[:, L["perm"]], L["s_hat_inv"])
    out = O.linear_mx(q, L)
    xv = O.e2m1_value(q["codes"])
    wv = O.e2m1_value(L["Wq_codes"])
    rv = O.e2m1_value(L["Rq_codes"])
    for m in range(M):
        for n in range(N):
            main = sum(Fraction(float(xv[m, k])) * Fraction(float(wv[n, k]))
                       * Fraction(2) ** int(q["e"][m, k // 32] + L["We"][n, k // 32]) for k in range(K))
            res = sum(Fraction(float(xv[m, k])) * Fraction(float(rv[n, k]))
                      * Fraction(2) ** int(q["e"][m, k // 32] + L["Re"][n, k // 32]) for k in range(r))
            assert Fraction(float(out["acc_main"][m, n])) == main and Fraction(float(out["acc_res"][m, n])) == res
    Wd = L["W_deq"]
    assert np.array_equal(L["R"], (L["W_hat"][:r] - Wd[:r]).astype(np.float32))
    rec = (Wd[:r] + L["R"]).astype(np.float32)
    ster = (Wd[:r] == 0) | ((np.abs(Wd[:r]) / 2 <= np.abs(L["W_hat"][:r])) & (np.abs(L["W_hat"][:r]) <= 2 * np.abs(Wd[:r])))
    assert np.array_equal(rec[ster], L["W_hat"][:r][ster])
    assert np.array_equal(L["Wq"], O.pack_fp4(L["Wq_codes"])) and L["Wq"].shape == (N, K // 2)
    assert L["Wsc"].shape == (N, K // 32) and L["Rsc"].shape == (N, r // 32)
    # scaling W and the activation maxima by 2^6 leaves s and the codes, and
    # adds 6 to every exponent
    L2 = O.calibrate_mx((W * np.float32(64.0)).astype(np.float32), a * np.float32(64.0), r=r)
    assert np.array_equal(L2["perm"], L["perm"]) and np.array_equal(L2["Wq_codes"], L["Wq_codes"])
    assert (L2["We"] - L["We"] == 6).all()
    # blocks run along K within one output column: growing one element of W^
    # changes the codes and exponent of its own block only
    Wh = L["W_hat"].copy()
    Wh[40, 3] = np.float32(50.0) * np.abs(Wh[:, 3]).max()
    c2, e2 = O.mx_quantize_rows(Wh.T)
    diff = np.argwhere(c2 != L["Wq_codes"])
    assert len(diff) and set(map(tuple, (diff // [1, 32]).tolist())) == {(3, 1)}
    assert np.argwhere(e2 != L["We"]).tolist() == [[3, 1]]


ALL_CHECKS = [check_pack, check_quantizer_golden, check_quantizer_bruteforce, check_smoothing,
              check_perm, check_fold_identity, check_compensator, check_int_gemm,
              check_dequant_identity, check_special_cases, check_worked_layer, check_bf16,
              check_permute_outputs, check_rank_trend, check_fma32, check_exp32, check_silu_mul,
              check_calibrate_columns, check_exp_split_constant, check_gptq_exact,
              check_gptq_special_cases, check_gptq_reduces_error, check_mx_quantizer, check_mx_layer]
