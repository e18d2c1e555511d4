"""CPU oracle for the SERQ quantized linear layer -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may
import this module. The HIP library never calls it and shares no code with
it: this is a plain, slow, step-by-step restatement of what the pages define,
used to check the GPU path element by element.

Sources (each cited below by its tag and a section of that page):
  [N]   "SERQ: Saliency-Aware Low-Rank Error Reconstruction for LLM
        Quantization", papernotes.org notes for ICLR 2026
        (sections 核心 idea, 方法详解 / 整体框架, 关键设计 1-3, 消融实验)
  [GDE] gist.science/de/paper/2603.08185, "Technische Zusammenfassung"
        (sections 2.A-2.C, 3, 4)
  [GJA] gist.science/ja/paper/2603.08185, "技術概要"
        (section 2 and its "計算フローの革新" paragraph)
  [RAD] AI Radio episode "SERQ: Saliency-Aware Low-Rank Error
        Reconstruction for LLM Quantization" (the paper-summary dialogue)

Notation (as on the pages): X is M x K (tokens x input channels), W is K x N
with Y = X W; s is the per-channel smoothing factor, P the saliency
permutation, X~ = X diag(s^-1), W~ = diag(s) W, W^ = P W~ = [W~_s; W~_r],
X^ = X~ P^-1 = [X~_s X~_r], r the rank (number of salient rows), R the r x N
compensator.

Arithmetic rules of this oracle (the pages fix none of them; these are the
readings the library must reproduce bit for bit):
  * every fp32 step below is one IEEE binary32 operation, round to nearest
    even, no fused multiply-add except the exactly rounded ones written out
    as fma32 (the MLP activation's exponential);
  * ``rne`` is round-half-to-even;
  * bf16 inputs widen exactly to fp32;
  * the final output y is evaluated in fp64 from exact integer accumulators
    and rounded once to fp32 or bf16.

Pinning status: every function here is pinned by tests/test_oracle_pins.py
(closed forms, identities the pages state, brute force on tiny inputs and
hand-derived fixtures under tests/golden/). Three conventions are fixed by
this contract rather than by the pages -- the smoothing-factor formula and its
floor, the tie order of the saliency sort, and the quantizer's reciprocal
rounding -- and are "parity unpinned" as far as the pages go: only their
internal consequences (balance, sortedness, error bounds) are pinned.
"""

from __future__ import annotations

import math

import numpy as np

F32 = np.float32
I4_MIN, I4_MAX = -8, 7
I8_MIN, I8_MAX = -128, 127
S_FLOOR = 1e-5          # floor on both channel maxima before forming s
ALPHA_DEFAULT = 0.5


def qrange(bits: int) -> tuple[int, int]:
    if bits == 4:
        return I4_MIN, I4_MAX
    if bits == 8:
        return I8_MIN, I8_MAX
    raise ValueError("bits must be 4 or 8")


# ---------------------------------------------------------------------------
# Step A -- static activation flattening.
# [N] 关键设计 1: per-channel static scaling in the SmoothQuant style,
# Y = XW = (X diag(s^-1))(diag(s) W), computed once at calibration and merged
# offline. [GDE] 2.A: the factors come from calibration and are folded into
# the weights. The pages do not print a formula for s; SmoothQuant's own
# per-channel rule s_j = max|X_j|^a / max|W_j|^(1-a) is taken, with a = 0.5 and
# a floor of 1e-5 on both maxima so that a dead channel gives a finite s.
# ---------------------------------------------------------------------------

def smoothing_factors(act_absmax: np.ndarray, w_rowmax: np.ndarray,
                      alpha: float = ALPHA_DEFAULT) -> tuple[np.ndarray, np.ndarray]:
    """Return (s, s_inv), both float32 vectors of length K.

    s_j is formed in fp64 and rounded once to fp32; for alpha = 0.5 this is
    fl32(sqrt(a_j) / sqrt(w_j)). s_inv_j = fl32(1 / s_j) (one fp32 divide).
    """
    # alpha is a binary32 parameter of the calibration call; use that value
    alpha = float(np.float32(alpha))
    a = np.maximum(np.asarray(act_absmax, dtype=np.float32).astype(np.float64), S_FLOOR)
    w = np.maximum(np.asarray(w_rowmax, dtype=np.float32).astype(np.float64), S_FLOOR)
    if alpha == 0.5:
        s64 = np.sqrt(a) / np.sqrt(w)
    else:
        # libm pow element by element (no vectorised approximation)
        s64 = np.array([math.pow(ai, alpha) / math.pow(wi, 1.0 - alpha) for ai, wi in zip(a, w)],
                       dtype=np.float64)
    s = s64.astype(np.float32)
    s_inv = (np.float32(1.0) / s).astype(np.float32)
    return s, s_inv


# ---------------------------------------------------------------------------
# Step B -- saliency ranking and the permutation P.
# [N] 关键设计 2: after flattening, activation outliers sit in the matching
# weight rows; assuming roughly normal original weights, salient rows of the
# folded weight are identified directly by their scale, and rows are
# permuted in descending saliency, W^ = P diag(s) W = [W~_s; W~_r].
# [GDE] 2.B: identification is based on the activations' scaling factors.
# Reading: saliency of row j is s_j; descending order; equal s keep the lower
# original index first (the pages leave ties open; several orders are equally
# valid, this one is fixed so that results are reproducible).
# ---------------------------------------------------------------------------

def saliency_order(s: np.ndarray) -> np.ndarray:
    """perm[i] = original channel placed at position i (int32)."""
    s = np.asarray(s, dtype=np.float32)
    return np.argsort(-s.astype(np.float64), kind="stable").astype(np.int32)


def fold_and_permute(W: np.ndarray, s: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """W^[i, n] = fl32(s[perm[i]] * W[perm[i], n])  (K x N float32)."""
    W = np.asarray(W, dtype=np.float32)
    return (s[perm][:, None].astype(np.float32) * W[perm, :]).astype(np.float32)


# ---------------------------------------------------------------------------
# The symmetric round-to-nearest quantizer used for weights, the compensator
# and activations. [GDE] 3: the method works with RTN (and GPTQ) and with the
# INT4 format; the integer range is [-8, 7] for 4-bit and [-128, 127] for
# 8-bit. Reading: scale = fl32(m / qmax) with m the group's absolute maximum,
# codes = clamp(rne(fl32(v * fl32(qmax / m)))). A group whose reciprocal
# fl32(qmax / m) overflows (an all-zero group in particular) gets scale 0
# and all-zero codes.
# ---------------------------------------------------------------------------

def quantize_group(v: np.ndarray, m, bits: int) -> tuple[np.ndarray, np.float32]:
    """Quantize one group ``v`` (any shape) with absolute maximum ``m``."""
    lo, hi = qrange(bits)
    v = np.asarray(v, dtype=np.float32)
    m = np.float32(m)
    with np.errstate(divide="ignore", over="ignore"):
        inv = np.float32(np.float32(hi) / m)
    if not np.isfinite(inv):
        return np.zeros(v.shape, np.int8), np.float32(0.0)
    scale = np.float32(m / np.float32(hi))
    t = (v * inv).astype(np.float32)
    q = np.clip(np.rint(t), lo, hi).astype(np.int8)
    return q, scale


def quantize_columns(A: np.ndarray, bits: int) -> tuple[np.ndarray, np.ndarray]:
    """Per-column quantization of a (rows x N) float32 matrix: one scale per
    column over all of its rows. Returns (codes int8 rows x N, scales N)."""
    A = np.asarray(A, dtype=np.float32)
    codes = np.zeros(A.shape, np.int8)
    scales = np.zeros(A.shape[1], np.float32)
    if A.shape[0] == 0:
        return codes, scales
    for n in range(A.shape[1]):
        col = A[:, n]
        codes[:, n], scales[n] = quantize_group(col, np.abs(col).max(), bits)
    return codes, scales


def quantize_rows(A: np.ndarray, bits: int) -> tuple[np.ndarray, np.ndarray]:
    """Per-row quantization (one scale per row, e.g. per token)."""
    A = np.asarray(A, dtype=np.float32)
    codes = np.zeros(A.shape, np.int8)
    scales = np.zeros(A.shape[0], np.float32)
    if A.shape[1] == 0:
        return codes, scales
    for i in range(A.shape[0]):
        row = A[i]
        codes[i], scales[i] = quantize_group(row, np.abs(row).max(), bits)
    return codes, scales


def dequantize_columns(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """fl32(code * scale) per element, scale per column."""
    return (codes.astype(np.float32) * scales[None, :].astype(np.float32)).astype(np.float32)


# ---------------------------------------------------------------------------
# Step C -- the single compensator R on the r salient rows.
# [N] 核心 idea: R = W~_s - Q(W~_s), built only for the r chosen rows;
# [RAD]: R is r by d and corrects the quantization error of the r salient
# rows; [N] 关键设计 2: R itself is quantized, so the whole path stays in low
# precision. Reading: Q(W~_s) is the main path's own dequantized weight for
# those rows (per-column scales over all K rows), so that before R is
# quantized X~_s (Q(W~_s) + R) = X~_s W~_s exactly in real arithmetic. R is
# quantized to int4 with one scale per output column over its r rows.
# ---------------------------------------------------------------------------

def compensator(W_hat: np.ndarray, W_deq: np.ndarray, r: int) -> np.ndarray:
    """R[i, n] = fl32(W^[i, n] - Q(W^)[i, n]) for i < r (r x N float32)."""
    return (W_hat[:r].astype(np.float32) - W_deq[:r].astype(np.float32)).astype(np.float32)


# ---------------------------------------------------------------------------
# Canonical 4-bit packing: byte t of a row holds code 2t in bits 0-3 and code
# 2t+1 in bits 4-7, each as 4-bit two's complement.
# ---------------------------------------------------------------------------

def pack_int4(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64)
    if c.shape[-1] % 2:
        raise ValueError("packing needs an even number of codes per row")
    lo = c[..., 0::2] & 0xF
    hi = c[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.int64)
    lo = p & 0xF
    hi = (p >> 4) & 0xF
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


# ---------------------------------------------------------------------------
# Offline calibration, end to end ([N] 整体框架: calibration fixes the scale
# factors, the salient rows and the permutation order).
# ---------------------------------------------------------------------------

def calibrate(W: np.ndarray, act_absmax: np.ndarray, *, alpha: float = ALPHA_DEFAULT,
              r: int, quantize_R: bool = True, s_override: np.ndarray | None = None) -> dict:
    """Calibrate one layer. ``W`` is K x N float32 (bf16 values widen exactly).

    Returns a dict with the library's outputs in their canonical layouts
    (``perm``, ``s_hat_inv``, ``Wq`` N x K/2 bytes, ``sw``, ``Rq`` N x r/2
    bytes, ``sr``) plus the intermediate values for tests (``s``, ``s_inv``,
    ``W_hat``, ``Wq_codes`` K x N, ``W_deq``, ``R``, ``Rq_codes`` r x N).

    Test hooks: ``s_override`` replaces s (e.g. all ones), ``quantize_R=False``
    keeps R in float (the ``R_float`` entry) for the exact-reconstruction
    special case.
    """
    W = np.asarray(W, dtype=np.float32)
    K, N = W.shape
    if K % 2 or r % 2 or not (0 <= r <= K):
        raise ValueError("need even K, even r with 0 <= r <= K")
    if s_override is None:
        s, s_inv = smoothing_factors(act_absmax, np.abs(W).max(axis=1), alpha)
    else:
        s = np.asarray(s_override, dtype=np.float32)
        s_inv = (np.float32(1.0) / s).astype(np.float32)
    perm = saliency_order(s)
    s_hat_inv = s_inv[perm].astype(np.float32)
    W_hat = fold_and_permute(W, s, perm)
    Wq_codes, sw = quantize_columns(W_hat, 4)
    W_deq = dequantize_columns(Wq_codes, sw)
    R = compensator(W_hat, W_deq, r)
    Rq_codes, sr = quantize_columns(R, 4)
    out = dict(K=K, N=N, r=r, s=s, s_inv=s_inv, perm=perm, s_hat_inv=s_hat_inv,
               W_hat=W_hat, Wq_codes=Wq_codes, sw=sw, W_deq=W_deq, R=R,
               Rq_codes=Rq_codes, sr=sr,
               Wq=pack_int4(Wq_codes.T), Rq=pack_int4(Rq_codes.T) if r else np.zeros((N, 0), np.uint8))
    if not quantize_R:
        out["R_float"] = R
    return out


def calibrate_columns(W: np.ndarray, act_absmax: np.ndarray, cols: np.ndarray, *,
                      alpha: float = ALPHA_DEFAULT, r: int) -> dict:
    """The same calibration, evaluated only for the output columns ``cols``.

    Per-column quantization makes every output column independent once s and
    P are known; s needs each input channel's maximum over all of W, which is
    one pass. Used to check full-size layers on sampled columns.
    """
    W = np.asarray(W, dtype=np.float32)
    s, s_inv = smoothing_factors(act_absmax, np.abs(W).max(axis=1), alpha)
    perm = saliency_order(s)
    Wc = W[:, cols]
    W_hat = fold_and_permute(Wc, s, perm)
    Wq_codes, sw = quantize_columns(W_hat, 4)
    W_deq = dequantize_columns(Wq_codes, sw)
    R = compensator(W_hat, W_deq, r)
    Rq_codes, sr = quantize_columns(R, 4)
    return dict(s=s, s_inv=s_inv, perm=perm, s_hat_inv=s_inv[perm], cols=np.asarray(cols),
                Wq_codes=Wq_codes, sw=sw, Rq_codes=Rq_codes, sr=sr,
                Wq=pack_int4(Wq_codes.T), Rq=pack_int4(Rq_codes.T) if r else np.zeros((len(cols), 0), np.uint8))


# ---------------------------------------------------------------------------
# GPTQ as the weight quantizer: SERQ(GPTQ).
# [GDE] 3 (Wichtige Beiträge): the method works with round-to-nearest and
# with GPTQ weight quantization; [N] 实验关键数据: the accuracy rows are
# SERQ(GPTQ). GPTQ (Frantar, Ashkboos, Hoefler and Alistarh, "GPTQ: Accurate
# Post-Training Quantization for Generative Pre-trained Transformers", ICLR
# 2023) quantizes the input rows of W one at a time in a fixed order and,
# after each row, moves that row's quantization error onto the rows not yet
# quantized so as to minimise the layer's squared output error on
# calibration inputs; the weights of the update come from the inverse of
# H = X^T X (upper Cholesky factor U of H^-1: row i's error e is divided by
# U[i, i] and subtracted, times U[i, j], from every later row j).
#
# Readings (the pages do not spell the combination out):
#   * the order is the saliency order P, and H is formed from the inputs the
#     layer sees, X^_cal = fl32(X_cal[:, perm] * s_hat_inv) (flattened,
#     permuted calibration activations): H[i, j] = sum_t x^[t,i] x^[t,j] in
#     fp64, summed over t in order (the products are exact in fp64);
#   * dampening as in GPTQ: lambda = damp * mean(diag H) added to the
#     diagonal (damp = 0.01); an all-zero H becomes the identity;
#   * the quantization grid is RTN's: one scale per output column from the
#     column maximum of W^ before any update, codes clamped to [-8, 7]; a
#     row's codes quantize its updated values rounded to fp32;
#   * the r salient rows are quantized first (they lead the order) and their
#     error is not propagated: the compensator R = W~_s - Q(W~_s) carries it,
#     so propagating it too would correct it twice. Their codes, R, Q(R) and
#     its scales are therefore RTN's; GPTQ acts on rows r..K-1 (r = 0: plain
#     GPTQ on W^);
#   * every step is one fp64 operation in a fixed order (the factorizations
#     by outer-product elimination, the update row by row), so that an
#     independent implementation reproduces the codes bit for bit.
# ---------------------------------------------------------------------------

GPTQ_DAMP = 0.01


def gptq_hessian(X_hat: np.ndarray, damp: float = GPTQ_DAMP) -> np.ndarray:
    """H = sum_t x^_t x^_t^T (fp64, t in order) plus damp * mean(diag H) on
    the diagonal; the identity when every input is zero."""
    X = np.asarray(X_hat, dtype=np.float32).astype(np.float64)
    K = X.shape[1]
    H = np.zeros((K, K), np.float64)
    for t in range(X.shape[0]):
        H += np.multiply.outer(X[t], X[t])
    d = 0.0
    for i in range(K):
        d += H[i, i]
    d = d / K
    if d == 0.0:
        return np.eye(K)
    lam = float(np.float32(damp)) * d
    H[np.arange(K), np.arange(K)] += lam
    return H


def gptq_inverse_factor(H: np.ndarray) -> np.ndarray:
    """Upper-triangular U with U^T U = H^-1: first V upper with H = V V^T
    (elimination from the last index), then U = V^-1 by back substitution.
    Both by outer-product updates, each element updated in a fixed order."""
    K = H.shape[0]
    A = np.array(H, dtype=np.float64)
    V = np.zeros((K, K), np.float64)
    for k in range(K - 1, -1, -1):
        if not A[k, k] > 0.0:
            raise ValueError("Hessian is not positive definite")
        v = np.sqrt(A[k, k])
        V[k, k] = v
        col = A[:k, k] / v
        V[:k, k] = col
        A[:k, :k] -= np.multiply.outer(col, col)
    B = np.eye(K)
    for k in range(K - 1, -1, -1):
        B[k, k:] /= V[k, k]
        B[:k, k:] -= np.multiply.outer(V[:k, k], B[k, k:])
    return B


def gptq_quantize(W_hat: np.ndarray, U: np.ndarray, r: int) -> np.ndarray:
    """GPTQ codes (K x N int8) of the folded, permuted weight W^ (fp32
    values), rows in order, on RTN's grid (scale per output column from the
    column maximum of W^), the first r rows' errors not propagated."""
    W_hat = np.asarray(W_hat, dtype=np.float32)
    K, N = W_hat.shape
    colmax = np.abs(W_hat).max(axis=0) if K else np.zeros(N, np.float32)
    sw = np.zeros(N, np.float32)
    inv = np.zeros(N, np.float32)
    for n in range(N):                      # the quantizer's scale and reciprocal, per column
        _, sw[n] = quantize_group(np.zeros(0, np.float32), colmax[n], 4)
        with np.errstate(divide="ignore", over="ignore"):
            inv[n] = np.float32(np.float32(7.0) / colmax[n])
    live = np.isfinite(inv) & (sw != 0)
    inv = np.where(live, inv, np.float32(0.0)).astype(np.float32)
    Wk = W_hat.astype(np.float64)
    codes = np.zeros((K, N), np.int8)
    for i in range(K):
        v = Wk[i].astype(np.float32)
        q = np.clip(np.rint((v * inv).astype(np.float32)), -8, 7)
        q = np.where(live, q, 0).astype(np.int8)
        codes[i] = q
        if i < r:
            continue
        deq = (q.astype(np.float32) * sw).astype(np.float32).astype(np.float64)
        err = (Wk[i] - deq) / U[i, i]
        Wk[i + 1:] -= np.multiply.outer(U[i, i + 1:], err)
    return codes


def calibrate_gptq(W: np.ndarray, act_absmax: np.ndarray, X_cal: np.ndarray, *,
                   alpha: float = ALPHA_DEFAULT, r: int, damp: float = GPTQ_DAMP) -> dict:
    """SERQ calibration with GPTQ codes on the non-salient rows.

    ``X_cal`` is T x K calibration activations in the original channel order
    (fp32 values). Returns calibrate()'s dict with Wq / Wq_codes / W_deq from
    GPTQ, plus ``H`` and ``U``."""
    base = calibrate(W, act_absmax, alpha=alpha, r=r)
    K, N = base["K"], base["N"]
    perm, shi = base["perm"], base["s_hat_inv"]
    X_hat = (np.asarray(X_cal, dtype=np.float32)[:, perm] * shi[None, :]).astype(np.float32)
    H = gptq_hessian(X_hat, damp)
    U = gptq_inverse_factor(H)
    codes = gptq_quantize(base["W_hat"], U, r)
    sw = base["sw"]
    assert np.array_equal(codes[:r], base["Wq_codes"][:r])
    out = dict(base)
    out.update(Wq_codes=codes, W_deq=dequantize_columns(codes, sw), Wq=pack_int4(codes.T), H=H, U=U,
               X_hat_cal=X_hat)
    return out


def weighted_error(X_hat: np.ndarray, W_hat: np.ndarray, W_deq: np.ndarray, R_deq: np.ndarray | None,
                   r: int) -> float:
    """||X^ W^ - (X^ Q(W^) + X^_s deq(Q(R)))||_F in fp64: the layer's output
    error on the calibration inputs with unquantized activations."""
    X = np.asarray(X_hat, np.float64)
    E = X @ (np.asarray(W_hat, np.float64) - np.asarray(W_deq, np.float64))
    if r and R_deq is not None:
        E = E - X[:, :r] @ np.asarray(R_deq, np.float64)
    return float(np.sqrt((E * E).sum()))


# ---------------------------------------------------------------------------
# The MXFP4 variant of the layer.
# [GDE] 3 (Wichtige Beiträge): SERQ is compatible with the INT4 and MXFP4
# formats; [GDE] 4 (Performance & Latenz): its speed is measured with MXFP4
# on hardware FP4 products, the residual adding about 1 %; [N] 实验关键数据
# sets it beside L2QER-MXFP4. The pages do not define MXFP4; it is the Open
# Compute Project's "OCP Microscaling Formats (MX) Specification" v1.0:
# blocks of 32 consecutive elements share one E8M0 scale X = 2^e, e in
# [-127, 127] (stored as the byte e + 127); each element is FP4 E2M1 (sign,
# two exponent bits with bias 1, one mantissa bit: magnitudes 0, 0.5, 1,
# 1.5, 2, 3, 4, 6). The spec's conversion: e = floor(log2(max |v|)) - 2 (2 is
# E2M1's largest exponent), then every element v / 2^e is rounded to the
# nearest E2M1 value, ties to the even one (mantissa bit 0), and saturated
# at +-6.
#
# Readings (the layer in MXFP4):
#   * the blocks run along the reduction dimension: per output column of W^
#     (32 consecutive rows), per token row of the activations, per output
#     column of R (32 consecutive salient rows); r and K multiples of 32;
#   * an all-zero block (and any block whose exponent would fall below the
#     E8M0 range) takes e = -127; its elements are rounded as above;
#   * s, P and W^ as in the integer layer; R = W~_s - Q(W~_s) with Q the MX
#     quantizer of W^ (the main path's own dequantized salient rows), in
#     fp32; Q(R) in MXFP4; the residual reuses the activation blocks of the
#     first r channels (no second quantization);
#   * Y = sum over blocks b of X_b W_b (sum_k x_k w_k) + sum over b < r/32 of
#     X_b R_b (sum_k x_k rho_k): the block scales are the only scales.
# FP4 codes are packed two per byte like the int4 codes (element 2t in the
# low nibble): sign bit 3, exponent bits 2-1, mantissa bit 0.
# ---------------------------------------------------------------------------

MX_BLOCK = 32
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])     # magnitude of code c & 7
E2M1_MAX_EXP = 2


def e2m1_round(t: np.ndarray) -> np.ndarray:
    """Nearest E2M1 code (0..15) to each value of t (exact scaled values),
    ties to the code with mantissa bit 0, magnitudes above 6 saturated; a
    value that rounds to zero gets code 0 (no negative zero)."""
    t = np.asarray(t, dtype=np.float64)
    a = np.minimum(np.abs(t), 6.0)
    d = np.abs(a[..., None] - E2M1_VALUES)                  # distance to every magnitude
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    even = (np.arange(8) & 1) == 0
    # among the nearest (two at a tie), the even one; else the only one
    pick = np.where(cand & even, 1, 0) + np.where(cand & ~even, 0.5, 0)
    mag = np.argmax(pick, axis=-1)
    sign = (t < 0) & (mag != 0)
    return (mag | (sign.astype(np.int64) << 3)).astype(np.uint8)


def e2m1_value(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64)
    v = E2M1_VALUES[c & 7]
    return np.where(c & 8, -v, v)


def mx_block_exponent(amax: np.ndarray) -> np.ndarray:
    """e = floor(log2(amax)) - 2 clamped to [-127, 127]; -127 for amax = 0."""
    a = np.asarray(amax, dtype=np.float32).astype(np.float64)
    # floor(log2 a) through frexp (a = m 2^ex, m in [1/2, 1)), exact for every binary32 value
    m, ex = np.frexp(np.where(a > 0, a, 1.0))
    fl = ex - 1
    e = np.where(a > 0, fl - E2M1_MAX_EXP, -127)
    return np.clip(e, -127, 127).astype(np.int64)


def mx_quantize_rows(A: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """MXFP4 along the last axis (length a multiple of 32): returns (codes
    uint8 0..15, same shape; exponents int64, one per block of 32)."""
    A = np.asarray(A, dtype=np.float32)
    *lead, L = A.shape
    if L % MX_BLOCK:
        raise ValueError("MX blocks need a length that is a multiple of 32")
    B = A.reshape(*lead, L // MX_BLOCK, MX_BLOCK).astype(np.float64)
    e = mx_block_exponent(np.abs(B).max(axis=-1).astype(np.float32) if L else np.zeros((*lead, 0)))
    t = B * np.exp2(-e.astype(np.float64))[..., None]       # exact: a power-of-two scaling in fp64
    codes = e2m1_round(t).reshape(*lead, L)
    return codes, e


def mx_dequantize_rows(codes: np.ndarray, e: np.ndarray) -> np.ndarray:
    """fp32 values code * 2^e (exact)."""
    *lead, L = codes.shape
    v = e2m1_value(codes).reshape(*lead, L // MX_BLOCK, MX_BLOCK) * np.exp2(e.astype(np.float64))[..., None]
    return v.reshape(*lead, L).astype(np.float32)


def calibrate_mx(W: np.ndarray, act_absmax: np.ndarray, *, alpha: float = ALPHA_DEFAULT, r: int) -> dict:
    """The layer calibrated for MXFP4: s, P and W^ as in calibrate(); Q(W^)
    in MXFP4 per output column (blocks along K), R on the r salient rows,
    Q(R) in MXFP4 per output column (blocks along r).

    Returns perm, s_hat_inv, Wq (N x K/2 packed FP4), Wsc (N x K/32 E8M0
    bytes), Rq (N x r/2), Rsc (N x r/32), and for tests W_hat, Wq_codes and
    We (N x K codes / N x K/32 exponents), W_deq (K x N), R, Rq_codes, Re."""
    W = np.asarray(W, dtype=np.float32)
    K, N = W.shape
    if K % MX_BLOCK or r % MX_BLOCK or not (0 <= r <= K):
        raise ValueError("the MX layer needs K and r multiples of 32, 0 <= r <= K")
    s, s_inv = smoothing_factors(act_absmax, np.abs(W).max(axis=1), alpha)
    perm = saliency_order(s)
    W_hat = fold_and_permute(W, s, perm)
    Wc, We = mx_quantize_rows(W_hat.T)                       # N x K codes, N x K/32 exponents
    W_deq = mx_dequantize_rows(Wc, We).T                     # K x N
    R = compensator(W_hat, W_deq, r)                         # r x N
    if r:
        Rc, Re = mx_quantize_rows(R.T)
    else:
        Rc, Re = np.zeros((N, 0), np.uint8), np.zeros((N, 0), np.int64)
    return dict(K=K, N=N, r=r, s=s, perm=perm, s_hat_inv=s_inv[perm].astype(np.float32), W_hat=W_hat,
                Wq_codes=Wc, We=We, W_deq=W_deq, R=R, Rq_codes=Rc, Re=Re,
                Wq=pack_fp4(Wc), Wsc=(We + 127).astype(np.uint8), Rq=pack_fp4(Rc), Rsc=(Re + 127).astype(np.uint8))


def pack_fp4(codes: np.ndarray) -> np.ndarray:
    """Two FP4 codes per byte, element 2t in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def quant_act_mx(X_perm: np.ndarray, s_hat_inv: np.ndarray) -> dict:
    """x^ = fl32(x * s_hat_inv), then MXFP4 per token row (blocks along K)."""
    x_hat = (np.asarray(X_perm, dtype=np.float32) * np.asarray(s_hat_inv, dtype=np.float32)[None, :]).astype(np.float32)
    codes, e = mx_quantize_rows(x_hat)
    return dict(codes=codes, e=e, packed=pack_fp4(codes), sc=(e + 127).astype(np.uint8), x_hat=x_hat)


def linear_mx(Xq: dict, layer: dict) -> dict:
    """acc_main[m, n] = sum_b 2^(ex_b + ew_b) sum_{k in b} x_k w_k over K and
    acc_res over the first r/32 blocks with Q(R); y = acc_main + acc_res.
    Evaluated in fp64 from the exact element values (each block's sum and
    every scaled product are exact; across blocks the fp64 rounding is far
    below fp32's)."""
    r = layer["r"]
    xv = e2m1_value(Xq["codes"])                                         # M x K
    M, K = xv.shape
    xs = xv.reshape(M, K // MX_BLOCK, MX_BLOCK) * np.exp2(Xq["e"].astype(np.float64))[..., None]
    wv = e2m1_value(layer["Wq_codes"]).reshape(layer["N"], K // MX_BLOCK, MX_BLOCK)
    ws = wv * np.exp2(layer["We"].astype(np.float64))[..., None]
    acc_main = xs.reshape(M, K) @ ws.reshape(layer["N"], K).T
    if r:
        rv = e2m1_value(layer["Rq_codes"]).reshape(layer["N"], r // MX_BLOCK, MX_BLOCK)
        rs = rv * np.exp2(layer["Re"].astype(np.float64))[..., None]
        acc_res = xs[:, : r // MX_BLOCK].reshape(M, r) @ rs.reshape(layer["N"], r).T
    else:
        acc_res = np.zeros_like(acc_main)
    # magnitude sums for the rounding bound of an fp32 accumulation
    mag = np.abs(xs.reshape(M, K)) @ np.abs(ws.reshape(layer["N"], K)).T
    if r:
        mag = mag + np.abs(xs[:, : r // MX_BLOCK].reshape(M, r)) @ np.abs(rs.reshape(layer["N"], r)).T
    return dict(acc_main=acc_main, acc_res=acc_res, y64=acc_main + acc_res, mag=mag)


# ---------------------------------------------------------------------------
# Offline propagation of a later layer's permutation into this layer's output
# columns. [N] 关键设计 3: the activation order a layer needs is produced by
# permuting the previous layer's weight columns offline (the down projection's
# order P4 is pushed into the gate/up columns), so no layer reorders at run
# time. [GDE] 2.C says the same.
# ---------------------------------------------------------------------------

def permute_outputs(layer: dict, perm_next: np.ndarray) -> dict:
    """New output column i is old column perm_next[i] (applied to Wq rows of
    the N-major layout, sw, Rq rows and sr)."""
    p = np.asarray(perm_next)
    out = dict(layer)
    out["Wq"] = layer["Wq"][p]
    out["sw"] = layer["sw"][p]
    out["Rq"] = layer["Rq"][p]
    out["sr"] = layer["sr"][p]
    for key in ("Wq_codes", "Rq_codes", "W_hat", "W_deq", "R"):
        if key in layer:
            out[key] = layer[key][:, p]
    return out


# ---------------------------------------------------------------------------
# Online step 1 -- activation quantization.
# [N] 整体框架: at inference the main path is a pure 4-bit GEMM on Q(X^);
# [N] 关键设计 3: activations arrive already in the saliency order (the
# previous layer's columns were permuted offline), so nothing is gathered
# here. Per-token symmetric quantization, int4 for W4A4 or int8 for W4A8
# ([N] 整体框架 output node "W4A4/W4A8"). x^ = fl32(x * s_hat_inv[k]).
# ---------------------------------------------------------------------------

def quant_act(X_perm: np.ndarray, s_hat_inv: np.ndarray, a_bits: int) -> dict:
    """Returns dict(codes M x K int8, sx M float32, packed bytes)."""
    Xp = np.asarray(X_perm, dtype=np.float32)
    x_hat = (Xp * np.asarray(s_hat_inv, dtype=np.float32)[None, :]).astype(np.float32)
    codes, sx = quantize_rows(x_hat, a_bits)
    packed = pack_int4(codes) if a_bits == 4 else codes.view(np.uint8).copy()
    return dict(codes=codes, sx=sx, packed=packed, x_hat=x_hat)


# ---------------------------------------------------------------------------
# Online step 2 -- the SERQ linear.
# [N] 关键设计 2: X^ W^ ~ X^_q W^_q + X~_{s,q} Q(R); the residual is a single
# (tokens x r) x (r x d) product, R is itself quantized, and there is no
# intermediate quantization. [GDE] 2.B writes the same operator with
# Q(X~_s); [GJA] 2 ("計算フローの革新") contrasts X_q W_q + X_{s,q} R_q with
# L2QER's serial two-factor form. Reading: X~_{s,q} is the first r columns of
# the already quantized activations (same codes, same per-token scale), i.e.
# no second quantization of the salient channels.
# ---------------------------------------------------------------------------

def linear_int(Xq_codes: np.ndarray, Wq_codes: np.ndarray, Rq_codes: np.ndarray,
               r: int) -> tuple[np.ndarray, np.ndarray]:
    """acc_main = Xq . Wq over all K, acc_res = Xq[:, :r] . Rq, exact int64.

    ``Wq_codes`` is K x N and ``Rq_codes`` r x N (codes, not packed)."""
    Xc = np.asarray(Xq_codes, dtype=np.int64)
    acc_main = Xc @ np.asarray(Wq_codes, dtype=np.int64)
    if r:
        acc_res = Xc[:, :r] @ np.asarray(Rq_codes, dtype=np.int64)
    else:
        acc_res = np.zeros_like(acc_main)
    if acc_main.size:
        assert np.abs(acc_main).max() < 2**31 and np.abs(acc_res).max() < 2**31
    return acc_main, acc_res


def epilogue(acc_main: np.ndarray, acc_res: np.ndarray, sx: np.ndarray, sw: np.ndarray,
             sr: np.ndarray) -> np.ndarray:
    """y = sx_m * (sw_n * acc_main + sr_n * acc_res) evaluated in fp64."""
    sx64 = np.asarray(sx, dtype=np.float64)[:, None]
    sw64 = np.asarray(sw, dtype=np.float64)[None, :]
    sr64 = np.asarray(sr, dtype=np.float64)[None, :]
    return sx64 * (sw64 * acc_main.astype(np.float64) + sr64 * acc_res.astype(np.float64))


def round_f64_to_bf16(y: np.ndarray) -> np.ndarray:
    """Round fp64 values once to bf16 (nearest even); returns float32 arrays
    holding the bf16 values. Values in the normal bf16 range only."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    u = y.view(np.uint64)
    drop = np.uint64(52 - 7)
    lsb = (u >> drop) & np.uint64(1)
    bias = (np.uint64(1) << (drop - np.uint64(1))) - np.uint64(1) + lsb
    u2 = ((u + bias) >> drop) << drop
    return u2.view(np.float64).astype(np.float32)


def linear(Xq: dict, layer: dict, *, out: str = "bf16") -> dict:
    """The layer output for quantized activations ``Xq`` (from quant_act)."""
    r = layer["r"]
    acc_main, acc_res = linear_int(Xq["codes"], layer["Wq_codes"], layer["Rq_codes"], r)
    y64 = epilogue(acc_main, acc_res, Xq["sx"], layer["sw"], layer["sr"])
    if out == "f32":
        y = y64.astype(np.float32)
    elif out == "bf16":
        y = round_f64_to_bf16(y64)
    else:
        raise ValueError("out must be 'f32' or 'bf16'")
    return dict(acc_main=acc_main, acc_res=acc_res, y64=y64, y=y)


def linear_float_residual(Xq: dict, layer: dict) -> np.ndarray:
    """Test hook: the residual with an unquantized R (fp64), for the special
    case r = K where the weight error is removed exactly."""
    r = layer["r"]
    xd = Xq["codes"].astype(np.float64) * Xq["sx"].astype(np.float64)[:, None]
    main = xd @ (layer["Wq_codes"].astype(np.float64) * layer["sw"].astype(np.float64)[None, :])
    res = xd[:, :r] @ layer["R"].astype(np.float64)
    return main + res


# ---------------------------------------------------------------------------
# The MLP activation between gate/up and down, fused with down's activation
# quantization. [N] 关键设计 3: the down projection's input permutation is
# pushed offline into the gate/up output channels, so h = silu(g) * u leaves
# the elementwise step already in down's saliency order and goes straight
# into the per-token quantizer, with no gather. The pages do not spell out
# the MLP nonlinearity; the reading is the LLaMA MLP, silu(g) = g * sigma(g)
# = g / (1 + e^-g). For bit-exact parity both implementations evaluate it
# with one fixed fp32 recipe (IEEE division; fused multiply-adds, each one
# exactly rounded, where written, and nowhere else):
#     e  = exp32(-g)            (argument clamped to [-80, 80])
#     sg = fl32(g / fl32(1 + e))
#     h  = fl32(sg * u)
# exp32 follows Cody and Waite's argument reduction: e^x = 2^n e^r with
# n = rne(fl32(x log2 e)) and r = fma(-n, c_lo, fma(-n, c_hi, x)), where
# c_hi + c_lo = ln 2 and c_hi = 22713 * 2^-15 has 15 significant bits (the
# clamp keeps |n| <= 116, 7 bits, so n c_hi has at most 22 significant bits
# and is exact, and the first fma is exact too); e^r (|r| <= ln2 / 2) is its
# Taylor polynomial to degree 7 in Horner form, p <- fma(p, r, 1/k!)
# (truncation below 2^-27 relative), then scaled by 2^n exactly. The clamp
# keeps every intermediate a normal number.
# ---------------------------------------------------------------------------

LOG2E_F32 = np.float32(1.0 / math.log(2.0))
LN2_HI_F32 = np.float32(0.693145751953125)                  # 22713 * 2^-15: 15 significant bits
LN2_LO_F32 = np.float32(math.log(2.0) - 0.693145751953125)
EXP_TAYLOR_F32 = [np.float32(1.0 / math.factorial(k)) for k in range(8)]   # 1/k!
EXP_ARG_CLAMP = np.float32(80.0)


def fma32(a, b, c) -> np.ndarray:
    """fl32(a * b + c) with one rounding (round to nearest even), for float32
    operands whose result is a normal number or zero. a * b is exact in
    binary64 (48 significant bits); the sum is rounded to odd in binary64
    (round to nearest, then, if inexact, the neighbour with an odd last bit
    toward the exact value -- the error comes from Knuth's two-sum), and
    that rounds correctly to binary32 since 53 >= 24 + 2 (Boldo and
    Melquiond, "Emulation of FMA and correctly rounded sums: proved
    algorithms using rounding to odd", IEEE Trans. Computers 2008)."""
    a64 = np.asarray(a, dtype=np.float32).astype(np.float64)
    b64 = np.asarray(b, dtype=np.float32).astype(np.float64)
    c64 = np.asarray(c, dtype=np.float32).astype(np.float64)
    p = a64 * b64
    s = p + c64
    bv = s - p
    t = (p - (s - bv)) + (c64 - bv)              # two-sum: p + c = s + t exactly
    even = (s.view(np.int64) & 1) == 0
    s = np.where((t != 0) & even, np.nextafter(s, np.where(t > 0, np.inf, -np.inf)), s)
    return s.astype(np.float32)


def exp32(x: np.ndarray) -> np.ndarray:
    """e^x for float32 x by the fixed recipe above (elementwise, float32)."""
    x = np.clip(np.asarray(x, dtype=np.float32), -EXP_ARG_CLAMP, EXP_ARG_CLAMP).astype(np.float32)
    n = np.rint((x * LOG2E_F32).astype(np.float32)).astype(np.float32)
    r = fma32(-n, LN2_HI_F32, x)
    r = fma32(-n, LN2_LO_F32, r)
    p = np.full(x.shape, EXP_TAYLOR_F32[7], np.float32)
    for k in range(6, -1, -1):
        p = fma32(p, r, EXP_TAYLOR_F32[k])
    return np.ldexp(p, n.astype(np.int32)).astype(np.float32)


def silu_mul(G: np.ndarray, U: np.ndarray) -> np.ndarray:
    """h = silu(g) * u elementwise in fp32 by the recipe above."""
    g = np.asarray(G, dtype=np.float32)
    u = np.asarray(U, dtype=np.float32)
    e = exp32(-g)
    s = (np.float32(1.0) + e).astype(np.float32)
    sg = (g / s).astype(np.float32)
    return (sg * u).astype(np.float32)


def silu_mul_quant_act(G: np.ndarray, U: np.ndarray, s_hat_inv: np.ndarray, a_bits: int) -> dict:
    """down's quantized input from the gate and up outputs (both M x K, in
    down's saliency order): quant_act(silu(G) * U)."""
    return quant_act(silu_mul(G, U), s_hat_inv, a_bits)
