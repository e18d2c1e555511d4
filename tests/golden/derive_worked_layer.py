"""Exact derivation of the worked 4 x 2 layer in worked_layer_4x2.json.

Every value is computed in exact rational arithmetic (Python fractions) and
rounded to binary32 (or bfloat16 for the output) by an explicit
round-to-nearest-even after each step that the layer performs in fp32. It
uses neither the oracle nor the library, so the fixture it checks pins both.
The steps follow papernotes.org's SERQ notes (关键设计 1: the SmoothQuant
factor folded into the weights; 关键设计 2: rows ordered by descending
saliency, the operator X^_q W^_q + X~_{s,q} Q(R); 核心 idea: R = W~_s − Q(W~_s)),
with this library's stated readings for what the pages leave open (the
factor max|X|^a / max|W|^(1-a) with a = 1/2, a stable descending sort, the
quantizer scale fl32(m/qmax) and codes rne(fl32(v fl32(qmax/m))) clamped).

Run directly to print the derived values next to the fixture's.
"""

from __future__ import annotations

import json
import math
import os
from fractions import Fraction as F

HERE = os.path.dirname(os.path.abspath(__file__))


def rne_int(x: F) -> int:
    """Nearest integer to x, ties to even."""
    fl = math.floor(x)
    rem = x - fl
    if rem > F(1, 2) or (rem == F(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


def round_float(x: F, mant_bits: int) -> F:
    """Nearest value with `mant_bits` significant bits (normal range), ties
    to even: 24 for binary32, 8 for bfloat16."""
    if x == 0:
        return F(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while F(2) ** e > a:
        e -= 1
    while F(2) ** (e + 1) <= a:
        e += 1
    ulp = F(2) ** (e - (mant_bits - 1))
    return sign * rne_int(a / ulp) * ulp


def f32(x) -> F:
    return round_float(F(x), 24)


def quantize(vals, qmax: int, qmin: int):
    m = max(abs(v) for v in vals)
    if m == 0:
        return [0] * len(vals), F(0)
    inv = f32(F(qmax) / m)
    scale = f32(m / qmax)
    return [max(qmin, min(qmax, rne_int(f32(v * inv)))) for v in vals], scale


def derive(inputs: dict) -> dict:
    W = [[F(v) for v in row] for row in inputs["W"]]
    a = [F(v) for v in inputs["act_absmax"]]
    r = inputs["r"]
    K, N = len(W), len(W[0])
    w = [max(abs(v) for v in row) for row in W]
    # s_j = sqrt(a_j) / sqrt(w_j): every a_j and w_j here is a perfect square
    # of a rational, so the square roots are exact.
    def sqrt(q: F) -> F:
        n, d = math.isqrt(q.numerator), math.isqrt(q.denominator)
        assert F(n, d) ** 2 == q, "the worked example uses exact squares"
        return F(n, d)
    s = [f32(sqrt(a[j]) / sqrt(w[j])) for j in range(K)]
    s_inv = [f32(1 / sj) for sj in s]
    perm = sorted(range(K), key=lambda j: (-s[j], j))
    W_hat = [[f32(s[p] * W[p][n]) for n in range(N)] for p in perm]
    Wq = [[0] * N for _ in range(K)]
    sw = []
    for n in range(N):
        codes, sc = quantize([W_hat[i][n] for i in range(K)], 7, -8)
        for i in range(K):
            Wq[i][n] = codes[i]
        sw.append(sc)
    W_deq = [[f32(Wq[i][n] * sw[n]) for n in range(N)] for i in range(K)]
    R = [[f32(W_hat[i][n] - W_deq[i][n]) for n in range(N)] for i in range(r)]
    Rq = [[0] * N for _ in range(r)]
    sr = []
    for n in range(N):
        codes, sc = quantize([R[i][n] for i in range(r)], 7, -8)
        for i in range(r):
            Rq[i][n] = codes[i]
        sr.append(sc)
    out = dict(s=s, perm=perm, s_hat_inv=[s_inv[p] for p in perm], W_hat=W_hat, Wq_codes=Wq, sw=sw,
               W_deq=W_deq, R=R, Rq_codes=Rq, sr=sr, x_hat=[], Xq_codes=[], sx=[], acc_main=[], acc_res=[],
               y_f32=[], y_bf16=[])
    for x in inputs["X"]:
        xp = [F(x[p]) for p in perm]
        xh = [f32(xp[k] * out["s_hat_inv"][k]) for k in range(K)]
        xc, sx = quantize(xh, 7, -8)
        am = [sum(xc[k] * Wq[k][n] for k in range(K)) for n in range(N)]
        ar = [sum(xc[k] * Rq[k][n] for k in range(r)) for n in range(N)]
        y = [sx * (sw[n] * am[n] + sr[n] * ar[n]) for n in range(N)]
        out["x_hat"].append(xh)
        out["Xq_codes"].append(xc)
        out["sx"].append(sx)
        out["acc_main"].append(am)
        out["acc_res"].append(ar)
        out["y_f32"].append([round_float(v, 24) for v in y])
        out["y_bf16"].append([round_float(v, 8) for v in y])
    return out


def load_fixture() -> dict:
    with open(os.path.join(HERE, "worked_layer_4x2.json")) as f:
        return json.load(f)


if __name__ == "__main__":
    fx = load_fixture()
    got = derive(fx["inputs"])
    for k, v in got.items():
        print(f"{k:10s} derived {json.dumps(v, default=float)}")
        print(f"{'':10s} fixture {json.dumps(fx['expected'].get(k))}")
