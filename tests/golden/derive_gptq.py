"""Exact derivation of GPTQ codes, for the pins of the oracle's GPTQ step.

GPTQ (Frantar, Ashkboos, Hoefler and Alistarh, "GPTQ: Accurate
Post-Training Quantization for Generative Pre-trained Transformers", ICLR
2023) rests on the optimal-brain-surgeon step: when row i of the weights is
quantized while the rows F = {i+1, ...} are still free, the change of the
free rows that minimises the squared output error over the calibration
inputs is

    w_F  <-  w_F - (w_i - q_i) * G[F, i] / G[i, i],   G = (H[{i} + F, {i} + F])^-1,

with H = X^T X. This script evaluates exactly that in rational arithmetic
(Python fractions): H exactly, the inverse of each trailing block by
Gauss-Jordan elimination, the update exactly. It never forms a Cholesky
factor, so it is an independent statement of what the oracle computes with
fp64 factorizations. The quantizer is the library's: per output column,
scale fl32(m/7) and reciprocal fl32(7/m) from the column maximum m of the
weights before any update; code = clamp(rne(fl32(fl32(w) * inv)), -8, 7).
The first r rows (the salient rows, whose error the SERQ compensator
carries) are quantized without an update, as the oracle's reading states.
Dampening: damp * mean(diag H) added to the diagonal (all-zero H: identity).

Run directly to print the fixture gptq_4x2.json's inputs and derived codes.
"""

from __future__ import annotations

import json
import math
import os
from fractions import Fraction as F

HERE = os.path.dirname(os.path.abspath(__file__))


def rne_int(x: F) -> int:
    fl = math.floor(x)
    rem = x - fl
    if rem > F(1, 2) or (rem == F(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


def f32(x: F) -> F:
    """Nearest binary32 value (normal range or zero), ties to even."""
    x = F(x)
    if x == 0:
        return F(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while F(2) ** e > a:
        e -= 1
    while F(2) ** (e + 1) <= a:
        e += 1
    ulp = F(2) ** (e - 23)
    return sign * rne_int(a / ulp) * ulp


def inverse(A):
    """Exact inverse of a square rational matrix (Gauss-Jordan)."""
    n = len(A)
    M = [list(row) + [F(int(i == j)) for j in range(n)] for i, row in enumerate(A)]
    for c in range(n):
        p = next(i for i in range(c, n) if M[i][c] != 0)
        M[c], M[p] = M[p], M[c]
        piv = M[c][c]
        M[c] = [v / piv for v in M[c]]
        for i in range(n):
            if i != c and M[i][c] != 0:
                f = M[i][c]
                M[i] = [a - f * b for a, b in zip(M[i], M[c])]
    return [row[n:] for row in M]


def gptq_codes(W_hat, X_hat, r: int, damp) -> list[list[int]]:
    """Codes (K x N) for the weights W_hat (K x N) and inputs X_hat (T x K),
    both given as exact binary32 values."""
    W = [[F(v) for v in row] for row in W_hat]
    X = [[F(v) for v in row] for row in X_hat]
    K, N = len(W), len(W[0])
    H = [[sum((X[t][i] * X[t][j] for t in range(len(X))), F(0)) for j in range(K)] for i in range(K)]
    d = sum((H[i][i] for i in range(K)), F(0)) / K
    if d == 0:
        H = [[F(int(i == j)) for j in range(K)] for i in range(K)]
    else:
        lam = F(damp) * d
        for i in range(K):
            H[i][i] += lam
    cmax = [max(abs(W[i][n]) for i in range(K)) for n in range(N)]
    scale = [f32(m / 7) if m else F(0) for m in cmax]
    inv = [f32(F(7) / m) if m else F(0) for m in cmax]
    codes = [[0] * N for _ in range(K)]
    for i in range(K):
        for n in range(N):
            if cmax[n] == 0:
                continue
            codes[i][n] = max(-8, min(7, rne_int(f32(f32(W[i][n]) * inv[n]))))
        if i < r or i == K - 1:
            continue
        idx = list(range(i, K))
        G = inverse([[H[a][b] for b in idx] for a in idx])
        for n in range(N):
            e = W[i][n] - f32(codes[i][n] * scale[n])
            for jj in range(1, len(idx)):
                W[idx[jj]][n] -= e * G[jj][0] / G[0][0]
    return codes


def load_fixture() -> dict:
    with open(os.path.join(HERE, "gptq_4x2.json")) as f:
        return json.load(f)


def derive(inputs: dict) -> dict:
    out = {}
    for case in inputs["cases"]:
        out[case["name"]] = gptq_codes(inputs["W_hat"], inputs["X_hat"], case["r"], F(case["damp"]))
    return out


if __name__ == "__main__":
    fx = load_fixture()
    got = derive(fx["inputs"])
    for k, v in got.items():
        print(k, v, "fixture:", fx["expected"][k])
