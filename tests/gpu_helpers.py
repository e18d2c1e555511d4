"""Helpers for the GPU parity tests: upload/download, oracle references on
sampled rows and columns, and the output tolerance.

Tolerance (fp32 output): the kernel forms t = fl(sw * acc_main) (acc_main is
exact in fp32, |acc| < 2^24), u = fma(sr, acc_res, t) and y = fl(sx * u):
three roundings of partial results bounded by F = sx (sw |acc_main| +
sr |acc_res|), so |y - y_exact| <= 3 * 2^-24 * F (1 + 2^-23) < 2^-21 F. This
is tighter than the 1e-3 relative figure the layer is specified with.
bf16 output: the fp32 value above rounded once more, so at most one bf16
spacing at |y_ref| away from the exactly rounded reference, plus 2^-21 F.
"""

from __future__ import annotations

import numpy as np
import torch

from oracle import serq_oracle as O

DEV = "cuda"


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_tensor(bits: np.ndarray) -> torch.Tensor:
    return dev(bits.view(np.int16)).view(torch.bfloat16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_spacing(v: np.ndarray) -> np.ndarray:
    """Distance to the next bf16 value above |v| (normal range)."""
    a = np.abs(v.astype(np.float32))
    e = np.floor(np.log2(np.maximum(a, np.float32(2.0 ** -126))))
    return np.exp2(e - 7)


def check_y(y_gpu: np.ndarray, acc_main: np.ndarray, acc_res: np.ndarray, sx, sw, sr, out: str):
    """Compare kernel outputs with the oracle epilogue on the same integer
    accumulators (already checked bit-exact by the caller)."""
    y64 = O.epilogue(acc_main, acc_res, sx, sw, sr)
    floor = (np.asarray(sx, np.float64)[:, None]
             * (np.asarray(sw, np.float64)[None, :] * np.abs(acc_main)
                + np.asarray(sr, np.float64)[None, :] * np.abs(acc_res)))
    if out == "f32":
        ref = y64.astype(np.float32)
        got = y_gpu.astype(np.float64)
        tol = 2.0 ** -21 * floor
    else:
        ref = O.round_f64_to_bf16(y64)
        got = bf16_bits_to_f32(y_gpu).astype(np.float64)
        tol = np.maximum(bf16_spacing(ref), bf16_spacing(got.astype(np.float32))) + 2.0 ** -21 * floor
    err = np.abs(got - ref.astype(np.float64))
    bad = err > tol
    assert not bad.any(), (f"{bad.sum()} outputs out of tolerance; worst at "
                           f"{np.unravel_index(np.argmax(err - tol), err.shape)}: got "
                           f"{got.flat[np.argmax(err - tol)]} ref {ref.flat[np.argmax(err - tol)]}")
    return ref


def sample(n: int, k: int, seed: int) -> np.ndarray:
    if n <= k:
        return np.arange(n)
    rng = np.random.default_rng(seed)
    s = rng.choice(n, k, replace=False)
    # always include the edges (first/last row or column: ragged tails)
    return np.unique(np.concatenate([s, [0, n - 1]]))
