"""Seeded synthetic workloads for the SERQ quantized linear layer.

This module only draws random numbers and lays them out. It holds none of
the method's arithmetic (no smoothing factor, no permutation, no
quantization), so both the CPU oracle and the HIP library can be fed from it
without sharing any of the computation they are compared on.

What the inputs stand in for
----------------------------
The SERQ pages (papernotes.org ICLR2026 notes, sections "研究背景与动机" and
"关键设计 1"; gist.science/de "Technische Zusammenfassung" §1) describe LLM
activations by their channel-wise outliers: a few input channels carry values
tens of times larger than the rest. Weights are taken as roughly normal (the
same notes, "关键设计 2", state the normal-weight assumption used to rank
salient rows). The pages evaluate on WikiText-2, Pile, MMLU and zero-shot
suites with trained LLaMA/Qwen weights; none of those are used here. These
generators stand in for them with

  * W ~ N(0, 0.02^2), K x N (so that Y = X W),
  * X ~ N(0, 1), M x K, with ``n_out`` randomly chosen outlier columns
    multiplied by ``f``,
  * a calibration batch X_cal of 256 rows drawn the same way, whose per
    channel absolute maximum is the calibration statistic.

Draw order (fixed, so that every consumer sees identical values):
  1. outlier channel indices ``rng.choice(K, n_out, replace=False)``
  2. ``W = 0.02 * standard_normal((K, N))``
  3. ``X_cal = standard_normal((256, K))``, outlier columns times ``f``
  4. ``X = standard_normal((M_max, K))``, outlier columns times ``f``
with ``rng = numpy.random.default_rng(SeedSequence([seed, tag]))``.
Every M of one layer uses the first M rows of the same X.

bfloat16 workloads round the fp32 draws to bfloat16 (round to nearest even)
here, at generation, so both sides consume identical bf16 values.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

CAL_ROWS = 256


def rng_for(seed: int, tag: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), int(tag)]))


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Input preparation only: a bf16 workload is *defined* as these values.
    Non-finite inputs are not produced by the generators.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    # in 32 bits: the largest finite pattern 0xFF7FFFFF plus 0x8000 does not wrap
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    lsb += np.uint32(0x7FFF)
    lsb += u
    lsb >>= np.uint32(16)
    return lsb.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class LayerInputs:
    """One synthetic linear layer.

    ``W`` (K x N) and ``X`` (M_max x K) are float32 arrays holding exactly the
    values of the workload (bf16-representable values for bf16 workloads).
    ``W_bits`` / ``X_bits`` hold the bf16 bit patterns when ``dtype`` is
    ``"bf16"``, else ``None``.
    """

    K: int
    N: int
    M_max: int
    dtype: str
    outliers: np.ndarray
    W: np.ndarray
    X_cal: np.ndarray
    X: np.ndarray
    act_absmax: np.ndarray
    W_bits: np.ndarray | None = None
    X_bits: np.ndarray | None = None
    meta: dict = field(default_factory=dict)


def make_layer(K: int, N: int, M_max: int, *, n_out: int, factor: float,
               seed: int, tag: int, dtype: str = "bf16",
               w_std: float = 0.02, draw_x: bool = True) -> LayerInputs:
    if dtype not in ("f32", "bf16"):
        raise ValueError("dtype must be 'f32' or 'bf16'")
    rng = rng_for(seed, tag)
    outl = np.sort(rng.choice(K, n_out, replace=False)) if n_out > 0 else np.zeros(0, np.int64)
    W = rng.standard_normal((K, N), dtype=np.float32)
    W *= np.float32(w_std)
    X_cal = rng.standard_normal((CAL_ROWS, K), dtype=np.float32)
    X_cal[:, outl] *= np.float32(factor)
    if draw_x:
        X = rng.standard_normal((M_max, K), dtype=np.float32)
        X[:, outl] *= np.float32(factor)
    else:
        X = np.zeros((M_max, K), np.float32)
    W_bits = X_bits = None
    if dtype == "bf16":
        W_bits = round_to_bf16_bits(W)
        W = bf16_bits_to_f32(W_bits).reshape(K, N)
        W_bits = W_bits.reshape(K, N)
        X_bits = round_to_bf16_bits(X).reshape(M_max, K)
        X = bf16_bits_to_f32(X_bits).reshape(M_max, K)
        X_cal = bf16_bits_to_f32(round_to_bf16_bits(X_cal)).reshape(CAL_ROWS, K)
    act_absmax = np.abs(X_cal).max(axis=0).astype(np.float32)
    return LayerInputs(K=K, N=N, M_max=M_max, dtype=dtype, outliers=outl, W=W,
                       X_cal=X_cal, X=X, act_absmax=act_absmax,
                       W_bits=W_bits, X_bits=X_bits)


def extra_weight(K: int, N: int, *, seed: int, tag: int, dtype: str = "bf16",
                 w_std: float = 0.02) -> tuple[np.ndarray, np.ndarray | None]:
    """A second weight matrix for a layer that shares its input (W_up next to
    W_gate). Only ``W`` is drawn from this tag's stream."""
    rng = rng_for(seed, tag)
    W = rng.standard_normal((K, N), dtype=np.float32)
    W *= np.float32(w_std)
    if dtype == "bf16":
        bits = round_to_bf16_bits(W).reshape(K, N)
        return bf16_bits_to_f32(bits).reshape(K, N), bits
    return W, None


# --------------------------------------------------------------------------
# The five workloads. Shapes: LLaMA-2-7B q_proj, LLaMA-3-8B MLP, LLaMA-2-70B
# MLP-shaped layer (one GPU's whole layer). Outlier share 1 % (0.5 % for the
# 70B shapes) of the input channels, scaled x50 (x100 for the 70B shapes).
# --------------------------------------------------------------------------

WORKLOADS = {
    "tiny": dict(layers={"tiny": dict(K=256, N=256, n_out=3, factor=40.0, tag=9)},
                 r=8, Ms=(16,), a_bits=4, dtype="f32", out="f32"),
    "q_proj": dict(layers={"q_proj": dict(K=4096, N=4096, n_out=40, factor=50.0, tag=0)},
                   r=64, Ms=(1, 16, 256, 2048), a_bits=4, dtype="bf16", out="bf16"),
    "mlp8b": dict(layers={"gate_up": dict(K=4096, N=14336, n_out=40, factor=50.0, tag=1, up_tag=2),
                          "down": dict(K=14336, N=4096, n_out=143, factor=50.0, tag=3)},
                  r=128, Ms=(1, 32, 4096), a_bits=4, dtype="bf16", out="bf16"),
    "mlp8b_w4a8": dict(layers={"gate_up": dict(K=4096, N=14336, n_out=40, factor=50.0, tag=1, up_tag=2),
                               "down": dict(K=14336, N=4096, n_out=143, factor=50.0, tag=3)},
                       r=128, Ms=(2048,), a_bits=8, dtype="bf16", out="bf16"),
    "l70b": dict(layers={"up70": dict(K=8192, N=28672, n_out=40, factor=100.0, tag=4),
                         "down70": dict(K=28672, N=8192, n_out=143, factor=100.0, tag=5)},
                 r=256, Ms=(1, 8192), a_bits=4, dtype="bf16", out="bf16"),
}


def workload_layer(workload: str, layer: str, *, M_max: int | None = None,
                   seed: int = 0, draw_x: bool = True) -> LayerInputs:
    wl = WORKLOADS[workload]
    spec = wl["layers"][layer]
    M = max(wl["Ms"]) if M_max is None else M_max
    li = make_layer(spec["K"], spec["N"], M, n_out=spec["n_out"], factor=spec["factor"],
                    seed=seed, tag=spec["tag"], dtype=wl["dtype"], draw_x=draw_x)
    li.meta.update(workload=workload, layer=layer, r=wl["r"], a_bits=wl["a_bits"], out=wl["out"])
    if "up_tag" in spec:
        Wu, Wu_bits = extra_weight(spec["K"], spec["N"], seed=seed, tag=spec["up_tag"], dtype=wl["dtype"])
        li.meta["W_up"] = Wu
        li.meta["W_up_bits"] = Wu_bits
    return li


def random_codes(rng: np.random.Generator, shape, bits: int) -> np.ndarray:
    """Uniform random signed codes of ``bits`` width (int8 array), for tests
    that drive the integer GEMM directly."""
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1))
    return rng.integers(lo, hi, size=shape, dtype=np.int64).astype(np.int8)
