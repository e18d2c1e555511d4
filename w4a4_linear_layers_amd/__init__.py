"""SERQ quantized linear layer for AMD MI355X (gfx950).

Thin Python front end of libserq (include/serq.h): argument marshalling
only. Calibration runs in the library's host code; ``quant_act`` and
``linear`` enqueue the library's HIP kernels on the current torch stream.
PyTorch provides device memory and streams, nothing else.

    layer = calibrate(W, act_absmax, r=64)          # offline, host
    dev = layer.to("cuda")
    xq, sx = quant_act(x_perm, dev)                  # x already in saliency order
    y = linear(xq, sx, dev, out_dtype=torch.bfloat16)
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import _lib
from ._lib import SERQ_BF16, SERQ_F32, SerqError, check

lib = _lib.lib

__all__ = ["SerqLayer", "DeviceLayer", "calibrate", "calibrate_gptq", "permute_outputs", "quant_act", "silu_mul_quant_act",
           "linear", "kernel_name", "rq_row_bytes", "SerqError", "Bf6Layer", "bf6_bytes", "prepack_bf6", "act_bf6",
           "linear_bf6", "bf6_kernel_name", "MxLayer", "calibrate_mx", "quant_act_mx", "linear_mx"]


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(__import__("ctypes").c_void_p) if a is not None and a.size else None


@dataclass
class SerqLayer:
    """Calibrated layer in host memory (canonical layouts of include/serq.h)."""

    K: int
    N: int
    r: int
    perm: np.ndarray        # K int32
    s_hat_inv: np.ndarray   # K float32
    Wq: np.ndarray          # N x K/2 uint8
    sw: np.ndarray          # N float32
    Rq: np.ndarray          # N x rq_row_bytes(r) uint8 (zero codes past r)
    sr: np.ndarray          # N float32

    def to(self, device="cuda") -> "DeviceLayer":
        import torch
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)  # noqa: E731
        return DeviceLayer(K=self.K, N=self.N, r=self.r, perm=t(self.perm), s_hat_inv=t(self.s_hat_inv),
                           Wq=t(self.Wq), sw=t(self.sw), Rq=t(self.Rq), sr=t(self.sr))

    def save(self, path: str) -> None:
        np.savez(path, K=self.K, N=self.N, r=self.r, perm=self.perm, s_hat_inv=self.s_hat_inv,
                 Wq=self.Wq, sw=self.sw, Rq=self.Rq, sr=self.sr)

    @staticmethod
    def load(path: str) -> "SerqLayer":
        z = np.load(path, allow_pickle=False)
        return SerqLayer(K=int(z["K"]), N=int(z["N"]), r=int(z["r"]), perm=z["perm"], s_hat_inv=z["s_hat_inv"],
                         Wq=z["Wq"], sw=z["sw"], Rq=z["Rq"], sr=z["sr"])


@dataclass
class DeviceLayer:
    """Calibrated layer in device memory (torch tensors)."""

    K: int
    N: int
    r: int
    perm: "object"
    s_hat_inv: "object"
    Wq: "object"
    sw: "object"
    Rq: "object"
    sr: "object"


def rq_row_bytes(r: int) -> int:
    """Bytes per row of the packed Q(R) buffer (serq_rq_row_bytes): r codes
    padded with zero codes to a multiple of 32."""
    b = lib.serq_rq_row_bytes(int(r))
    if b < 0:
        raise ValueError("r must be >= 0")
    return b


def calibrate(W, act_absmax, *, r: int, alpha: float = 0.5, w_dtype: str | None = None) -> SerqLayer:
    """Offline calibration (serq_calibrate). ``W`` is K x N: a float32 array,
    a uint16 array of bf16 bit patterns (``w_dtype="bf16"``), or a CPU torch
    tensor of dtype float32 / bfloat16."""
    try:
        import torch
        if isinstance(W, torch.Tensor):
            if W.dtype == torch.bfloat16:
                W = W.contiguous().view(torch.int16).numpy().view(np.uint16)
                w_dtype = "bf16"
            else:
                W = W.contiguous().float().numpy()
        if isinstance(act_absmax, torch.Tensor):
            act_absmax = act_absmax.float().numpy()
    except ImportError:  # pragma: no cover
        pass
    W = np.ascontiguousarray(W)
    if w_dtype is None:
        w_dtype = "bf16" if W.dtype == np.uint16 else "f32"
    if w_dtype == "bf16":
        W = np.ascontiguousarray(W, dtype=np.uint16)
        dt = SERQ_BF16
    else:
        W = np.ascontiguousarray(W, dtype=np.float32)
        dt = SERQ_F32
    K, N = W.shape
    amax = np.ascontiguousarray(act_absmax, dtype=np.float32)
    if amax.shape != (K,):
        raise ValueError("act_absmax must have K entries")
    perm = np.empty(K, np.int32)
    shi = np.empty(K, np.float32)
    Wq = np.empty((N, K // 2), np.uint8)
    sw = np.empty(N, np.float32)
    Rq = np.zeros((N, rq_row_bytes(r)), np.uint8)
    sr = np.zeros(N, np.float32)
    check("serq_calibrate", lib.serq_calibrate(_ptr(W), dt, K, N, _ptr(amax), float(alpha), r, _ptr(perm),
                                               _ptr(shi), _ptr(Wq), _ptr(sw), _ptr(Rq) if r else None,
                                               _ptr(sr) if r else None))
    return SerqLayer(K=K, N=N, r=r, perm=perm, s_hat_inv=shi, Wq=Wq, sw=sw, Rq=Rq, sr=sr)


def _host_matrix(A, dtype_hint):
    """A float32 array, a uint16 array of bf16 bit patterns, or a CPU torch
    tensor of dtype float32 / bfloat16 -> (contiguous array, SERQ dtype)."""
    try:
        import torch
        if isinstance(A, torch.Tensor):
            if A.dtype == torch.bfloat16:
                A = A.contiguous().view(torch.int16).numpy().view(np.uint16)
                dtype_hint = "bf16"
            else:
                A = A.contiguous().float().numpy()
    except ImportError:  # pragma: no cover
        pass
    A = np.ascontiguousarray(A)
    if dtype_hint is None:
        dtype_hint = "bf16" if A.dtype == np.uint16 else "f32"
    if dtype_hint == "bf16":
        return np.ascontiguousarray(A, dtype=np.uint16), SERQ_BF16
    return np.ascontiguousarray(A, dtype=np.float32), SERQ_F32


def calibrate_gptq(W, act_absmax, X_cal, *, r: int, alpha: float = 0.5, damp: float = 0.01,
                   w_dtype: str | None = None, x_dtype: str | None = None) -> SerqLayer:
    """Offline calibration with GPTQ weight codes (serq_calibrate_gptq).
    ``X_cal`` is T x K calibration activations in the original channel
    order (float32, bf16 bit patterns with ``x_dtype="bf16"``, or a CPU torch
    tensor); ``W`` and ``act_absmax`` as for ``calibrate``."""
    W, wdt = _host_matrix(W, w_dtype)
    X, xdt = _host_matrix(X_cal, x_dtype)
    K, N = W.shape
    if X.ndim != 2 or X.shape[1] != K:
        raise ValueError(f"X_cal must be T x {K}")
    try:
        import torch
        if isinstance(act_absmax, torch.Tensor):
            act_absmax = act_absmax.float().numpy()
    except ImportError:  # pragma: no cover
        pass
    amax = np.ascontiguousarray(act_absmax, dtype=np.float32)
    if amax.shape != (K,):
        raise ValueError("act_absmax must have K entries")
    perm = np.empty(K, np.int32)
    shi = np.empty(K, np.float32)
    Wq = np.empty((N, K // 2), np.uint8)
    sw = np.empty(N, np.float32)
    Rq = np.zeros((N, rq_row_bytes(r)), np.uint8)
    sr = np.zeros(N, np.float32)
    check("serq_calibrate_gptq", lib.serq_calibrate_gptq(
        _ptr(W), wdt, K, N, _ptr(amax), float(alpha), r, _ptr(X), xdt, X.shape[0], float(damp), _ptr(perm),
        _ptr(shi), _ptr(Wq), _ptr(sw), _ptr(Rq) if r else None, _ptr(sr) if r else None))
    return SerqLayer(K=K, N=N, r=r, perm=perm, s_hat_inv=shi, Wq=Wq, sw=sw, Rq=Rq, sr=sr)


def permute_outputs(layer: SerqLayer, perm_next) -> SerqLayer:
    """Push the next layer's input order into this layer's output channels
    (serq_permute_outputs), in place on the host arrays; returns ``layer``."""
    p = np.ascontiguousarray(perm_next, dtype=np.int32)
    check("serq_permute_outputs",
          lib.serq_permute_outputs(_ptr(p), layer.K, layer.N, layer.r, _ptr(layer.Wq), _ptr(layer.sw),
                                   _ptr(layer.Rq) if layer.r else None, _ptr(layer.sr) if layer.r else None))
    return layer


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def _need_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("device tensors must be contiguous CUDA tensors")


def _act_out(out, M, K, a_bits, device):
    """The (xq, sx) buffers: new ones, or the caller's after checking that
    they are device tensors of exactly the sizes the kernels write."""
    import torch
    shape = (M, K // 2 if a_bits == 4 else K)
    if out is None:
        xq = torch.empty(shape, dtype=torch.uint8 if a_bits == 4 else torch.int8, device=device)
        return xq, torch.empty(M, dtype=torch.float32, device=device)
    xq, sx = out
    _need_cuda(xq, sx)
    if tuple(xq.shape) != shape or xq.element_size() != 1 or tuple(sx.shape) != (M,) or sx.dtype != torch.float32:
        raise ValueError(f"out must be (xq {shape} of 1-byte codes, sx ({M},) float32)")
    return xq, sx


def quant_act(x, layer_or_sinv, *, a_bits: int = 4, out=None):
    """Per-token activation quantization (serq_quant_act) on the current
    stream. ``x`` is M x K float32 or bfloat16, already in saliency order.
    Returns (xq, sx): uint8 M x K/2 (a_bits 4) or int8 M x K, float32 M."""
    import torch
    sinv = layer_or_sinv.s_hat_inv if isinstance(layer_or_sinv, DeviceLayer) else layer_or_sinv
    _need_cuda(x, sinv)
    M, K = x.shape
    if x.dtype == torch.bfloat16:
        dt = SERQ_BF16
    elif x.dtype == torch.float32:
        dt = SERQ_F32
    else:
        raise ValueError("x must be float32 or bfloat16")
    if sinv.numel() != K:
        raise ValueError(f"s_hat_inv has {sinv.numel()} entries for K = {K}")
    xq, sx = _act_out(out, M, K, a_bits, x.device)
    check("serq_quant_act", lib.serq_quant_act(x.data_ptr(), dt, M, K, sinv.data_ptr(), a_bits,
                                               xq.data_ptr(), sx.data_ptr(), _stream()))
    return xq, sx


def silu_mul_quant_act(g, u, layer_or_sinv, *, a_bits: int = 4, out=None):
    """The MLP step before down (serq_silu_mul_quant_act) on the current
    stream: quant_act(silu(g) * u). ``g`` and ``u`` are M x K float32 or
    bfloat16 views with the same row stride (e.g. the two halves of a gate/up
    output M x 2K), already in down's saliency order; ``layer_or_sinv`` is the
    down layer (or its s_hat_inv). Returns (xq, sx) as quant_act does."""
    import torch
    sinv = layer_or_sinv.s_hat_inv if isinstance(layer_or_sinv, DeviceLayer) else layer_or_sinv
    if g.dim() != 2 or g.shape != u.shape or g.dtype != u.dtype:
        raise ValueError("g and u must be M x K tensors of one dtype")
    M, K = g.shape
    if M > 1 and g.stride(0) != u.stride(0):
        raise ValueError("g and u must share their row stride")
    if (K > 1 and (g.stride(1) != 1 or u.stride(1) != 1)) or not g.is_cuda or not u.is_cuda:
        raise ValueError("g and u must be CUDA tensors with unit column stride")
    if not sinv.is_cuda or not sinv.is_contiguous():
        raise ValueError("s_hat_inv must be a contiguous CUDA tensor")
    if g.dtype == torch.bfloat16:
        dt = SERQ_BF16
    elif g.dtype == torch.float32:
        dt = SERQ_F32
    else:
        raise ValueError("g and u must be float32 or bfloat16")
    if sinv.numel() != K:
        raise ValueError(f"s_hat_inv has {sinv.numel()} entries for K = {K}")
    xq, sx = _act_out(out, M, K, a_bits, g.device)
    ld = g.stride(0) if M > 1 else K             # one row: the stride is never used
    check("serq_silu_mul_quant_act", lib.serq_silu_mul_quant_act(
        g.data_ptr(), u.data_ptr(), ld, dt, M, K, sinv.data_ptr(), a_bits, xq.data_ptr(), sx.data_ptr(), _stream()))
    return xq, sx


def linear(xq, sx, layer: DeviceLayer, *, a_bits: int = 4, out_dtype=None, out=None, debug: bool = False):
    """The SERQ linear (serq_linear) on the current stream. Returns Y (M x N)
    or, with ``debug=True``, (Y, acc_main, acc_res)."""
    import torch
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    _need_cuda(xq, sx, layer.Wq, layer.sw, layer.Rq if layer.r else None, layer.sr if layer.r else None)
    M = xq.shape[0]
    K, N, r = layer.K, layer.N, layer.r
    if xq.dim() != 2 or xq.shape[1] != (K // 2 if a_bits == 4 else K) or xq.element_size() != 1:
        raise ValueError(f"xq must be M x {K // 2 if a_bits == 4 else K} codes of one byte for this layer")
    if tuple(sx.shape) != (M,) or sx.dtype != torch.float32:
        raise ValueError(f"sx must be ({M},) float32")
    if out_dtype == torch.bfloat16:
        dt = SERQ_BF16
    elif out_dtype == torch.float32:
        dt = SERQ_F32
    else:
        raise ValueError("out_dtype must be float32 or bfloat16")
    if out is None:
        y = torch.empty((M, N), dtype=out_dtype, device=xq.device)
    else:
        y = out
        _need_cuda(y)
        if tuple(y.shape) != (M, N) or y.dtype != out_dtype:
            raise ValueError(f"out must be a ({M}, {N}) {out_dtype} tensor")
    am = ar = None
    if debug:
        am = torch.empty((M, N), dtype=torch.int32, device=xq.device)
        ar = torch.empty((M, N), dtype=torch.int32, device=xq.device)
    check("serq_linear", lib.serq_linear(
        xq.data_ptr(), sx.data_ptr(), a_bits, layer.Wq.data_ptr(), layer.sw.data_ptr(),
        layer.Rq.data_ptr() if r else None, layer.sr.data_ptr() if r else None, M, K, N, r,
        y.data_ptr(), dt, am.data_ptr() if debug else None, ar.data_ptr() if debug else None, _stream()))
    return (y, am, ar) if debug else y


def kernel_name(M: int, K: int, N: int, r: int, a_bits: int = 4) -> str | None:
    s = lib.serq_linear_kernel_name(M, K, N, r, a_bits)
    return s.decode() if s else None


# ------------------------------------------------------------------ bf6 route

def bf6_bytes(rows: int, k: int) -> int:
    """Bytes of a rows x k matrix in the bf6 tile layout (serq_bf6_bytes)."""
    b = lib.serq_bf6_bytes(int(rows), int(k))
    if b < 0:
        raise ValueError("rows and k must be >= 0")
    return b


@dataclass
class Bf6Layer:
    """A calibrated layer's weights in the bf6 tile layout (serq_prepack_bf6),
    host numpy arrays or, after ``to``, device tensors."""

    K: int
    N: int
    r: int
    W6: "object"            # bf6_bytes(N, K) uint8
    sw: "object"            # N float32
    R6: "object"            # bf6_bytes(N, r) uint8 (empty when r == 0)
    sr: "object"            # N float32

    def to(self, device="cuda") -> "Bf6Layer":
        import torch
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)  # noqa: E731
        return Bf6Layer(K=self.K, N=self.N, r=self.r, W6=t(self.W6), sw=t(self.sw), R6=t(self.R6), sr=t(self.sr))


def _prepack(codes: np.ndarray, rows: int, k: int, pitch: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    if codes.shape != (rows, pitch):
        raise ValueError(f"packed codes must be {rows} x {pitch} bytes")
    out = np.empty(bf6_bytes(rows, k), np.uint8)
    check("serq_prepack_bf6", lib.serq_prepack_bf6(_ptr(codes), rows, k, pitch, _ptr(out)))
    return out


def prepack_bf6(layer: SerqLayer) -> Bf6Layer:
    """Offline: Q(W^) and Q(R) of a host layer re-encoded as bf6 (host)."""
    W6 = _prepack(layer.Wq, layer.N, layer.K, layer.K // 2)
    R6 = _prepack(layer.Rq, layer.N, layer.r, rq_row_bytes(layer.r)) if layer.r else np.zeros(0, np.uint8)
    return Bf6Layer(K=layer.K, N=layer.N, r=layer.r, W6=W6, sw=np.asarray(layer.sw, np.float32), R6=R6,
                    sr=np.asarray(layer.sr, np.float32))


def act_bf6(xq, K: int, *, out=None):
    """W4A4 activation codes (quant_act's xq, M x K/2) re-encoded in the bf6
    tile layout on the current stream (serq_act_bf6). Returns a uint8 tensor
    of bf6_bytes(M, K) bytes."""
    import torch
    _need_cuda(xq)
    if xq.dim() != 2 or xq.shape[1] != K // 2 or xq.element_size() != 1:
        raise ValueError(f"xq must be M x {K // 2} packed int4 codes")
    M = xq.shape[0]
    n = bf6_bytes(M, K)
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device=xq.device)
    else:
        _need_cuda(out)
        if out.numel() != n or out.element_size() != 1:
            raise ValueError(f"out must hold {n} bytes")
    check("serq_act_bf6", lib.serq_act_bf6(xq.data_ptr(), M, K, out.data_ptr(), _stream()))
    return out


def linear_bf6(x6, sx, layer: Bf6Layer, *, out_dtype=None, out=None, debug: bool = False):
    """serq_linear_bf6 on the current stream: the W4A4 linear on bf6 operands
    (``x6`` from act_bf6, ``sx`` from quant_act). Returns Y (M x N) or, with
    ``debug=True``, (Y, acc_main, acc_res); bit-identical to ``linear``."""
    import torch
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    K, N, r = layer.K, layer.N, layer.r
    _need_cuda(x6, sx, layer.W6, layer.sw, layer.R6 if r else None, layer.sr if r else None)
    if sx.dim() != 1 or sx.dtype != torch.float32:
        raise ValueError("sx must be a float32 vector")
    M = sx.shape[0]
    if x6.numel() != bf6_bytes(M, K) or x6.element_size() != 1:
        raise ValueError(f"x6 must hold bf6_bytes({M}, {K}) bytes")
    if layer.W6.numel() != bf6_bytes(N, K) or (r and layer.R6.numel() != bf6_bytes(N, r)):
        raise ValueError("layer buffers do not match its sizes")
    if out_dtype == torch.bfloat16:
        dt = SERQ_BF16
    elif out_dtype == torch.float32:
        dt = SERQ_F32
    else:
        raise ValueError("out_dtype must be float32 or bfloat16")
    if out is None:
        y = torch.empty((M, N), dtype=out_dtype, device=x6.device)
    else:
        y = out
        _need_cuda(y)
        if tuple(y.shape) != (M, N) or y.dtype != out_dtype:
            raise ValueError(f"out must be a ({M}, {N}) {out_dtype} tensor")
    am = ar = None
    if debug:
        am = torch.empty((M, N), dtype=torch.int32, device=x6.device)
        ar = torch.empty((M, N), dtype=torch.int32, device=x6.device)
    check("serq_linear_bf6", lib.serq_linear_bf6(
        x6.data_ptr(), sx.data_ptr(), layer.W6.data_ptr(), layer.sw.data_ptr(),
        layer.R6.data_ptr() if r else None, layer.sr.data_ptr() if r else None, M, K, N, r,
        y.data_ptr(), dt, am.data_ptr() if debug else None, ar.data_ptr() if debug else None, _stream()))
    return (y, am, ar) if debug else y


def bf6_kernel_name(M: int, N: int, r: int = 0) -> str | None:
    """The tile serq_linear_bf6 launches for these sizes."""
    s = lib.serq_linear_bf6_kernel_name(M, N, r)
    return s.decode() if s else None


# ------------------------------------------------------------------ MXFP4

@dataclass
class MxLayer:
    """A layer calibrated for MXFP4 (serq_calibrate_mx): FP4 codes two per
    byte and one E8M0 exponent byte per 32 elements along K; host numpy
    arrays or, after ``to``, device tensors."""

    K: int
    N: int
    r: int
    perm: "object"          # K int32
    s_hat_inv: "object"     # K float32
    Wq: "object"            # N x K/2 uint8
    Wsc: "object"           # N x K/32 uint8
    Rq: "object"            # N x r/2 uint8
    Rsc: "object"           # N x r/32 uint8

    def to(self, device="cuda") -> "MxLayer":
        import torch
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)  # noqa: E731
        return MxLayer(K=self.K, N=self.N, r=self.r, perm=t(self.perm), s_hat_inv=t(self.s_hat_inv),
                       Wq=t(self.Wq), Wsc=t(self.Wsc), Rq=t(self.Rq), Rsc=t(self.Rsc))


def calibrate_mx(W, act_absmax, *, r: int, alpha: float = 0.5, w_dtype: str | None = None) -> MxLayer:
    """Offline MXFP4 calibration (serq_calibrate_mx); arguments as for
    ``calibrate``; K and r multiples of 32."""
    W, wdt = _host_matrix(W, w_dtype)
    K, N = W.shape
    amax = np.ascontiguousarray(act_absmax, dtype=np.float32)
    if amax.shape != (K,):
        raise ValueError("act_absmax must have K entries")
    perm = np.empty(K, np.int32)
    shi = np.empty(K, np.float32)
    Wq = np.empty((N, K // 2), np.uint8)
    Wsc = np.empty((N, K // 32), np.uint8)
    Rq = np.zeros((N, r // 2), np.uint8)
    Rsc = np.zeros((N, r // 32), np.uint8)
    check("serq_calibrate_mx", lib.serq_calibrate_mx(
        _ptr(W), wdt, K, N, _ptr(amax), float(alpha), r, _ptr(perm), _ptr(shi), _ptr(Wq), _ptr(Wsc),
        _ptr(Rq) if r else None, _ptr(Rsc) if r else None))
    return MxLayer(K=K, N=N, r=r, perm=perm, s_hat_inv=shi, Wq=Wq, Wsc=Wsc, Rq=Rq, Rsc=Rsc)


def quant_act_mx(x, layer_or_sinv, *, out=None):
    """MXFP4 activation quantization (serq_quant_act_mx) on the current
    stream: ``x`` M x K float32 or bfloat16 in saliency order. Returns
    (xq uint8 M x K/2, xsc uint8 M x K/32)."""
    import torch
    sinv = layer_or_sinv.s_hat_inv if isinstance(layer_or_sinv, MxLayer) else layer_or_sinv
    _need_cuda(x, sinv)
    M, K = x.shape
    if x.dtype == torch.bfloat16:
        dt = SERQ_BF16
    elif x.dtype == torch.float32:
        dt = SERQ_F32
    else:
        raise ValueError("x must be float32 or bfloat16")
    if sinv.numel() != K or K % 32:
        raise ValueError(f"s_hat_inv must have K = {K} entries and K a multiple of 32")
    if out is None:
        xq = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
        xsc = torch.empty((M, K // 32), dtype=torch.uint8, device=x.device)
    else:
        xq, xsc = out
        _need_cuda(xq, xsc)
        if tuple(xq.shape) != (M, K // 2) or tuple(xsc.shape) != (M, K // 32) or xq.element_size() != 1 \
                or xsc.element_size() != 1:
            raise ValueError(f"out must be (uint8 {M} x {K // 2}, uint8 {M} x {K // 32})")
    check("serq_quant_act_mx", lib.serq_quant_act_mx(x.data_ptr(), dt, M, K, sinv.data_ptr(), xq.data_ptr(),
                                                     xsc.data_ptr(), _stream()))
    return xq, xsc


def linear_mx(xq, xsc, layer: MxLayer, *, out_dtype=None, out=None, debug: bool = False):
    """The MXFP4 SERQ linear (serq_linear_mx) on the current stream. Returns
    Y (M x N) or, with ``debug=True``, (Y, acc_main, acc_res) in fp32."""
    import torch
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    K, N, r = layer.K, layer.N, layer.r
    _need_cuda(xq, xsc, layer.Wq, layer.Wsc, layer.Rq if r else None, layer.Rsc if r else None)
    M = xq.shape[0]
    if tuple(xq.shape) != (M, K // 2) or tuple(xsc.shape) != (M, K // 32):
        raise ValueError(f"xq, xsc must be M x {K // 2} and M x {K // 32} for this layer")
    if tuple(layer.Wq.shape) != (N, K // 2) or tuple(layer.Wsc.shape) != (N, K // 32):
        raise ValueError("layer buffers do not match its sizes")
    if out_dtype == torch.bfloat16:
        dt = SERQ_BF16
    elif out_dtype == torch.float32:
        dt = SERQ_F32
    else:
        raise ValueError("out_dtype must be float32 or bfloat16")
    if out is None:
        y = torch.empty((M, N), dtype=out_dtype, device=xq.device)
    else:
        y = out
        _need_cuda(y)
        if tuple(y.shape) != (M, N) or y.dtype != out_dtype:
            raise ValueError(f"out must be a ({M}, {N}) {out_dtype} tensor")
    am = ar = None
    if debug:
        am = torch.empty((M, N), dtype=torch.float32, device=xq.device)
        ar = torch.empty((M, N), dtype=torch.float32, device=xq.device)
    check("serq_linear_mx", lib.serq_linear_mx(
        xq.data_ptr(), xsc.data_ptr(), layer.Wq.data_ptr(), layer.Wsc.data_ptr(),
        layer.Rq.data_ptr() if r else None, layer.Rsc.data_ptr() if r else None, M, K, N, r, y.data_ptr(), dt,
        am.data_ptr() if debug else None, ar.data_ptr() if debug else None, _stream()))
    return (y, am, ar) if debug else y
