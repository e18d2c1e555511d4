"""ctypes binding to libserq.so (include/serq.h).

Loads the in-tree library and declares the C signatures. There is no
fallback: if the library is missing or cannot be loaded, importing the
package raises, so nothing can silently run on the CPU instead of the HIP
kernels.
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("SERQ_LIB", os.path.join(PKG, "libserq.so"))

SERQ_OK, SERQ_EINVAL, SERQ_EALIGN, SERQ_EUNSUPPORTED, SERQ_EHIP = 0, -1, -2, -3, -4
SERQ_F32, SERQ_BF16 = 0, 1

# every symbol include/serq.h declares
EXPORTS = ("serq_strerror", "serq_abi_version", "serq_calibrate", "serq_calibrate_gptq", "serq_permute_outputs",
           "serq_quant_act", "serq_silu_mul_quant_act", "serq_linear", "serq_linear_kernel_name",
           "serq_rq_row_bytes", "serq_bf6_bytes", "serq_prepack_bf6", "serq_act_bf6", "serq_linear_bf6",
           "serq_linear_bf6_kernel_name", "serq_calibrate_mx", "serq_quant_act_mx", "serq_linear_mx")


class SerqError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg} ({status})")
        self.status = status


def _load() -> ctypes.CDLL:
    # libserq.so needs libamdhip64.so.7. PyTorch ships its own HIP runtime
    # under that soname; if torch is imported first the library binds to that
    # same runtime, otherwise a second runtime would be loaded next to torch's
    # and the two would not share devices, streams or allocations.
    try:
        import torch  # noqa: F401
    except ImportError:  # pragma: no cover - library use without PyTorch
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libserq.so not found at {LIB_PATH}; build it with "
                          f"`python w4a4_linear_layers_amd/build.py` (or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    vp, ip, fp, i32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_int
    lib.serq_strerror.argtypes = [ip]
    lib.serq_strerror.restype = ctypes.c_char_p
    lib.serq_abi_version.argtypes = []
    lib.serq_abi_version.restype = ip
    lib.serq_calibrate.argtypes = [vp, i32, ip, ip, vp, fp, ip, vp, vp, vp, vp, vp, vp]
    lib.serq_calibrate.restype = ip
    lib.serq_calibrate_gptq.argtypes = [vp, i32, ip, ip, vp, fp, ip, vp, i32, ip, fp, vp, vp, vp, vp, vp, vp]
    lib.serq_calibrate_gptq.restype = ip
    lib.serq_permute_outputs.argtypes = [vp, ip, ip, ip, vp, vp, vp, vp]
    lib.serq_permute_outputs.restype = ip
    lib.serq_quant_act.argtypes = [vp, i32, ip, ip, vp, ip, vp, vp, vp]
    lib.serq_quant_act.restype = ip
    lib.serq_silu_mul_quant_act.argtypes = [vp, vp, ip, i32, ip, ip, vp, ip, vp, vp, vp]
    lib.serq_silu_mul_quant_act.restype = ip
    lib.serq_linear.argtypes = [vp, vp, ip, vp, vp, vp, vp, ip, ip, ip, ip, vp, i32, vp, vp, vp]
    lib.serq_linear.restype = ip
    lib.serq_linear_kernel_name.argtypes = [ip, ip, ip, ip, ip]
    lib.serq_linear_kernel_name.restype = ctypes.c_char_p
    lib.serq_rq_row_bytes.argtypes = [ip]
    lib.serq_rq_row_bytes.restype = ip
    lib.serq_bf6_bytes.argtypes = [ip, ip]
    lib.serq_bf6_bytes.restype = ctypes.c_int64
    lib.serq_prepack_bf6.argtypes = [vp, ip, ip, ip, vp]
    lib.serq_prepack_bf6.restype = ip
    lib.serq_act_bf6.argtypes = [vp, ip, ip, vp, vp]
    lib.serq_act_bf6.restype = ip
    lib.serq_linear_bf6.argtypes = [vp, vp, vp, vp, vp, vp, ip, ip, ip, ip, vp, i32, vp, vp, vp]
    lib.serq_linear_bf6.restype = ip
    lib.serq_linear_bf6_kernel_name.argtypes = [ip, ip, ip]
    lib.serq_linear_bf6_kernel_name.restype = ctypes.c_char_p
    lib.serq_calibrate_mx.argtypes = [vp, i32, ip, ip, vp, fp, ip, vp, vp, vp, vp, vp, vp]
    lib.serq_calibrate_mx.restype = ip
    lib.serq_quant_act_mx.argtypes = [vp, i32, ip, ip, vp, vp, vp, vp]
    lib.serq_quant_act_mx.restype = ip
    lib.serq_linear_mx.argtypes = [vp, vp, vp, vp, vp, vp, ip, ip, ip, ip, vp, i32, vp, vp, vp]
    lib.serq_linear_mx.restype = ip
    return lib


lib = _load()


def check(fn: str, status: int) -> None:
    if status != SERQ_OK:
        raise SerqError(fn, status, lib.serq_strerror(status).decode())
