"""ctypes loader for libqaff.so (the C ABI of include/qaff.h). Nothing here computes: it finds the
library, declares the signatures and turns a non-OK status into an exception."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqaff.so")

QAFF_OK = 0
QAFF_ERR_INVALID_ARGUMENT = 1
QAFF_ERR_UNSUPPORTED = 2
QAFF_ERR_DEVICE = 3

QAFF_F32 = 0
QAFF_BF16 = 1
QAFF_F16 = 2

PATHS = {"auto": 0, "gemv": 1, "gemm": 2, "gemv_mfma": 3}

EXPORTS = ("qaff_dequantize", "qaff_qmm", "qaff_qmm_ex", "qaff_dequant_rows", "qaff_last_error",
           "qaff_status_string", "qaff_abi_version", "qaff_gemv_max_m", "qaff_gemv_mfma_min_m",
           "qaff_gemv_gate_up", "qaff_gemv_silu_gate", "qaff_gather_qmm", "qaff_gather_qmm_ex",
           "qaff_quantize", "qaff_qmm_nt", "qaff_qmm_nt_workspace_size", "qaff_qmm_nt_static",
           "qaff_qmm_nt_static_max_bytes", "qaff_qmm_ws", "qaff_qmm_workspace_size",
           "qaff_promote_dtype",
           "qaff_dequantize_typed", "qaff_qmm_typed", "qaff_quantize_typed", "qaff_gather_qmm_typed",
           "qaff_qmm_nt_typed")

ABI_VERSION = 1


class QaffError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Loads the in-tree libqaff.so. Raises if it is not built: there is no fallback path."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m quantized_matmul_mlx_amd.build` "
                           "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.qaff_dequantize.argtypes = [vp, vp, vp, i64, i64, i32, i32, vp, ctypes.c_int, vp]
    lib.qaff_qmm.argtypes = [vp, ctypes.c_int, i64, vp, vp, vp, i64, i64, i32, i32, vp, vp]
    lib.qaff_qmm_ex.argtypes = [vp, ctypes.c_int, i64, vp, vp, vp, i64, i64, i32, i32, vp, vp,
                                ctypes.c_int]
    lib.qaff_dequant_rows.argtypes = [vp, vp, vp, i64, i64, i32, i32, vp, i64, vp, ctypes.c_int, vp]
    lib.qaff_gemv_gate_up.argtypes = [vp, i64, vp, vp, vp, vp, vp, vp, i64, i64, i32, i32, vp, vp, vp]
    lib.qaff_gemv_silu_gate.argtypes = [vp, vp, i64, vp, vp, vp, i64, i64, i32, i32, vp, vp, vp]
    gather = [vp, ctypes.c_int, i64, i64, vp, vp, vp, i64, i64, i64, i32, i32, vp, vp, i64, i32, vp, vp]
    lib.qaff_promote_dtype.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.qaff_promote_dtype.restype = ctypes.c_int
    lib.qaff_dequantize_typed.argtypes = [vp, vp, vp, ctypes.c_int, i64, i64, i32, i32, vp, ctypes.c_int, vp]
    lib.qaff_qmm_typed.argtypes = [vp, ctypes.c_int, i64, vp, vp, vp, ctypes.c_int, i64, i64, i32, i32, vp, vp]
    lib.qaff_qmm_nt.argtypes = [vp, ctypes.c_int, i64, vp, vp, vp, i64, i64, i32, i32, vp, ctypes.c_size_t, vp, vp]
    lib.qaff_qmm_nt_static.argtypes = [vp, ctypes.c_int, i64, vp, vp, vp, i64, i64, i32, i32, vp, vp]
    lib.qaff_qmm_nt_typed.argtypes = [vp, ctypes.c_int, i64, vp, vp, vp, ctypes.c_int, i64, i64, i32, i32, vp,
                                      ctypes.c_size_t, vp, vp]
    lib.qaff_qmm_nt_static_max_bytes.argtypes = []
    lib.qaff_qmm_nt_static_max_bytes.restype = ctypes.c_size_t
    lib.qaff_qmm_nt_workspace_size.argtypes = [i64, i64, i64, i32]
    lib.qaff_qmm_nt_workspace_size.restype = ctypes.c_size_t
    lib.qaff_qmm_ws.argtypes = [vp, ctypes.c_int, i64, vp, vp, vp, i64, i64, i32, i32, vp, ctypes.c_size_t, vp, vp]
    lib.qaff_qmm_workspace_size.argtypes = [i64, i64, i64, i32, i32]
    lib.qaff_qmm_workspace_size.restype = ctypes.c_size_t
    lib.qaff_quantize.argtypes = [vp, ctypes.c_int, i64, i64, i32, i32, vp, vp, vp, vp]
    lib.qaff_quantize_typed.argtypes = [vp, ctypes.c_int, i64, i64, i32, i32, vp, vp, vp, ctypes.c_int, vp]
    lib.qaff_gather_qmm.argtypes = gather
    lib.qaff_gather_qmm_ex.argtypes = gather + [ctypes.c_int]
    lib.qaff_gather_qmm_typed.argtypes = [vp, ctypes.c_int, i64, i64, vp, vp, vp, ctypes.c_int, i64, i64, i64, i32,
                                          i32, vp, vp, i64, i32, vp, vp]
    for f in (lib.qaff_dequantize, lib.qaff_qmm, lib.qaff_qmm_ex, lib.qaff_dequant_rows,
              lib.qaff_gemv_gate_up, lib.qaff_gemv_silu_gate, lib.qaff_gather_qmm, lib.qaff_gather_qmm_ex,
              lib.qaff_gather_qmm_typed,
              lib.qaff_quantize, lib.qaff_quantize_typed, lib.qaff_qmm_nt, lib.qaff_qmm_nt_static,
              lib.qaff_qmm_nt_typed, lib.qaff_dequantize_typed, lib.qaff_qmm_typed, lib.qaff_qmm_ws):
        f.restype = ctypes.c_int
    lib.qaff_last_error.restype = ctypes.c_char_p
    lib.qaff_last_error.argtypes = []
    lib.qaff_status_string.restype = ctypes.c_char_p
    lib.qaff_status_string.argtypes = [ctypes.c_int]
    lib.qaff_abi_version.restype = ctypes.c_int
    lib.qaff_gemv_max_m.restype = ctypes.c_int
    lib.qaff_gemv_mfma_min_m.restype = ctypes.c_int
    if lib.qaff_abi_version() != ABI_VERSION:
        raise RuntimeError(f"libqaff ABI {lib.qaff_abi_version()} != expected {ABI_VERSION}")
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != QAFF_OK:
        lib = load()
        name = lib.qaff_status_string(status).decode()
        raise QaffError(status, f"{name}: {lib.qaff_last_error().decode()}")
