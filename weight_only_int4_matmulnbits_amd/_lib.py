"""ctypes loader for libmnb.so (the C ABI declared in include/mnb.h).

torch is imported first so that the HIP runtime torch loaded is the one the
library binds to (both carry the soname libamdhip64.so.7); after loading, the
process maps are checked for a second runtime.  There is no fallback: without
the compiled library every call raises.
"""

from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  -- must precede the library load (HIP runtime)

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmnb.so")

MNB_OK = 0
STATUS_NAMES = {0: "MNB_OK", -1: "MNB_E_ARG", -2: "MNB_E_UNSUPPORTED",
                -3: "MNB_E_ALIGN", -4: "MNB_E_OVERFLOW", -5: "MNB_E_HIP"}
F32, BF16 = 0, 1

# every symbol include/mnb.h declares
EXPORTS = (
    "mnb_validate", "mnb_packed_weight_bytes", "mnb_scale_bytes",
    "mnb_zero_point_bytes", "mnb_gemv_max_k", "mnb_pack", "mnb_gemv",
    "mnb_gemm", "mnb_dequant", "mnb_matmul_sequence", "mnb_graph_create",
    "mnb_graph_launch", "mnb_graph_destroy", "mnb_status_string",
    "mnb_last_error", "mnb_version", "mnb_import_qdq", "mnb_qdq_is_native",
    "mnb_gather_rows", "mnb_argmax", "mnb_gemv_silu_mul",
    "mnb_workspace_bytes", "mnb_argmax_workspace_bytes",
    "mnb_sequence_workspace_bytes", "mnb_gemm_noalloc",
    "mnb_gemm_silu_workspace_bytes", "mnb_gemm_silu_mul", "mnb_gemv_rmsnorm",
    "mnb_step_workspace_bytes", "mnb_step_create", "mnb_step_launch", "mnb_step_check",
    "mnb_step_destroy", "mnb_step_trace_bytes", "mnb_step_set_trace",
)


class Desc(ctypes.Structure):
    """mnb_desc."""
    _fields_ = [("K", ctypes.c_int64), ("N", ctypes.c_int64),
                ("bits", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32),
                ("has_zero_points", ctypes.c_int32),
                ("accuracy_level", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class MatmulArgs(ctypes.Structure):
    """mnb_matmul_args."""
    _fields_ = [("desc", Desc), ("M", ctypes.c_int64),
                ("a", ctypes.c_void_p), ("b_packed", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("zp_packed", ctypes.c_void_p),
                ("bias", ctypes.c_void_p), ("y", ctypes.c_void_p)]


class MnbError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {detail}")


_lib = None


def _hip_runtimes_mapped():
    try:
        with open("/proc/self/maps") as f:
            paths = {line.split()[-1] for line in f if "libamdhip64" in line}
    except OSError:
        return set()
    return {p for p in paths if p.startswith("/")}


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it was never built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: the HIP library must be built first "
            "(python -c 'import __graft_entry__ as g; g.build()'); there is "
            "no CPU fallback")
    L = ctypes.CDLL(LIB_PATH)
    missing = [s for s in EXPORTS if not hasattr(L, s)]
    if missing:
        raise RuntimeError(f"{LIB_PATH} lacks symbols {missing}")
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise RuntimeError(f"two HIP runtimes are mapped: {sorted(runtimes)}")
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    pd = ctypes.POINTER(Desc)
    L.mnb_validate.argtypes = [pd, i64]
    L.mnb_validate.restype = ctypes.c_int
    for f in ("mnb_packed_weight_bytes", "mnb_scale_bytes", "mnb_zero_point_bytes"):
        getattr(L, f).argtypes = [pd]
        getattr(L, f).restype = ctypes.c_size_t
    L.mnb_gemv_max_k.argtypes = [pd]
    L.mnb_gemv_max_k.restype = i64
    L.mnb_pack.argtypes = [pd, vp, vp, vp, vp, vp]
    L.mnb_pack.restype = ctypes.c_int
    sz = ctypes.c_size_t
    L.mnb_gemv.argtypes = [pd, i64, vp, vp, vp, vp, vp, vp, vp]
    L.mnb_gemv.restype = ctypes.c_int
    L.mnb_gemm.argtypes = [pd, i64, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.mnb_gemm.restype = ctypes.c_int
    L.mnb_gemm_noalloc.argtypes = [pd, i64, vp, vp, vp, vp, vp, vp, vp]
    L.mnb_gemm_noalloc.restype = ctypes.c_int
    L.mnb_workspace_bytes.argtypes = [pd, i64]
    L.mnb_workspace_bytes.restype = sz
    L.mnb_argmax_workspace_bytes.argtypes = [i64, i64]
    L.mnb_argmax_workspace_bytes.restype = sz
    L.mnb_dequant.argtypes = [pd, vp, vp, vp, i32, vp, vp]
    L.mnb_dequant.restype = ctypes.c_int
    L.mnb_import_qdq.argtypes = [pd, i32, vp, vp, vp, vp, vp, vp, vp]
    L.mnb_import_qdq.restype = ctypes.c_int
    L.mnb_qdq_is_native.argtypes = [pd, i32]
    L.mnb_qdq_is_native.restype = ctypes.c_int
    L.mnb_gather_rows.argtypes = [pd, vp, i64, vp, vp, vp, vp, vp]
    L.mnb_gather_rows.restype = ctypes.c_int
    L.mnb_argmax.argtypes = [i32, i64, i64, vp, vp, vp, sz, vp]
    L.mnb_argmax.restype = ctypes.c_int
    L.mnb_gemv_silu_mul.argtypes = [pd, i64, vp, vp, vp, vp, vp, vp, vp]
    L.mnb_gemv_silu_mul.restype = ctypes.c_int
    L.mnb_gemm_silu_workspace_bytes.argtypes = [pd, i64]
    L.mnb_gemm_silu_workspace_bytes.restype = sz
    L.mnb_gemm_silu_mul.argtypes = [pd, i64, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.mnb_gemm_silu_mul.restype = ctypes.c_int
    L.mnb_gemv_rmsnorm.argtypes = [pd, i64, vp, vp, ctypes.c_float, vp, vp, vp, vp, vp, vp]
    L.mnb_gemv_rmsnorm.restype = ctypes.c_int
    pa = ctypes.POINTER(MatmulArgs)
    L.mnb_sequence_workspace_bytes.argtypes = [pa, i64]
    L.mnb_sequence_workspace_bytes.restype = sz
    L.mnb_matmul_sequence.argtypes = [pa, i64, vp, sz, vp]
    L.mnb_matmul_sequence.restype = ctypes.c_int
    L.mnb_graph_create.argtypes = [pa, i64, vp, sz, ctypes.POINTER(vp)]
    L.mnb_graph_create.restype = ctypes.c_int
    L.mnb_graph_launch.argtypes = [vp, vp]
    L.mnb_graph_launch.restype = ctypes.c_int
    L.mnb_graph_destroy.argtypes = [vp]
    L.mnb_graph_destroy.restype = ctypes.c_int
    L.mnb_step_workspace_bytes.argtypes = [pa, i64]
    L.mnb_step_workspace_bytes.restype = sz
    L.mnb_step_create.argtypes = [pa, i64, vp, sz, ctypes.POINTER(vp)]
    L.mnb_step_create.restype = ctypes.c_int
    for f in ("mnb_step_launch", "mnb_step_check"):
        getattr(L, f).argtypes = [vp, vp]
        getattr(L, f).restype = ctypes.c_int
    L.mnb_step_destroy.argtypes = [vp]
    L.mnb_step_destroy.restype = ctypes.c_int
    L.mnb_step_trace_bytes.argtypes = [vp]
    L.mnb_step_trace_bytes.restype = sz
    L.mnb_step_set_trace.argtypes = [vp, vp, sz]
    L.mnb_step_set_trace.restype = ctypes.c_int
    for f in ("mnb_status_string",):
        getattr(L, f).argtypes = [ctypes.c_int]
        getattr(L, f).restype = ctypes.c_char_p
    for f in ("mnb_last_error", "mnb_version"):
        getattr(L, f).argtypes = []
        getattr(L, f).restype = ctypes.c_char_p
    _lib = L
    return L


def check(status: int, where: str) -> None:
    if status != MNB_OK:
        detail = lib().mnb_last_error().decode(errors="replace")
        raise MnbError(status, where, detail)
