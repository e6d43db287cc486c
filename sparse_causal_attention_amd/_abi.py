"""ctypes declarations of the C ABI in include/sa.h (argument marshalling only).

Loads the in-tree libsa.so.  There is no fallback: if the library has not
been built, importing the functions that need it raises with the command that
builds it.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; SA_LIBRARY names another build of the same sources (for
# comparing two builds in one process tree on one GPU)
LIB_PATH = os.environ.get("SA_LIBRARY") or os.path.join(_PKG, "libsa.so")

SA_OK, SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED, SA_ERR_SHAPE_MISMATCH, SA_ERR_WORKSPACE, SA_ERR_HIP = range(6)
SA_F32, SA_BF16 = 0, 1
SA_SCORE_DOT, SA_SCORE_COORD, SA_SCORE_UNIFORM = 0, 1, 2
SA_ALGO_AUTO, SA_ALGO_GATHER, SA_ALGO_BAND = 0, 1, 2
SA_GRAPH_DISTANCE, SA_GRAPH_CSR = 0, 1
SA_MAX_DILATED = 64
SA_NOALLOC_SCRATCH_BYTES = 16 << 20

i64 = ctypes.c_int64
i32 = ctypes.c_int32
vp = ctypes.c_void_p


class SaAttnDesc(ctypes.Structure):
    _fields_ = [
        ("B", i64), ("H", i64), ("T", i64), ("D", i64),
        ("dtype", i32), ("grad_dtype", i32), ("score", i32), ("algo", i32),
        ("scale", ctypes.c_float),
        ("stride_q", i64 * 3), ("stride_k", i64 * 3), ("stride_v", i64 * 3),
        ("stride_o", i64 * 3), ("stride_do", i64 * 3),
        ("stride_dq", i64 * 3), ("stride_dk", i64 * 3), ("stride_dv", i64 * 3),
        ("H_kv", i64),
    ]


EXPORTED = (
    "sa_build_graph", "sa_build_graph_csr", "sa_graph_kind", "sa_graph_device_bytes", "sa_graph_upload",
    "sa_graph_info", "sa_graph_rows", "sa_graph_rows_reverse", "sa_graph_free",
    "sa_fwd", "sa_bwd_workspace_size", "sa_bwd", "sa_bwd_noalloc", "sa_decode", "sa_describe_plan",
    "sa_status_str",
)

_lib = None


class SaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().sa_status_str(status).decode() if _lib is not None else str(status)
        super().__init__("%s: %s (status %d)" % (where, msg, status))


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            "libsa.so is not built (expected at %s); run "
            "`python -m sparse_causal_attention_amd.build` first" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    L.sa_build_graph.restype = i32
    L.sa_build_graph.argtypes = [i64, i64, vp, i32, ctypes.POINTER(vp)]
    L.sa_build_graph_csr.restype = i32
    L.sa_build_graph_csr.argtypes = [i64, vp, vp, ctypes.POINTER(vp)]
    L.sa_graph_kind.restype = i32
    L.sa_graph_kind.argtypes = [vp, ctypes.POINTER(i32)]
    L.sa_graph_device_bytes.restype = i32
    L.sa_graph_device_bytes.argtypes = [vp, ctypes.POINTER(ctypes.c_size_t)]
    L.sa_graph_upload.restype = i32
    L.sa_graph_upload.argtypes = [vp, vp, ctypes.c_size_t, vp]
    L.sa_graph_info.restype = i32
    L.sa_graph_info.argtypes = [vp, vp, vp, vp, vp, vp]
    L.sa_graph_rows.restype = i32
    L.sa_graph_rows.argtypes = [vp, i64, i64, vp, vp, i64]
    L.sa_graph_rows_reverse.restype = i32
    L.sa_graph_rows_reverse.argtypes = [vp, i64, i64, vp, vp, i64]
    L.sa_graph_free.restype = None
    L.sa_graph_free.argtypes = [vp]
    L.sa_fwd.restype = i32
    L.sa_fwd.argtypes = [vp, ctypes.POINTER(SaAttnDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.sa_bwd_workspace_size.restype = i32
    L.sa_bwd_workspace_size.argtypes = [vp, ctypes.POINTER(SaAttnDesc), ctypes.POINTER(ctypes.c_size_t)]
    L.sa_bwd.restype = i32
    L.sa_bwd.argtypes = [vp, ctypes.POINTER(SaAttnDesc)] + [vp] * 17 + [vp, ctypes.c_size_t, vp]
    L.sa_bwd_noalloc.restype = i32
    L.sa_bwd_noalloc.argtypes = [vp, ctypes.POINTER(SaAttnDesc)] + [vp] * 17 + [vp]
    L.sa_decode.restype = i32
    L.sa_decode.argtypes = [vp, ctypes.POINTER(SaAttnDesc)] + [vp] * 11
    L.sa_describe_plan.restype = i32
    L.sa_describe_plan.argtypes = [vp, ctypes.POINTER(SaAttnDesc), i32, ctypes.c_char_p, ctypes.c_size_t]
    L.sa_status_str.restype = ctypes.c_char_p
    L.sa_status_str.argtypes = [i32]
    _lib = L
    return L


def check(status: int, where: str):
    if status != SA_OK:
        raise SaError(status, where)
