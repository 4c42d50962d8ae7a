"""ctypes declarations of libpisa's C ABI (include/pisa.h).

Loading is explicit and loud: if libpisa.so has not been built, every entry
point raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpisa.so")
PROBE_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpisa_probe.so")

PISA_OK = 0
STATUS_NAMES = {0: "PISA_OK", 1: "PISA_ERR_NULL", 2: "PISA_ERR_SHAPE", 3: "PISA_ERR_ARG",
                4: "PISA_ERR_DTYPE", 5: "PISA_ERR_WORKSPACE", 6: "PISA_ERR_HIP"}
DTYPE_BF16 = 0
DTYPE_FP32 = 1
MODE_APPROX = 0
MODE_DROP = 1
MODE_ZEROTH = 2
MODE_FIRST = 3
ROUTE_AUTO = 0
ROUTE_IN_KERNEL = 1
ROUTE_TWO_LAUNCH = 2
NORM_FROBENIUS = 0
NORM_SPECTRAL = 1

# every symbol the header declares
EXPORTS = ("pisa_version", "pisa_status_string", "pisa_last_error", "pisa_workspace_size",
           "pisa_packed_size", "pisa_precompute", "pisa_precompute_noalloc", "pisa_route",
           "pisa_attention", "pisa_attention_split_workspace_size", "pisa_attention_split",
           "pisa_route_attention")
# ... and every symbol include/pisa_probe.h declares (libpisa_probe.so)
PROBE_EXPORTS = ("pisa_probe_chunk_rate", "pisa_probe_read_rate")


class PisaShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("seq_lens", ctypes.c_void_p)]


class PisaStats(ctypes.Structure):
    _fields_ = [("centroid", ctypes.c_void_p), ("vsum", ctypes.c_void_p), ("H", ctypes.c_void_p),
                ("Hbar", ctypes.c_void_p), ("M", ctypes.c_void_p), ("packed", ctypes.c_void_p),
                ("Ht", ctypes.c_void_p), ("m_norm", ctypes.c_int32)]


class PisaError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        self.status = status
        super().__init__(f"{fn} -> {STATUS_NAMES.get(status, status)}: {detail}")


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpisa.so once and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m piecewise_block_sparse_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    sp, stp = ctypes.POINTER(PisaShape), ctypes.POINTER(PisaStats)
    lib.pisa_version.restype = i32
    lib.pisa_version.argtypes = []
    lib.pisa_status_string.restype = ctypes.c_char_p
    lib.pisa_status_string.argtypes = [i32]
    lib.pisa_last_error.restype = ctypes.c_char_p
    lib.pisa_last_error.argtypes = []
    lib.pisa_workspace_size.restype = sz
    lib.pisa_workspace_size.argtypes = [sp]
    lib.pisa_packed_size.restype = sz
    lib.pisa_packed_size.argtypes = [sp]
    lib.pisa_precompute.restype = i32
    lib.pisa_precompute.argtypes = [sp, vp, vp, stp, vp, sz, vp]
    lib.pisa_precompute_noalloc.restype = i32
    lib.pisa_precompute_noalloc.argtypes = [sp, vp, vp, stp, vp]
    lib.pisa_route.restype = i32
    lib.pisa_route.argtypes = [sp, vp, vp, vp, i32, ctypes.c_double, ctypes.c_double, vp, vp]
    lib.pisa_attention.restype = i32
    lib.pisa_attention.argtypes = [sp, vp, vp, vp, vp, i32, stp, i32, ctypes.c_float, vp, vp]
    lib.pisa_attention_split_workspace_size.restype = sz
    lib.pisa_attention_split_workspace_size.argtypes = [sp, i32, i32]
    lib.pisa_attention_split.restype = i32
    lib.pisa_attention_split.argtypes = [sp, vp, vp, vp, vp, i32, stp, i32, ctypes.c_float, i32, vp,
                                         vp, sz, vp]
    lib.pisa_route_attention.restype = i32
    lib.pisa_route_attention.argtypes = [sp, vp, vp, vp, stp, i32, ctypes.c_double, i32,
                                         ctypes.c_double, vp, vp, i32, vp]
    _lib = lib
    return lib


def check(fn: str, status: int) -> None:
    if status != PISA_OK:
        raise PisaError(fn, status, load().pisa_last_error().decode())


def load_probe(path: str = PROBE_PATH) -> ctypes.CDLL:
    """Load the measurement probe library (include/pisa_probe.h)."""
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m piecewise_block_sparse_amd.build`")
    lib = ctypes.CDLL(path)
    lib.pisa_probe_chunk_rate.restype = ctypes.c_int
    lib.pisa_probe_chunk_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.POINTER(ctypes.c_double)]
    lib.pisa_probe_read_rate.restype = ctypes.c_int
    lib.pisa_probe_read_rate.argtypes = [ctypes.c_size_t, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    return lib
