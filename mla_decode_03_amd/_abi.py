"""ctypes declarations of the libmla.so C ABI (include/mla.h).  No compute here."""
from __future__ import annotations

import ctypes
import os

D_QK = 576
D_V = 512
PAGE = 64
MAX_ROWS = 128
DTYPE_F32 = 0
DTYPE_BF16 = 1

MLA_OK = 0
MLA_ERR_NULL = 1
MLA_ERR_SHAPE = 2
MLA_ERR_DTYPE = 3
MLA_ERR_ALIGN = 4
MLA_ERR_WORKSPACE = 5
MLA_ERR_UNSUPPORTED = 6
MLA_ERR_LAUNCH = 7
MLA_ERR_DEVICE = 8
MLA_ERR_BAD_INPUT = 9

# Exported functions, as declared in include/mla.h.
EXPORTS = ("mla_status_string", "mla_device_num_cus", "mla_metadata_bytes", "mla_workspace_bytes",
           "mla_get_metadata", "mla_decode", "mla_decode_ex", "mla_decode_splits", "mla_decode_splits_timed", "mla_combine",
           "mla_plan_error", "mla_hbm_read_probe", "mla_decode_noalloc")

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmla.so")
_lib = None


class MlaError(RuntimeError):
    def __init__(self, code: int, what: str = ""):
        self.code = int(code)
        msg = status_string(code) if _lib is not None else "status %d" % code
        super().__init__("%s: %s (%d)" % (what, msg, code) if what else "%s (%d)" % (msg, code))


class Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("q_len", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("block_table_stride", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("topk", ctypes.c_int32)]


class PlanOptions(ctypes.Structure):
    _fields_ = [("num_workgroups", ctypes.c_int32), ("min_blocks_per_wg", ctypes.c_int32),
                ("row_split", ctypes.c_int32), ("fixed_split_blocks", ctypes.c_int32),
                ("split_rule", ctypes.c_int32), ("segment_cost", ctypes.c_int32),
                ("plan_in_decode", ctypes.c_int32)]


class Variant(ctypes.Structure):
    _fields_ = [("sinks", ctypes.c_void_p), ("indices", ctypes.c_void_p)]


class CPlan(ctypes.Structure):
    _fields_ = [("metadata", ctypes.c_void_p), ("metadata_bytes", ctypes.c_size_t),
                ("grid_wg", ctypes.c_int32), ("row_split", ctypes.c_int32),
                ("rows_per_wg", ctypes.c_int32), ("max_partials", ctypes.c_int32),
                ("batch", ctypes.c_int32), ("rows", ctypes.c_int32),
                ("plan_in_decode", ctypes.c_int32), ("min_blocks", ctypes.c_int32),
                ("fixed_blocks", ctypes.c_int32), ("split_rule", ctypes.c_int32),
                ("segment_cost", ctypes.c_int32), ("topk", ctypes.c_int32)]


def lib_path() -> str:
    return _LIB_PATH


def lib():
    """Load libmla.so (built in-tree).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("libmla.so not found at %s: build it with `python -m mla_decode_03_amd.build` "
                               "(the decode has no fallback path)" % _LIB_PATH)
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.mla_status_string.restype = ctypes.c_char_p
        L.mla_status_string.argtypes = [i32]
        L.mla_device_num_cus.restype = i32
        L.mla_device_num_cus.argtypes = [ctypes.POINTER(i32)]
        L.mla_metadata_bytes.restype = sz
        L.mla_metadata_bytes.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(PlanOptions), i32]
        L.mla_workspace_bytes.restype = sz
        L.mla_workspace_bytes.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(PlanOptions), i32]
        L.mla_get_metadata.restype = i32
        L.mla_get_metadata.argtypes = [ctypes.POINTER(Problem), vp, ctypes.POINTER(PlanOptions), i32,
                                       ctypes.POINTER(CPlan), vp]
        L.mla_decode.restype = i32
        L.mla_decode.argtypes = [ctypes.POINTER(Problem), vp, vp, vp, vp, ctypes.c_float, vp, vp,
                                 ctypes.POINTER(CPlan), vp, sz, vp]
        V = ctypes.POINTER(Variant)
        L.mla_decode_ex.restype = i32
        L.mla_decode_ex.argtypes = [ctypes.POINTER(Problem), V, vp, vp, vp, vp, ctypes.c_float, vp, vp,
                                    ctypes.POINTER(CPlan), vp, sz, vp]
        L.mla_decode_splits.restype = i32
        L.mla_decode_splits.argtypes = [ctypes.POINTER(Problem), V, vp, vp, vp, vp, ctypes.c_float, vp, vp,
                                        ctypes.POINTER(CPlan), vp, sz, vp]
        L.mla_decode_splits_timed.restype = i32
        L.mla_decode_splits_timed.argtypes = [ctypes.POINTER(Problem), V, vp, vp, vp, vp, ctypes.c_float, vp,
                                              vp, ctypes.POINTER(CPlan), vp, sz, vp, vp, vp]
        L.mla_combine.restype = i32
        L.mla_combine.argtypes = [ctypes.POINTER(Problem), V, vp, vp, ctypes.POINTER(CPlan), vp, sz, vp]
        L.mla_plan_error.restype = i32
        L.mla_plan_error.argtypes = [ctypes.POINTER(CPlan), vp]
        L.mla_decode_noalloc.restype = i32
        L.mla_decode_noalloc.argtypes = [ctypes.POINTER(Problem), V, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp]
        L.mla_hbm_read_probe.restype = i32
        L.mla_hbm_read_probe.argtypes = [vp, sz, i32, i32, vp, vp]
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().mla_status_string(int(code)).decode()


def check(rc: int, what: str) -> None:
    if rc != MLA_OK:
        raise MlaError(rc, what)


def opt_ref(options):
    return ctypes.byref(options) if options is not None else None
