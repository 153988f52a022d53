"""CPU oracle for MLA decode: TEST INFRASTRUCTURE ONLY.

Only `tests/`, `__graft_entry__.smoke()` and the CPU-baseline leg of `bench.py`
may import this package.  The product library neither links nor calls it, and it
shares no code with the HIP path (no kernels, headers, helpers or constants).

Contents:
  decode()   float64 decode of a paged case (C + OpenMP, `mla_oracle.c`): page
             gather, naive dot products, two-pass softmax, weighted value sum.
  combine()  log-sum-exp merge of partial results over disjoint key sets
             (`combine.py`).
  brute      pure-Python reference on a dense (unpaged) key list (`brute.py`).

The pages define MLA decode only as the two chained GEMMs of the TileLang notes'
FlashMLA example ("TileLang: bridging programmability and performance in modern
neural kernels", section "A complete example: two-stage optimisation of
FlashMLA"); every function here names the reading of the problem it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .combine import combine  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

DTYPE_CODES = {"f32": 0, "bf16": 1}


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        lib.mla_oracle_decode.restype = ctypes.c_int
        lib.mla_oracle_decode.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_double, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_int32,
            ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32]
        lib.mla_oracle_max_threads.restype = ctypes.c_int32
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().mla_oracle_max_threads())


def decode(q, kv, block_table, cache_seqlens, *, scale: float, dtype: str = "f32",
           causal: bool = False, rows=None, d_v: int = 512, page: int | None = None,
           threads: int = 0, sinks=None, indices=None):
    """float64 MLA decode.

    q:  [B, T, H, d_qk] float32 values, or uint16 bf16 bits when dtype == "bf16"
    kv: [num_pages, page, d_qk] same dtype convention
    block_table: [B, stride] int32; cache_seqlens: [B] int32
    rows: optional flat row ids (b*T + t)*H + h to compute; default all rows.
    sinks: optional per-head sink logits [H] (an extra softmax term with a zero value
           row; see mla_oracle.c), taken as float64.
    indices: optional sparse token lists [B, T, topk] int32 (-1 = unused entry); each
           row then attends to exactly its (b, t) list.  Needs causal False.
    Returns (out [n_rows, d_v] float64, lse [n_rows] float64), rows in the order asked.
    """
    q = np.ascontiguousarray(q)
    kv = np.ascontiguousarray(kv)
    want = np.uint16 if dtype == "bf16" else np.float32
    assert q.dtype == want and kv.dtype == want, (q.dtype, kv.dtype, dtype)
    B, T, H, d_qk = q.shape
    npages, pg, d_qk2 = kv.shape
    assert d_qk2 == d_qk
    if page is not None:
        assert page == pg
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    lens = np.ascontiguousarray(cache_seqlens, dtype=np.int32)
    assert bt.ndim == 2 and bt.shape[0] == B and lens.shape == (B,)
    if rows is None:
        n_rows = B * T * H
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        n_rows = rows_arr.size
    sk = None
    if sinks is not None:
        sk = np.ascontiguousarray(sinks, dtype=np.float64)
        assert sk.shape == (H,), sk.shape
    idx, topk = None, 0
    if indices is not None:
        idx = np.ascontiguousarray(indices, dtype=np.int32)
        assert idx.ndim == 3 and idx.shape[:2] == (B, T), idx.shape
        topk = idx.shape[2]
    out = np.empty((n_rows, d_v), dtype=np.float64)
    lse = np.empty((n_rows,), dtype=np.float64)
    rc = _load().mla_oracle_decode(
        q.ctypes.data, kv.ctypes.data, DTYPE_CODES[dtype],
        bt.ctypes.data, bt.shape[1], lens.ctypes.data,
        B, T, H, npages, pg, d_qk, d_v, int(bool(causal)), float(scale),
        sk.ctypes.data if sk is not None else None,
        idx.ctypes.data if idx is not None else None, topk,
        rows_arr.ctypes.data if rows_arr is not None else None, n_rows,
        out.ctypes.data, lse.ctypes.data, int(threads))
    if rc != 0:
        raise RuntimeError("mla_oracle_decode failed with code %d" % rc)
    return out, lse


def decode_case(case, rows=None, threads: int = 0, sinks=None, indices=None):
    """decode() on a `mla_inputs.Case`."""
    return decode(case.q_array(), case.kv_array(), case.block_table, case.cache_seqlens,
                  scale=case.scale, dtype=case.dtype, causal=case.causal, rows=rows,
                  threads=threads, sinks=sinks, indices=indices)
