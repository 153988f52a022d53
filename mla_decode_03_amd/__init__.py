"""MLA decode on MI355X (gfx950): thin Python binding over libmla.so.

Argument marshalling only.  Every step of the decode (split planning, the split-KV
MFMA kernel, the log-sum-exp combine) runs in the HIP library; this module passes
`tensor.data_ptr()` values and the current HIP stream through ctypes.  PyTorch is
used for device memory and streams only.  There is no fallback: if the library
is missing, every call raises.

The C ABI (include/mla.h) defines the operation:

    out[b, t, h, :] = sum_p softmax_p(scale * q[b, t, h, :] . k_p) * k_p[:512]
    lse[b, t, h]    = ln sum_p exp(scale * q[b, t, h, :] . k_p)

over the cached rows k_p (576 wide) of sequence b, gathered from 64-token pages
through the block table, with optional causal masking among the q_len new tokens.
With `sinks` (float32 [H] on the device) head h's softmax gains one more term
exp(sinks[h]) whose value row is zero (attention sinks; mla_decode_ex).  With `indices`
(int32 [B, T, topk] on the device, a problem made with topk) each (b, t) attends to
exactly its listed token positions, -1 entries unused (sparse decode; mla_decode_ex).
"""
from __future__ import annotations

import ctypes
import os

from . import _abi
from ._abi import (D_QK, D_V, DTYPE_BF16, DTYPE_F32, MAX_ROWS, PAGE, MlaError, PlanOptions,  # noqa: F401
                   Problem, lib, lib_path)

__all__ = ["D_QK", "D_V", "PAGE", "MAX_ROWS", "DTYPE_BF16", "DTYPE_F32", "MlaError", "Problem",
           "PlanOptions", "Plan", "lib", "lib_path", "metadata_bytes", "workspace_bytes",
           "get_metadata", "decode", "decode_splits", "combine", "make_problem", "Decoder",
           "device_num_cus", "hbm_read_probe", "decode_noalloc"]


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def device_num_cus() -> int:
    n = ctypes.c_int32(0)
    _abi.check(lib().mla_device_num_cus(ctypes.byref(n)), "mla_device_num_cus")
    return int(n.value)


def make_problem(q, kv_cache, block_table, causal: bool = False, topk: int = 0) -> Problem:
    """Problem descriptor from tensors: q [B, T, H, 576], kv [pages, 64, 576], block_table [B, stride];
    topk > 0 makes a sparse problem (index lists of topk entries per (b, t))."""
    import torch
    B, T, H, d = q.shape
    assert d == D_QK and kv_cache.shape[1:] == (PAGE, D_QK), (q.shape, kv_cache.shape)
    if q.dtype == torch.bfloat16:
        dt = DTYPE_BF16
    elif q.dtype == torch.float32:
        dt = DTYPE_F32
    else:
        raise MlaError(_abi.MLA_ERR_DTYPE, "q dtype %s" % q.dtype)
    if kv_cache.dtype != q.dtype:
        raise MlaError(_abi.MLA_ERR_DTYPE, "kv_cache dtype %s != q dtype %s" % (kv_cache.dtype, q.dtype))
    return Problem(batch=B, q_len=T, num_heads=H, causal=int(bool(causal)),
                   num_pages=kv_cache.shape[0], block_table_stride=block_table.stride(0),
                   max_blocks_per_seq=block_table.shape[1], dtype=dt, topk=int(topk))


def metadata_bytes(problem: Problem, options: PlanOptions | None = None, num_cus: int = 0) -> int:
    return int(lib().mla_metadata_bytes(ctypes.byref(problem), _abi.opt_ref(options), num_cus))


def workspace_bytes(problem: Problem, options: PlanOptions | None = None, num_cus: int = 0) -> int:
    return int(lib().mla_workspace_bytes(ctypes.byref(problem), _abi.opt_ref(options), num_cus))


class Plan:
    """A split plan: the device metadata tensor plus the host-side launch shape."""

    def __init__(self, metadata, c_plan):
        self.metadata = metadata
        self.c_plan = c_plan

    @property
    def grid_wg(self) -> int:
        return int(self.c_plan.grid_wg)

    @property
    def max_partials(self) -> int:
        return int(self.c_plan.max_partials)

    def error(self, stream=None) -> int:
        """Device-side input fault flag (synchronises the stream); 0 = none."""
        return int(lib().mla_plan_error(ctypes.byref(self.c_plan), _stream_handle(stream)))


def get_metadata(problem: Problem, cache_seqlens, metadata, options: PlanOptions | None = None,
                 num_cus: int = 0, stream=None) -> Plan:
    """Run the split planner on the device; `metadata` is a caller-owned uint8/int32 tensor."""
    c_plan = _abi.CPlan(metadata=metadata.data_ptr(),
                        metadata_bytes=metadata.numel() * metadata.element_size())
    rc = lib().mla_get_metadata(ctypes.byref(problem), _ptr(cache_seqlens), _abi.opt_ref(options),
                                num_cus, ctypes.byref(c_plan), _stream_handle(stream))
    _abi.check(rc, "mla_get_metadata")
    return Plan(metadata, c_plan)


def _variant(sinks, indices=None):
    """ctypes variant argument: None (plain decode) or a pointer to an mla_variant_t."""
    if sinks is None and indices is None:
        return None
    return ctypes.byref(_abi.Variant(sinks=sinks.data_ptr() if sinks is not None else None,
                                     indices=indices.data_ptr() if indices is not None else None))


def decode(problem: Problem, q, kv_cache, block_table, cache_seqlens, scale: float, out, lse,
           plan: Plan | None = None, workspace=None, stream=None, sinks=None, indices=None) -> None:
    """Enqueue the decode; outputs are written into `out` and `lse` (caller-owned).
    `sinks` (float32 [H]) and `indices` (int32 [B, T, topk]) device tensors select the
    attention-sink and sparse variants (mla_decode_ex)."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(q), _ptr(kv_cache), _ptr(block_table), _ptr(cache_seqlens), ctypes.c_float(scale),
            _ptr(out), _ptr(lse), ctypes.byref(plan.c_plan) if plan is not None else None,
            _ptr(workspace), ctypes.c_size_t(ws_bytes), _stream_handle(stream))
    if sinks is None and indices is None:
        _abi.check(lib().mla_decode(ctypes.byref(problem), *args), "mla_decode")
    else:
        _abi.check(lib().mla_decode_ex(ctypes.byref(problem), _variant(sinks, indices), *args), "mla_decode_ex")


def decode_splits(problem: Problem, q, kv_cache, block_table, cache_seqlens, scale: float, out, lse,
                  plan: Plan, workspace, stream=None, sinks=None, indices=None, events=None) -> None:
    """Enqueue only the split-KV decode kernel (partials for split sequences).  events: an
    optional (start, stop) pair of timing torch.cuda.Event, bound to the kernel's own start
    and end (mla_decode_splits_timed)."""
    ws_bytes = workspace.numel() * workspace.element_size()
    args = (ctypes.byref(problem), _variant(sinks, indices), _ptr(q), _ptr(kv_cache), _ptr(block_table),
            _ptr(cache_seqlens), ctypes.c_float(scale), _ptr(out), _ptr(lse), ctypes.byref(plan.c_plan),
            _ptr(workspace), ctypes.c_size_t(ws_bytes), _stream_handle(stream))
    if events is None:
        _abi.check(lib().mla_decode_splits(*args), "mla_decode_splits")
    else:
        start, stop = (ctypes.c_void_p(e.cuda_event) for e in events)
        _abi.check(lib().mla_decode_splits_timed(*args, start, stop), "mla_decode_splits_timed")


def combine(problem: Problem, out, lse, plan: Plan, workspace, stream=None, sinks=None) -> None:
    """Enqueue only the log-sum-exp combine of the split partials."""
    ws_bytes = workspace.numel() * workspace.element_size()
    rc = lib().mla_combine(ctypes.byref(problem), _variant(sinks), _ptr(out), _ptr(lse),
                           ctypes.byref(plan.c_plan),
                           _ptr(workspace), ctypes.c_size_t(ws_bytes), _stream_handle(stream))
    _abi.check(rc, "mla_combine")


def decode_noalloc(problem: Problem, q, kv_cache, block_table, cache_seqlens, scale: float, out, lse,
                   stream=None, sinks=None) -> None:
    """Enqueue the decode through mla_decode_noalloc: default plan and split partials in the
    library's own device scratch (no buffers from the caller but inputs and outputs).
    Calls that overlap on one device race on that scratch."""
    rc = lib().mla_decode_noalloc(ctypes.byref(problem), _variant(sinks), _ptr(q), _ptr(kv_cache),
                                  _ptr(block_table), _ptr(cache_seqlens), ctypes.c_float(scale), _ptr(out),
                                  _ptr(lse), _stream_handle(stream))
    _abi.check(rc, "mla_decode_noalloc")


def hbm_read_probe(src, mode: int, sink, num_workgroups: int = 0, nbytes: int | None = None, stream=None) -> None:
    """Enqueue the HBM streaming-read probe over `src` (a device tensor; `nbytes` of it,
    default all): mode 0 = vector loads, mode 1 = the decode's global->LDS copies.
    `sink` is a device uint32/int32 tensor with at least one element per workgroup."""
    n = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    rc = lib().mla_hbm_read_probe(_ptr(src), ctypes.c_size_t(n), int(mode), int(num_workgroups), _ptr(sink),
                                  _stream_handle(stream))
    _abi.check(rc, "mla_hbm_read_probe")


class Decoder:
    """Owns the metadata and workspace buffers for one problem shape.

    decoder = Decoder(q, kv, block_table, causal)
    out, lse = decoder(q, kv, block_table, cache_seqlens, scale)
    """

    def __init__(self, q, kv_cache, block_table, causal: bool = False, split: bool = True,
                 options: PlanOptions | None = None, num_cus: int = 0, topk: int = 0):
        import torch
        self.problem = make_problem(q, kv_cache, block_table, causal, topk)
        self.options = options
        self.num_cus = num_cus
        self.split = split and self.problem.dtype == DTYPE_BF16
        # float32 problems are never split; their plan only carries the device-side fault flag
        self.planned = split
        dev = q.device
        if self.planned:
            mb = metadata_bytes(self.problem, options, num_cus)
            wb = workspace_bytes(self.problem, options, num_cus) if self.split else 0
            if mb == 0:
                raise MlaError(_abi.MLA_ERR_SHAPE, "invalid problem for planning")
            self.metadata = torch.empty(mb, dtype=torch.uint8, device=dev)
            self.workspace = torch.empty(max(wb, 16), dtype=torch.uint8, device=dev)
        else:
            self.metadata = None
            self.workspace = None
        self.plan = None

    def plan_for(self, cache_seqlens, stream=None) -> Plan | None:
        """The plan for these lengths.  With options.plan_in_decode the decode launches
        re-plan from the lengths they are given, so the plan is made once and reused."""
        if not self.planned:
            return None
        if self.plan is not None and self.options is not None and self.options.plan_in_decode:
            return self.plan
        self.plan = get_metadata(self.problem, cache_seqlens, self.metadata, self.options,
                                 self.num_cus, stream)
        return self.plan

    def __call__(self, q, kv_cache, block_table, cache_seqlens, scale: float, out=None, lse=None,
                 replan: bool = True, stream=None, sinks=None, indices=None):
        import torch
        B, T, H, _ = q.shape
        if out is None:
            out = torch.empty((B, T, H, D_V), dtype=q.dtype, device=q.device)
        if lse is None:
            lse = torch.empty((B, T, H), dtype=torch.float32, device=q.device)
        if replan or self.plan is None:
            self.plan_for(cache_seqlens, stream)
        decode(self.problem, q, kv_cache, block_table, cache_seqlens, scale, out, lse,
               self.plan, self.workspace, stream, sinks, indices)
        return out, lse


def _lib_loaded_path() -> str:
    return os.path.realpath(lib_path())
