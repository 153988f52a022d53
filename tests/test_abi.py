"""C-ABI boundary checks that need no GPU: the library loads, exports every symbol the
header declares (and nothing else), and every host-checkable argument fault returns
its status code before anything is enqueued."""
import ctypes
import os
import re

import pytest

import mla_decode_03_amd as m
from mla_decode_03_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^MLA_API\s+[\w\s\*]+?\b(mla_\w+)\s*\(", text, flags=re.M)))


def _exported():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", _abi.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    return sorted(line.split()[-1] for line in out.splitlines() if " T " in line)


def test_library_exports_exactly_the_header():
    declared = _declared()
    assert declared == sorted(_abi.EXPORTS)
    assert _exported() == declared
    L = m.lib()
    for name in declared:
        assert hasattr(L, name)


def test_status_strings():
    for code in range(10):
        assert _abi.status_string(code)
    assert _abi.status_string(0) == "ok"
    assert "unknown" in _abi.status_string(99)


def _problem(**kw):
    base = dict(batch=4, q_len=1, num_heads=128, causal=0, num_pages=64, block_table_stride=16,
                max_blocks_per_seq=16, dtype=m.DTYPE_BF16)
    base.update(kw)
    return m.Problem(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(num_heads=129), _abi.MLA_ERR_SHAPE),
    (dict(q_len=2, num_heads=65), _abi.MLA_ERR_SHAPE),
    (dict(q_len=0), _abi.MLA_ERR_SHAPE),
    (dict(batch=-1), _abi.MLA_ERR_SHAPE),
    (dict(num_pages=0), _abi.MLA_ERR_SHAPE),
    (dict(block_table_stride=8), _abi.MLA_ERR_SHAPE),
    (dict(causal=2), _abi.MLA_ERR_SHAPE),
    (dict(dtype=7), _abi.MLA_ERR_DTYPE),
])
def test_decode_rejects_bad_problem(kw, code):
    p = _problem(**kw)
    fake = ctypes.c_void_p(0x10000)
    rc = m.lib().mla_decode(ctypes.byref(p), fake, fake, fake, fake, 1.0, fake, fake, None, None, 0, None)
    assert rc == code
    assert m.metadata_bytes(p, None, 256) == 0 and m.workspace_bytes(p, None, 256) == 0


def test_decode_rejects_null_and_misaligned():
    p = _problem()
    a = ctypes.c_void_p(0x10000)
    L = m.lib()
    assert L.mla_decode(None, a, a, a, a, 1.0, a, a, None, None, 0, None) == _abi.MLA_ERR_NULL
    assert L.mla_decode(ctypes.byref(p), None, a, a, a, 1.0, a, a, None, None, 0, None) == _abi.MLA_ERR_NULL
    assert L.mla_decode(ctypes.byref(p), a, a, a, a, 1.0, a, None, None, None, 0, None) == _abi.MLA_ERR_NULL
    odd = ctypes.c_void_p(0x10008)  # 8-byte aligned only
    assert L.mla_decode(ctypes.byref(p), odd, a, a, a, 1.0, a, a, None, None, 0, None) == _abi.MLA_ERR_ALIGN
    assert L.mla_decode(ctypes.byref(p), a, a, ctypes.c_void_p(0x10002), a, 1.0, a, a, None, None, 0,
                        None) == _abi.MLA_ERR_ALIGN
    # batch 0 is a no-op, even with null buffers
    p0 = _problem(batch=0)
    assert L.mla_decode(ctypes.byref(p0), None, None, None, None, 1.0, None, None, None, None, 0, None) == 0


def test_plan_sizes_and_workspace_checks():
    p = _problem()
    mb = m.metadata_bytes(p, None, 256)
    wb = m.workspace_bytes(p, None, 256)
    # header + cu_blocks[B+1] + 3 per unit + wg_begin[grid+1] + wg_seq[grid] int32 words
    assert mb == 4 * (16 + 5 + 3 * 4 + 257 + 256)
    # partial slots: grid + min(grid, units), each rows_per_wg rows of a compensated bf16
    # pair (hi and lo halves) and a float32 (LSE, normalising factor) pair, plus 16 words
    # of low-half flags a slot
    def part(slots, rows):
        return slots * rows * 512 * 4 + (slots * rows * 8 + 15) // 16 * 16 + slots * 64
    assert wb == part(256 + 4, 128)
    opts = m.PlanOptions(num_workgroups=8, min_blocks_per_wg=1, row_split=2)
    assert m.workspace_bytes(p, opts, 256) == part(8 + 8, 64)
    assert m.workspace_bytes(p, m.PlanOptions(row_split=3), 256) == 0  # unsupported split
    # batch-invariant plan: one workgroup and one partial slot per possible chunk
    fo = m.PlanOptions(fixed_split_blocks=5, row_split=2, num_workgroups=3)
    grid = 4 * 2 * 4                                       # units * ceil(16 / 5)
    assert m.metadata_bytes(p, fo, 256) == 4 * (16 + 5 + 3 * 8 + 2 * grid + 1)
    assert m.workspace_bytes(p, fo, 256) == part(grid, 64)
    assert m.workspace_bytes(p, fo, 80) == m.workspace_bytes(p, fo, 256)   # no CU dependence
    # partition rule: 0 (cost model), 1 (pages) or 2 (cost); anything else is refused
    for rule in (0, 1, 2):
        assert m.metadata_bytes(p, m.PlanOptions(split_rule=rule), 256) == mb
    assert m.metadata_bytes(p, m.PlanOptions(split_rule=3), 256) == 0
    assert m.metadata_bytes(p, m.PlanOptions(split_rule=-1), 256) == 0
    L = m.lib()
    a = ctypes.c_void_p(0x10000)
    # metadata buffer too small: refused before any launch
    plan = _abi.CPlan(metadata=0x10000, metadata_bytes=mb - 4)
    assert L.mla_get_metadata(ctypes.byref(p), a, None, 256, ctypes.byref(plan), None) == _abi.MLA_ERR_WORKSPACE
    plan = _abi.CPlan(metadata=None, metadata_bytes=mb)
    assert L.mla_get_metadata(ctypes.byref(p), a, None, 256, ctypes.byref(plan), None) == _abi.MLA_ERR_NULL
    plan = _abi.CPlan(metadata=0x10004, metadata_bytes=mb)
    assert L.mla_get_metadata(ctypes.byref(p), a, None, 256, ctypes.byref(plan), None) == _abi.MLA_ERR_ALIGN
    # a plan for another problem, or an undersized workspace, is refused by mla_decode
    good = _abi.CPlan(metadata=0x10000, metadata_bytes=mb, grid_wg=256, row_split=1, rows_per_wg=128,
                      max_partials=260, batch=4, rows=128)
    assert L.mla_decode(ctypes.byref(p), a, a, a, a, 1.0, a, a, ctypes.byref(good), a, wb - 1,
                        None) == _abi.MLA_ERR_WORKSPACE
    assert L.mla_decode(ctypes.byref(p), a, a, a, a, 1.0, a, a, ctypes.byref(good), None, wb,
                        None) == _abi.MLA_ERR_NULL
    other = _abi.CPlan(metadata=0x10000, metadata_bytes=mb, grid_wg=256, row_split=1, rows_per_wg=128,
                       max_partials=260, batch=5, rows=128)
    assert L.mla_decode(ctypes.byref(p), a, a, a, a, 1.0, a, a, ctypes.byref(other), a, wb,
                        None) == _abi.MLA_ERR_SHAPE
    # the scale must be positive and finite (checked before any launch)
    for bad in (0.0, -0.5, float("inf"), float("nan"), 3e38):
        assert L.mla_decode(ctypes.byref(p), a, a, a, a, bad, a, a, ctypes.byref(good), a, wb,
                            None) == _abi.MLA_ERR_SHAPE, bad


def test_variant_checks():
    """mla_decode_ex: a misaligned sinks pointer is refused before any launch, by every
    entry that takes the variant."""
    p = _problem()
    a = ctypes.c_void_p(0x10000)
    L = m.lib()
    bad = ctypes.byref(_abi.Variant(sinks=0x10002))
    assert L.mla_decode_ex(ctypes.byref(p), bad, a, a, a, a, 1.0, a, a, None, None, 0,
                           None) == _abi.MLA_ERR_ALIGN
    mb, wb = m.metadata_bytes(p, None, 256), m.workspace_bytes(p, None, 256)
    plan = _abi.CPlan(metadata=0x10000, metadata_bytes=mb, grid_wg=256, row_split=1, rows_per_wg=128,
                      max_partials=260, batch=4, rows=128)
    assert L.mla_decode_splits(ctypes.byref(p), bad, a, a, a, a, 1.0, a, a, ctypes.byref(plan), a, wb,
                               None) == _abi.MLA_ERR_ALIGN
    assert L.mla_combine(ctypes.byref(p), bad, a, a, ctypes.byref(plan), a, wb, None) == _abi.MLA_ERR_ALIGN
    # the problem is checked first, with or without a variant
    p129 = _problem(num_heads=129)
    assert L.mla_decode_ex(ctypes.byref(p129), bad, a, a, a, a, 1.0, a, a, None, None, 0,
                           None) == _abi.MLA_ERR_SHAPE


def test_sparse_problem_checks():
    L = m.lib()
    a = ctypes.c_void_p(0x10000)
    sp = _problem(q_len=2, num_heads=128, topk=100)           # 256 rows: fine for a sparse problem
    # planned as batch*q_len units of ceil(100/64) = 2 blocks, 128 rows each
    mb = m.metadata_bytes(sp, None, 256)
    assert mb == 4 * (16 + 9 + 3 * 8 + 257 + 256)
    # workspace: partials (256-byte aligned), then the row lists and the counts
    part = (256 + 8) * 128 * 2056 + (256 + 8) * 64
    rows = 8 * 128 * 4
    assert m.workspace_bytes(sp, None, 256) == ((part + 255) // 256 * 256) + rows + 256
    assert m.metadata_bytes(_problem(q_len=2, num_heads=128), None, 256) == 0   # dense: too many rows
    assert m.metadata_bytes(_problem(topk=-1), None, 256) == 0
    assert m.metadata_bytes(_problem(topk=8, causal=1), None, 256) == 0         # lists replace causal
    assert m.metadata_bytes(_problem(topk=8, dtype=m.DTYPE_F32), None, 256) == 0
    # the decode needs the lists and a plan
    assert L.mla_decode(ctypes.byref(sp), a, a, a, a, 1.0, a, a, None, None, 0, None) == _abi.MLA_ERR_NULL
    v = ctypes.byref(_abi.Variant(indices=0x10000))
    assert L.mla_decode_ex(ctypes.byref(sp), v, a, a, a, a, 1.0, a, a, None, None, 0,
                           None) == _abi.MLA_ERR_UNSUPPORTED
    bad = ctypes.byref(_abi.Variant(indices=0x10002))
    assert L.mla_decode_ex(ctypes.byref(sp), bad, a, a, a, a, 1.0, a, a, None, None, 0,
                           None) == _abi.MLA_ERR_ALIGN


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_abi, "_lib", None)
    monkeypatch.setattr(_abi, "_LIB_PATH", str(tmp_path / "libmla.so"))
    with pytest.raises(RuntimeError, match="no fallback"):
        _abi.lib()


def test_hbm_probe_argument_checks():
    """Every host-checkable fault of the streaming-read probe returns its status before
    anything is enqueued (an explicit workgroup count: no device query)."""
    L = m.lib()
    src, sink = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000)
    mib = 1 << 20
    assert L.mla_hbm_read_probe(None, mib, 0, 4, sink, None) == _abi.MLA_ERR_NULL
    assert L.mla_hbm_read_probe(src, mib, 0, 4, None, None) == _abi.MLA_ERR_NULL
    assert L.mla_hbm_read_probe(src, mib, 2, 4, sink, None) == _abi.MLA_ERR_UNSUPPORTED
    assert L.mla_hbm_read_probe(src, mib, -1, 4, sink, None) == _abi.MLA_ERR_UNSUPPORTED
    assert L.mla_hbm_read_probe(ctypes.c_void_p(0x100008), mib, 0, 4, sink, None) == _abi.MLA_ERR_ALIGN
    assert L.mla_hbm_read_probe(src, mib, 1, 4, ctypes.c_void_p(0x200002), None) == _abi.MLA_ERR_ALIGN
    # chunks: equal, a positive multiple of 16 KiB, below 4 GiB
    assert L.mla_hbm_read_probe(src, 0, 0, 4, sink, None) == _abi.MLA_ERR_SHAPE
    assert L.mla_hbm_read_probe(src, mib + 16384, 0, 4, sink, None) == _abi.MLA_ERR_SHAPE   # not divisible by 4 x 16 KiB
    assert L.mla_hbm_read_probe(src, 3 * 16384, 1, 2, sink, None) == _abi.MLA_ERR_SHAPE    # 24 KiB chunks
    assert L.mla_hbm_read_probe(src, 1 << 33, 0, 2, sink, None) == _abi.MLA_ERR_SHAPE      # 4 GiB chunks


def test_noalloc_host_checks():
    """mla_decode_noalloc's checks that need no device: null and invalid problems, batch 0
    (a no-op), and the sparse form it does not serve."""
    L = m.lib()
    args = (None, None, None, None, ctypes.c_float(1.0), None, None, None)
    assert L.mla_decode_noalloc(None, None, *args) == _abi.MLA_ERR_NULL
    assert L.mla_decode_noalloc(ctypes.byref(_problem(num_heads=129)), None, *args) == _abi.MLA_ERR_SHAPE
    assert L.mla_decode_noalloc(ctypes.byref(_problem(dtype=5)), None, *args) == _abi.MLA_ERR_DTYPE
    assert L.mla_decode_noalloc(ctypes.byref(_problem(batch=0)), None, *args) == _abi.MLA_OK
    assert L.mla_decode_noalloc(ctypes.byref(_problem(topk=64)), None, *args) == _abi.MLA_ERR_UNSUPPORTED
