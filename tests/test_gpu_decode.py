"""Parity of the HIP decode path (through the C ABI) against the float64 oracle."""
import numpy as np
import pytest

import oracle
from gpu_util import ATOL, compare, oracle_rows, run, say, to_device
from mla_inputs import make_case, make_config, poison_unused

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_decode_03_amd as mla
    mla.lib()


def _case(B, T, H, lens, seed, causal=False, dtype="bf16", extra_pages=0):
    return make_case(batch=B, q_len=T, num_heads=H, seqlens=lens, dtype=dtype, causal=causal,
                     seed=seed, extra_pages=extra_pages)


def test_config0_fp32_full():
    case = make_config(0)
    say("config0 fp32", case.name)
    ref_o, ref_l = oracle_rows(case)
    o, l, _ = run(case)
    s = compare(o, l, ref_o, ref_l, "config0")
    assert s["max_abs"] < 1e-4  # fp32 path: far inside the bf16 tolerance


@pytest.mark.parametrize("B,T,H,lens,causal", [
    (4, 1, 128, [1, 31, 32, 33], False),          # four row tiles; chunk tails
    (3, 1, 48, [64, 65, 1000], False),            # a part-filled row tile
    (2, 2, 64, [0, 97], True),                    # causal q_len 2, an empty sequence
    (1, 1, 16, [4096], False),
])
def test_fp32_matrix_core_shapes(B, T, H, lens, causal):
    """The fp32 path on the fp32 matrix cores: 32-row tiles (part-filled ones too), 32-key
    chunks with ragged tails, causal rows, empty sequences."""
    case = _case(B, T, H, lens, seed=40 + B + H, causal=causal, dtype="f32")
    say("fp32 mfma", B, T, H, lens, causal)
    ref_o, ref_l = oracle_rows(case)
    o, l, _ = run(case)
    s = compare(o, l, ref_o, ref_l, "fp32 %dx%dx%d" % (B, T, H))
    assert s["max_abs"] < 1e-4 and s["max_lse"] < 1e-5


SMALL = [
    # (B, T, H, lens, causal): token counts crossing page edges; every row/wave layout
    (2, 1, 128, [1, 70], False),
    (3, 1, 128, [63, 64, 65], False),
    (2, 1, 128, [4095, 4097], False),
    (4, 2, 16, [2, 65, 100, 128], True),
    (3, 2, 16, [1, 3, 64], True),
    (3, 1, 64, [200, 1, 129], False),
    (2, 1, 16, [300, 5], False),
    (2, 1, 48, [130, 77], False),
    (2, 1, 100, [150, 40], False),
    (2, 2, 64, [66, 130], True),
    (3, 1, 128, [0, 50, 0], False),
]


@pytest.mark.parametrize("mode", ["plan", "forced_splits", "unsplit", "fixed_splits", "cost_rule"])
@pytest.mark.parametrize("B,T,H,lens,causal", SMALL)
def test_small_parity(B, T, H, lens, causal, mode):
    import mla_decode_03_amd as mla
    case = _case(B, T, H, lens, seed=B * 100 + T * 10 + H + len(mode), causal=causal)
    say("small", B, T, H, lens, causal, mode)
    ref_o, ref_l = oracle_rows(case)
    kw = {}
    if mode == "forced_splits":
        kw = dict(options=mla.PlanOptions(num_workgroups=7, min_blocks_per_wg=1))
    elif mode == "unsplit":
        kw = dict(split=False)
    elif mode == "fixed_splits":
        kw = dict(options=mla.PlanOptions(fixed_split_blocks=2))
    elif mode == "cost_rule":
        kw = dict(options=mla.PlanOptions(num_workgroups=5, min_blocks_per_wg=1, split_rule=2))
    o, l, _ = run(case, **kw)
    compare(o, l, ref_o, ref_l, "small %s" % mode)


@pytest.mark.parametrize("idx", [1, 2, 3, 4])
def test_full_config_every_row(idx):
    """Full-size workloads, default plan, every row against the oracle: in the launch
    configuration the benchmark times (the plan computed inside the decode launch), and
    with a planner launch before the decode."""
    import mla_decode_03_amd as mla
    case = make_config(idx)
    say("config", idx, case.name, "pages", case.num_pages)
    ref_o, ref_l = oracle_rows(case)
    for in_decode in (1, 0):
        o, l, _ = run(case, options=mla.PlanOptions(plan_in_decode=in_decode))
        compare(o, l, ref_o, ref_l, "config%d, all %d rows, plan_in_decode=%d" % (idx, o.shape[0], in_decode))


def test_split_counts_agree():
    """Different split plans (1 .. many workgroups per sequence) each meet the oracle
    tolerance and agree with each other to the bf16 rounding of P: every split fixes its
    own reference max, so the rounding errors of P (2^-9 relative) land differently;
    the outputs then differ by about 2^-9 * |v| / sqrt(effective keys), ~1e-4 here."""
    import mla_decode_03_amd as mla
    case = _case(2, 1, 128, [3000, 1500], seed=7)
    t = to_device(case)
    ref_o, ref_l = oracle_rows(case)
    res = []
    for nwg in (1, 2, 7, 64, 256):
        say("splits nwg", nwg)
        o, l, _ = run(case, tensors=t, options=mla.PlanOptions(num_workgroups=nwg, min_blocks_per_wg=1))
        compare(o, l, ref_o, ref_l, "nwg=%d" % nwg)
        res.append((o, l))
    o0, l0 = res[0]
    for o, l in res[1:]:
        assert np.max(np.abs(l - l0)) < 1e-4
        # a bf16 ulp of the output (2^-8..2^-7 relative) plus the P-rounding noise
        assert np.all(np.abs(o - o0) <= 2 ** -7 * np.abs(o0) + 2e-3)
        # two independent roundings (output and P, ~2e-3 relative L2 each vs the oracle)
        assert np.linalg.norm(o - o0) / np.linalg.norm(o0) < 5e-3


@pytest.mark.parametrize("H,nwg,with_sinks", [(128, 8, False), (33, 12, True), (16, 40, False)])
def test_grouped_merge(H, nwg, with_sinks):
    """Plans that average 8 or more partials per unit take the grouped merge (4 thread
    groups per row, then one LDS exchange): 8 partials (each group's 2 in one batch), 12
    (groups of 3 in batches of 4, one split read again with no weight), 40 with 16 heads
    (several batches); 33 heads leave the last workgroup's second row empty; with sinks
    too.  Every row meets the oracle."""
    import mla_decode_03_amd as mla
    from mla_inputs import make_sinks
    case = _case(1, 1, H, [3000], seed=80 + nwg)
    sinks = make_sinks(H, seed=6) if with_sinks else None
    say("grouped merge", H, nwg, with_sinks)
    ref_o, ref_l = oracle_rows(case, sinks=sinks)
    o, l, dec = run(case, options=mla.PlanOptions(num_workgroups=nwg, min_blocks_per_wg=1), sinks=sinks)
    assert dec.plan.grid_wg == nwg
    compare(o, l, ref_o, ref_l, "grouped merge H=%d nwg=%d" % (H, nwg))


def _scale_blocks(case, factor, rope_only):
    """Multiply block j of every sequence by factor(j): its rope dims only, or whole rows
    (keys and values alike), re-rounded to bf16."""
    from mla_inputs import bf16_bits_to_f32, f32_to_bf16_bits
    for b in range(case.batch):
        for j in range((int(case.cache_seqlens[b]) + 63) // 64):
            pg = int(case.block_table[b, j])
            x = case.kv[pg].copy()
            if rope_only:
                x[:, 512:] *= np.float32(factor(j))
            else:
                x *= np.float32(factor(j))
            bits = f32_to_bf16_bits(x).reshape(x.shape)
            case.kv_bits[pg] = bits
            case.kv[pg] = bf16_bits_to_f32(bits).reshape(bits.shape)


def test_merge_rescales_as_the_largest_partial_grows():
    """Keys whose rope dims grow block by block (values untouched) make the largest LSE
    seen by the merge rise at every group of four one-block partials, by under one unit
    early and by tens late, so the running sums are rescaled at every group and the early
    groups still carry weight (32 and 40 partials per sequence); the merged rows must meet
    the oracle."""
    import mla_decode_03_amd as mla
    case = _case(2, 1, 128, [2048, 2560], seed=77)
    _scale_blocks(case, lambda j: 2.0 ** (j / 6.0), rope_only=True)
    say("merge rescale", case.cache_seqlens.tolist())
    ref_o, ref_l = oracle_rows(case)
    # the partial LSEs really climb: the whole sequence's LSE is far above its first block's
    first = oracle.decode_case(_first_blocks(case, 1))[1]
    assert np.all(ref_l - first > 5.0)
    o, l, _ = run(case, options=mla.PlanOptions(fixed_split_blocks=1))
    compare(o, l, ref_o, ref_l, "merge rescale")


def test_merge_of_large_cancelling_partials():
    """Whole rows (keys and values) scaled by min(2^(j/6), 16) in block j: late one-block
    partials are peaked (their P is exact to a few ulps) and hold values up to ~16x the
    unit scale, and rows whose merge cancels them come out small.  A float64 model of the
    kernel's rounding puts bf16-only partials at 1.4x the absolute bound on this case, and
    the compensated pair (bf16 high half plus the low half stored for row quarters with
    |o| > 1)
    at 0.36x.  The low halves must have been written, and every row must meet the oracle.
    (Past about 16x, with block scales that keep growing, the bf16 rounding of P alone
    exceeds the absolute bound, whatever the partials' precision.)"""
    import torch
    import mla_decode_03_amd as mla
    case = _case(2, 1, 128, [2048, 2560], seed=77)
    _scale_blocks(case, lambda j: min(2.0 ** (j / 6.0), 16.0), rope_only=False)
    say("merge of large cancelling partials", case.cache_seqlens.tolist())
    ref_o, ref_l = oracle_rows(case)
    o, l, dec = run(case, options=mla.PlanOptions(fixed_split_blocks=1))
    torch.cuda.synchronize()
    rows = dec.plan.max_partials * 128                 # partial rows of the workspace
    # after the high halves and the (LSE, factor) pairs (padded to 16 bytes): 16 flag words
    # per slot, 4 bits per row
    off = rows * 1024 + (rows * 8 + 15) // 16 * 16
    words = dec.workspace[off: off + dec.plan.max_partials * 64].view(torch.int32).cpu().numpy().view(np.uint32)
    flags = np.stack([(words >> (4 * j)) & 15 for j in range(8)], axis=1).reshape(-1)
    # only the slots the plan uses were written; the rest of the region is uninitialised
    say("  partial rows with a low half:", int((flags != 0).sum()))
    assert (flags != 0).sum() > 1000
    compare(o, l, ref_o, ref_l, "large cancelling partials")


@pytest.mark.parametrize("H", [128, 16])
@pytest.mark.parametrize("mode", ["unsplit", "split2"])
def test_late_score_spike_takes_the_second_pass(mode, H):
    """One page in the middle of each sequence gets its keys' rope dims scaled by 40
    (values untouched): its scores sit tens of log2 units above the first page's maxima,
    so the page sums pass 2^16 and the workgroup decodes its range again from an upper
    bound of every row's scores.  Some rows' sums pass the cap through many large terms
    rather than one.  Out and lse must still meet the oracle."""
    import mla_decode_03_amd as mla
    from mla_inputs import bf16_bits_to_f32, f32_to_bf16_bits
    case = _case(3, 1, H, [1000, 300, 64 * 5], seed=91)
    for b, j in [(0, 7), (1, 2), (2, 4)]:
        pg = int(case.block_table[b, j])
        x = case.kv[pg].copy()
        x[:, 512:] *= np.float32(40.0)
        bits = f32_to_bf16_bits(x).reshape(x.shape)
        case.kv_bits[pg] = bits
        case.kv[pg] = bf16_bits_to_f32(bits).reshape(bits.shape)
    say("score spike", mode, H, case.cache_seqlens.tolist())
    ref_o, ref_l = oracle_rows(case)
    # the spike dominates: each sequence's lse is far above its first block's
    first = oracle.decode_case(_first_blocks(case, 1))[1]
    assert np.all(ref_l - first > 16.0 * np.log(2.0))
    if mode == "unsplit":
        o, l, _ = run(case, split=False)
    else:
        o, l, _ = run(case, options=mla.PlanOptions(fixed_split_blocks=2))
    compare(o, l, ref_o, ref_l, "score spike " + mode)


def _first_blocks(case, n):
    """The same case cut to each sequence's first n blocks."""
    import dataclasses
    lens = np.minimum(case.cache_seqlens, 64 * n).astype(np.int32)
    return dataclasses.replace(case, cache_seqlens=lens)


@pytest.mark.parametrize("rs", [2, 4])
def test_row_split(rs):
    import mla_decode_03_amd as mla
    case = _case(3, 1, 128, [700, 64, 1], seed=11 + rs)
    say("row_split", rs)
    ref_o, ref_l = oracle_rows(case)
    o, l, _ = run(case, options=mla.PlanOptions(num_workgroups=24, min_blocks_per_wg=1, row_split=rs))
    compare(o, l, ref_o, ref_l, "row_split=%d" % rs)


def test_page_permutation_is_bit_exact_and_deterministic():
    import torch
    case = _case(3, 1, 128, [500, 130, 64], seed=21)
    q, kv, bt, lens = to_device(case)
    o1, l1, dec = run(case, tensors=(q, kv, bt, lens))
    o1b, l1b, _ = run(case, tensors=(q, kv, bt, lens), decoder=dec)
    assert np.array_equal(o1, o1b) and np.array_equal(l1, l1b)       # run-to-run identical
    perm = torch.from_numpy(np.random.default_rng(5).permutation(case.num_pages)).cuda()
    kv2 = torch.empty_like(kv)
    kv2[perm] = kv
    bt2 = torch.where(bt >= 0, perm[bt.clamp(min=0).long()].int(), bt)
    o2, l2, _ = run(case, tensors=(q, kv2, bt2, lens), decoder=dec)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_poisoned_unused_slots_never_leak():
    case = _case(3, 2, 16, [70, 129, 2], seed=31, causal=True, extra_pages=3)
    poison_unused(case)
    say("poison")
    ref_o, ref_l = oracle_rows(case)
    for split in (True, False):
        o, l, _ = run(case, split=split)
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(l[np.isfinite(ref_l)]))
        compare(o, l, ref_o, ref_l, "poison split=%s" % split)


def test_device_plan_matches_mirror():
    import torch
    import mla_decode_03_amd as mla
    from plan_mirror import make_plan, to_words
    rng = np.random.default_rng(3)
    lens = [int(x) for x in rng.integers(0, 5000, size=37)]
    case = _case(37, 1, 128, lens, seed=41)
    q, kv, bt, lt = to_device(case)
    for opts in (mla.PlanOptions(num_workgroups=256, min_blocks_per_wg=4),
                 mla.PlanOptions(num_workgroups=50, min_blocks_per_wg=1, row_split=2)):
        dec = mla.Decoder(q, kv, bt, options=opts, num_cus=256)
        plan = dec.plan_for(lt)
        torch.cuda.synchronize()
        words = plan.metadata.view(torch.int32).cpu().numpy()
        ref = make_plan(lens, row_split=opts.row_split or 1, grid_wg=opts.num_workgroups,
                        min_blocks=opts.min_blocks_per_wg)
        hdr, arrays = to_words(ref, opts.num_workgroups, 128, plan.max_partials,
                               case.block_table.shape[1])
        assert list(words[:16]) == hdr
        assert list(words[16:16 + len(arrays)]) == arrays


@pytest.mark.parametrize("kind", ["auto", "pages", "cost", "row_split2", "fixed", "h16", "sparse", "even",
                                  "wide", "wide512", "b300", "few_cost"])
def test_plan_in_decode_matches_planner(kind):
    """A plan made with plan_in_decode = 1 and reused: every decode launch re-plans from the
    lengths it is given.  Its outputs equal the planner-kernel path's bit for bit, the
    metadata it leaves for the combine equals the CPU mirror's words, and a later step
    with other lengths (same plan object) equals a fresh plan for those lengths.  The kinds
    reach each form of the in-launch planning: registers only (even), the cut tables
    (ragged batches up to 256 sequences: auto, pages, cost, h16, wide, and wide512, whose
    512 workgroups take each thread's pricing loop twice) and the general
    block-wide computation (row split, fixed chunks, 300 sequences, and few_cost, whose
    sequences could each hold more cuts than the tables take)."""
    import torch
    import mla_decode_03_amd as mla
    from mla_inputs import make_topk_indices
    from plan_mirror import make_plan, to_words
    rng = np.random.default_rng(71)
    H = 16 if kind == "h16" else 128
    lens = [int(x) for x in rng.integers(0, 3000, size=23)]
    lens[3] = 0
    if kind == "even":       # every sequence 16 blocks, shares of 4 blocks: the equal-share cut
        lens = [1000] * 40
    elif kind in ("wide", "wide512", "b300"):
        lens = [int(x) for x in rng.integers(0, 1200, size=300 if kind == "b300" else 200)]
        lens[5] = lens[77] = 0
    elif kind == "few_cost":  # three sequences of up to 313 blocks over 512 workgroups
        lens = [20000, 7, 19000]
    case = _case(len(lens), 1, H, lens, seed=72, extra_pages=40)
    say("plan in decode", kind)
    q, kv, bt, lt = to_device(case)
    base = dict(num_workgroups=160 if kind == "even" else 96, min_blocks_per_wg=2)
    base.update({"auto": {}, "pages": dict(split_rule=1), "cost": dict(split_rule=2), "row_split2": dict(row_split=2),
                 "fixed": dict(fixed_split_blocks=5), "h16": {}, "sparse": {}, "even": {},
                 "wide": dict(num_workgroups=256), "b300": dict(num_workgroups=256),
                 "wide512": dict(num_workgroups=512, min_blocks_per_wg=1),
                 "few_cost": dict(num_workgroups=512, min_blocks_per_wg=1, split_rule=2)}[kind])
    topk, ix = 0, None
    if kind == "sparse":
        idx = make_topk_indices(case.cache_seqlens, case.q_len, 100, seed=3)
        topk, ix = 100, torch.from_numpy(idx).to(q.device)
    fused = mla.Decoder(q, kv, bt, options=mla.PlanOptions(plan_in_decode=1, **base), num_cus=256, topk=topk)
    plain = mla.Decoder(q, kv, bt, options=mla.PlanOptions(**base), num_cus=256, topk=topk)
    later = [max(0, x - 700) for x in lens] if kind != "even" else [x + 24 for x in lens]
    for step, lv in enumerate((lens, later)):
        lt2 = torch.tensor(lv, dtype=torch.int32, device=q.device)
        o1, l1 = fused(q, kv, bt, lt2, case.scale, indices=ix)
        o2, l2 = plain(q, kv, bt, lt2, case.scale, indices=ix)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), (kind, step)
        assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), (kind, step)
        if kind != "sparse":
            words = fused.metadata.view(torch.int32).cpu().numpy()
            ref = make_plan(lv, row_split=base.get("row_split", 1), grid_wg=fused.plan.grid_wg,
                            min_blocks=base["min_blocks_per_wg"], max_blocks=case.block_table.shape[1],
                            rule={0: "auto", 1: "pages", 2: "cost"}[base.get("split_rule", 0)],
                            fixed_blocks=base.get("fixed_split_blocks", 0), rows=H)
            hdr, arrays = to_words(ref, fused.plan.grid_wg, H, fused.plan.max_partials, case.block_table.shape[1])
            assert list(words[:16]) == hdr, (kind, step)
            assert list(words[16:16 + len(arrays)]) == arrays, (kind, step)


@pytest.mark.parametrize("rule", [0, 1, 2])
def test_device_plan_rules_match_mirror(rule):
    """Both partition rules and the cost model's choice, bit for bit against the mirror:
    a ragged batch kept in LDS and a 5000-sequence batch (row_split 2) that is not."""
    import torch
    import mla_decode_03_amd as mla
    from plan_mirror import RULES, make_plan, to_words
    name = {v: k for k, v in RULES.items()}[rule]
    rng = np.random.default_rng(9 + rule)
    for B, rs, grid, hi, segq in ((61, 1, 256, 9000, 0), (5000, 2, 256, 300, 0), (40, 4, 100, 3000, 23)):
        lens = [int(x) for x in rng.integers(0, hi, size=B)]
        lens[3] = 0
        maxb = (max(lens) + 63) // 64 + 1
        prob = mla.Problem(batch=B, q_len=1, num_heads=128, causal=0, num_pages=1, block_table_stride=maxb,
                           max_blocks_per_seq=maxb, dtype=mla.DTYPE_BF16)
        opts = mla.PlanOptions(num_workgroups=grid, min_blocks_per_wg=1, row_split=rs, split_rule=rule,
                               segment_cost=segq)
        meta = torch.empty(mla.metadata_bytes(prob, opts, 256), dtype=torch.uint8, device="cuda")
        lt = torch.tensor(lens, dtype=torch.int32, device="cuda")
        plan = mla.get_metadata(prob, lt, meta, opts, 256)
        torch.cuda.synchronize()
        words = meta.view(torch.int32).cpu().numpy()
        ref = make_plan(lens, row_split=rs, grid_wg=grid, min_blocks=1, rule=name, seg_q=segq or None)
        hdr, arrays = to_words(ref, grid, 128, plan.max_partials, maxb)
        say("plan rule %s B=%d rs=%d: kept rule %d, worst pages %d cost %d" % (name, B, rs, ref["rule"],
                                                                             ref["cost_pages"], ref["cost_balanced"]))
        assert list(words[:16]) == hdr
        assert list(words[16:16 + len(arrays)]) == arrays


def test_device_fixed_plan_matches_mirror():
    import torch
    import mla_decode_03_amd as mla
    from plan_mirror import make_plan, to_words
    rng = np.random.default_rng(4)
    lens = [int(x) for x in rng.integers(0, 5000, size=29)]
    lens[5] = 0
    case = _case(29, 1, 128, lens, seed=42)
    q, kv, bt, lt = to_device(case)
    maxb = case.block_table.shape[1]
    for C, rs in ((3, 1), (16, 2), (1, 1)):
        opts = mla.PlanOptions(fixed_split_blocks=C, row_split=rs)
        dec = mla.Decoder(q, kv, bt, options=opts, num_cus=256)
        plan = dec.plan_for(lt)
        torch.cuda.synchronize()
        grid = 29 * rs * (-(-maxb // C))
        assert plan.grid_wg == grid and plan.max_partials == grid
        words = plan.metadata.view(torch.int32).cpu().numpy()
        ref = make_plan(lens, row_split=rs, grid_wg=grid, fixed_blocks=C)
        hdr, arrays = to_words(ref, grid, 128, plan.max_partials, maxb)
        say("fixed plan C=%d rs=%d: %d chunks of %d slots" % (C, rs, ref["num_wg"], grid))
        assert list(words[:16]) == hdr
        assert list(words[16:16 + len(arrays)]) == arrays


@pytest.mark.parametrize("H, sparse", [(128, False), (16, False), (128, True)])
def test_timed_decode_matches_untimed(H, sparse):
    """mla_decode_splits_timed writes what mla_decode_splits writes, bit for bit, and its
    events time the decode kernel (a positive duration, below the whole enqueue-to-sync time)."""
    import time
    import torch
    import mla_decode_03_amd as mla
    from mla_inputs import make_topk_indices
    case = _case(3, 1, H, [300, 1000, 65], seed=61)
    say("timed decode", H, sparse)
    q, kv, bt, lens = to_device(case)
    topk, ix = 0, None
    if sparse:
        idx = make_topk_indices(case.cache_seqlens, case.q_len, 64, seed=5)
        topk, ix = 64, torch.from_numpy(idx).to(q.device)
    dec = mla.Decoder(q, kv, bt, causal=case.causal, topk=topk)
    plan = dec.plan_for(lens)
    R = case.q_len * H
    results = []
    for timed in (False, True):
        out = torch.zeros((case.batch, case.q_len, H, 512), dtype=torch.bfloat16, device=q.device)
        lse = torch.zeros((case.batch, case.q_len, H), dtype=torch.float32, device=q.device)
        dec.workspace.zero_()
        ev = None
        if timed:
            ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for e in ev:
                e.record()                   # creates the events
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        mla.decode_splits(dec.problem, q, kv, bt, lens, case.scale, out, lse, plan, dec.workspace,
                          indices=ix, events=ev)
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3
        if timed:
            ms = ev[0].elapsed_time(ev[1])
            say("  kernel %.4f ms, enqueue to sync %.4f ms" % (ms, wall_ms))
            assert 0.0 < ms <= wall_ms
        results.append((out.view(torch.int16).cpu().numpy(), lse.cpu().numpy(), dec.workspace.cpu().numpy()))
    (o0, l0, w0), (o1, l1, w1) = results
    assert np.array_equal(o0, o1) and np.array_equal(l0.view(np.int32), l1.view(np.int32))
    assert np.array_equal(w0, w1)


def test_fixed_split_plan_is_batch_invariant():
    """With fixed-size splits a sequence's output bits do not depend on the rest of the
    batch (its position, its neighbours, the batch size) nor on the CU count; the balanced
    plan gives no such promise.  Every run also meets the oracle."""
    import torch
    import mla_decode_03_amd as mla
    lens = [3000, 129, 777, 64, 2500, 1]
    case = _case(len(lens), 1, 128, lens, seed=71)
    q, kv, bt, lt = to_device(case)
    ref_o, ref_l = oracle_rows(case)
    R = 128
    opts = mla.PlanOptions(fixed_split_blocks=4)

    def decode(idx, num_cus):
        ix = torch.tensor(idx, device=q.device)
        qs, bts, ls = q[ix].contiguous(), bt[ix].contiguous(), lt[ix].contiguous()
        dec = mla.Decoder(qs, kv, bts, options=opts, num_cus=num_cus)
        out, lse = dec(qs, kv, bts, ls, case.scale)
        torch.cuda.synchronize()
        return (out.view(torch.int16).cpu().numpy().reshape(len(idx), R, 512),
                lse.cpu().numpy().reshape(len(idx), R))

    full_o, full_l = decode(list(range(len(lens))), 256)
    o64 = full_o.view(np.uint16).astype(np.uint32) << 16
    compare(o64.view(np.float32).astype(np.float64).reshape(-1, 512), full_l.reshape(-1).astype(np.float64),
            ref_o, ref_l, "fixed splits, whole batch")
    for idx, cus in (([4, 0], 256), ([2, 2, 0, 5, 1], 80), ([0], 7), ([3, 4, 1, 0, 2, 5, 4], 256)):
        say("  invariance", idx, cus)
        o, l = decode(idx, cus)
        for j, b in enumerate(idx):
            assert np.array_equal(o[j], full_o[b]), (idx, j, b)
            assert np.array_equal(l[j].view(np.uint32), full_l[b].view(np.uint32)), (idx, j, b)


def test_bad_page_is_flagged_and_poisoned():
    import mla_decode_03_amd as mla
    case = _case(3, 1, 128, [200, 300, 100], seed=51)
    case.block_table[1, 2] = case.num_pages + 1000      # out of the pool
    say("bad page")
    q, kv, bt, lens = to_device(case)
    o, l, dec = run(case, tensors=(q, kv, bt, lens))
    assert dec.plan.error() == mla._abi.MLA_ERR_BAD_INPUT
    assert dec.plan.error() == 0                          # the flag was cleared
    R = 128
    assert np.all(np.isnan(o[R:2 * R])) and np.all(np.isnan(l[R:2 * R]))
    good = np.r_[0:R, 2 * R:3 * R]
    case.block_table[1, 2] = 0
    ref_o, ref_l = oracle_rows(case, rows=good)
    compare(o[good], l[good], ref_o, ref_l, "other sequences")


def test_tolerance_is_not_vacuous():
    """The elementwise bound alone is loose at long lengths; the relative-L2 gate is what
    catches a wrong kernel.  A plausible bug (V taken from the wrong 512 columns) must fail."""
    case = _case(1, 1, 16, [4096], seed=61)
    ref_o, ref_l = oracle_rows(case)
    o, l, _ = run(case)
    compare(o, l, ref_o, ref_l, "baseline")
    case2 = _case(1, 1, 16, [4096], seed=61)
    case2.kv[..., :512] = case2.kv[..., 64:576]          # the mistake, made in the oracle input
    case2.kv_bits = None
    bad_o, _ = oracle_rows(_case_f32(case2))
    with pytest.raises(AssertionError):
        compare(o, l, bad_o, ref_l, "wrong-V oracle")
    assert ATOL > 0


def test_fp32_bad_page_is_flagged_and_poisoned():
    """The float32 path takes a plan only for the fault flag: a bad page poisons its
    sequence and raises the flag; the other sequences are untouched."""
    import mla_decode_03_amd as mla
    case = _case(3, 1, 16, [200, 300, 100], seed=52, dtype="f32")
    case.block_table[1, 3] = -5
    q, kv, bt, lens = to_device(case)
    o, l, dec = run(case, tensors=(q, kv, bt, lens))
    assert dec.plan is not None
    assert dec.plan.error() == mla._abi.MLA_ERR_BAD_INPUT
    assert dec.plan.error() == 0
    R = 16
    assert np.all(np.isnan(o[R:2 * R])) and np.all(np.isnan(l[R:2 * R]))
    good = np.r_[0:R, 2 * R:3 * R]
    case.block_table[1, 3] = 0
    ref_o, ref_l = oracle_rows(case, rows=good)
    compare(o[good], l[good], ref_o, ref_l, "fp32 other sequences")


def _case_f32(case):
    case.dtype = "f32"
    return case


# ---- attention sinks (mla_decode_ex) -----------------------------------------------------

SINK_CASES = [
    (2, 1, 128, [1, 70], False),
    (3, 1, 128, [0, 50, 4097], False),
    (3, 2, 16, [1, 3, 64], True),
    (2, 1, 48, [130, 77], False),
]


@pytest.mark.parametrize("mode", ["plan", "forced_splits", "unsplit", "fixed_splits"])
@pytest.mark.parametrize("B,T,H,lens,causal", SINK_CASES)
def test_sink_parity(B, T, H, lens, causal, mode):
    """Sinks enter once per row: in the decode epilogue for unsplit ranges, in the combine
    for split ones; every plan must meet the oracle with sinks."""
    import mla_decode_03_amd as mla
    from mla_inputs import make_sinks
    case = _case(B, T, H, lens, seed=500 + B * 10 + T + H, causal=causal)
    sinks = make_sinks(H, seed=H + T)
    say("sink", B, T, H, lens, causal, mode)
    ref_o, ref_l = oracle_rows(case, sinks=sinks)
    kw = {"unsplit": dict(split=False),
          "forced_splits": dict(options=mla.PlanOptions(num_workgroups=7, min_blocks_per_wg=1)),
          "fixed_splits": dict(options=mla.PlanOptions(fixed_split_blocks=1)),
          "plan": {}}[mode]
    o, l, _ = run(case, sinks=sinks, **kw)
    compare(o, l, ref_o, ref_l, "sink %s" % mode)


def test_sink_fp32_path():
    from mla_inputs import make_sinks
    case = _case(2, 2, 16, [0, 200], seed=77, causal=True, dtype="f32")
    sinks = make_sinks(16, seed=5, lo=-2.0, hi=8.0)
    ref_o, ref_l = oracle_rows(case, sinks=sinks)
    o, l, _ = run(case, sinks=sinks)
    s = compare(o, l, ref_o, ref_l, "sink fp32")
    assert s["max_abs"] < 1e-4


def test_sink_minus_inf_is_bit_identical_to_plain():
    case = _case(3, 1, 128, [700, 64, 0], seed=78)
    q, kv, bt, lens = to_device(case)
    o0, l0, dec = run(case, tensors=(q, kv, bt, lens))
    o1, l1, _ = run(case, tensors=(q, kv, bt, lens), decoder=dec, sinks=np.full(128, -np.inf, np.float32))
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_sink_full_headline_every_row():
    """The benchmark's workload and launch configuration (default plan, computed inside the
    decode launch), with sinks, every row."""
    import mla_decode_03_amd as mla
    from mla_inputs import make_sinks
    case = make_config(1)
    sinks = make_sinks(case.num_heads, seed=1)
    o, l, _ = run(case, sinks=sinks, options=mla.PlanOptions(plan_in_decode=1))
    ref_o, ref_l = oracle_rows(case, sinks=sinks)
    compare(o, l, ref_o, ref_l, "config1 sinks, all %d rows" % o.shape[0])


# ---- sparse (top-k) decode --------------------------------------------------------------

SPARSE_CASES = [
    # (B, T, H, lens, topk, pad_frac, dup_frac)
    (2, 1, 128, [300, 5000], 128, 0.1, 0.05),
    (3, 2, 64, [100, 2000, 64], 200, 0.3, 0.0),
    (2, 1, 16, [70, 1], 64, 0.0, 0.0),          # sequence 1 lists one token, 63 unused
    (2, 2, 128, [4100, 900], 700, 0.05, 0.02),  # 256 rows per sequence: one unit per (b, t)
]


@pytest.mark.parametrize("mode", ["plan", "forced_splits", "fixed_splits", "pages_rule"])
@pytest.mark.parametrize("B,T,H,lens,topk,pad,dup", SPARSE_CASES)
def test_sparse_parity(B, T, H, lens, topk, pad, dup, mode):
    import mla_decode_03_amd as mla
    from mla_inputs import make_topk_indices
    case = _case(B, T, H, lens, seed=600 + B + T + H + topk)
    idx = make_topk_indices(case.cache_seqlens, T, topk, seed=topk + B, pad_frac=pad, dup_frac=dup)
    say("sparse", B, T, H, lens, topk, mode)
    ref_o, ref_l = oracle_rows(case, indices=idx)
    kw = {"plan": {}, "forced_splits": dict(options=mla.PlanOptions(num_workgroups=7, min_blocks_per_wg=1)),
          "fixed_splits": dict(options=mla.PlanOptions(fixed_split_blocks=1)),
          "pages_rule": dict(options=mla.PlanOptions(split_rule=1))}[mode]
    o, l, _ = run(case, indices=idx, **kw)
    compare(o, l, ref_o, ref_l, "sparse %s" % mode)


def test_sparse_with_sinks_and_empty_lists():
    from mla_inputs import make_sinks, make_topk_indices
    case = _case(3, 1, 128, [800, 60, 3000], seed=71)
    idx = make_topk_indices(case.cache_seqlens, 1, 256, seed=3, pad_frac=0.2)
    idx[1] = -1                                   # nothing listed: out 0, lse = the sink
    sinks = make_sinks(128, seed=9)
    ref_o, ref_l = oracle_rows(case, sinks=sinks, indices=idx)
    o, l, _ = run(case, sinks=sinks, indices=idx)
    compare(o, l, ref_o, ref_l, "sparse + sinks")
    assert np.all(o[128:256] == 0) and np.allclose(l[128:256], sinks, atol=1e-6)


def test_sparse_full_list_matches_the_dense_decode():
    """Listing every position in order reads the same keys in the same blocks.  With
    one-block splits both paths cut every sequence at the same block edges (the sparse
    units' blocks past their lists are empty partials of weight 0, and every unit is
    split, so every row goes through the merge), and at 64 heads, where the sparse and
    dense decodes run one schedule, their outputs agree bit for bit.  (The dense 128-row
    decode runs a schedule of its own, which the sparse lists do not use.)"""
    import mla_decode_03_amd as mla
    L = [1000, 4096, 130]
    case = _case(3, 1, 64, L, seed=72)
    topk = 4096
    idx = np.full((3, 1, topk), -1, np.int32)
    for b, n in enumerate(L):
        idx[b, 0, :n] = np.arange(n)
    opts = mla.PlanOptions(fixed_split_blocks=1)
    o_d, l_d, _ = run(case, options=opts)
    o_s, l_s, _ = run(case, options=opts, indices=idx)
    ref_o, ref_l = oracle_rows(case)
    compare(o_s, l_s, ref_o, ref_l, "sparse full list")
    assert np.array_equal(o_s, o_d) and np.array_equal(l_s, l_d)
    o_128, l_128, _ = run(_case(3, 1, 128, L, seed=72), options=opts, indices=idx)
    ref_o, ref_l = oracle_rows(_case(3, 1, 128, L, seed=72))
    compare(o_128, l_128, ref_o, ref_l, "sparse full list, 128 heads")


def test_sparse_bad_entry_is_flagged_and_poisoned():
    import mla_decode_03_amd as mla
    from mla_inputs import make_topk_indices
    case = _case(3, 1, 128, [200, 300, 100], seed=73)
    idx = make_topk_indices(case.cache_seqlens, 1, 96, seed=4)
    idx[1, 0, 5] = 300                            # sequence 1 holds 300 tokens: out of range
    q, kv, bt, lens = to_device(case)
    o, l, dec = run(case, tensors=(q, kv, bt, lens), indices=idx)
    assert dec.plan.error() == mla._abi.MLA_ERR_BAD_INPUT
    R = 128
    assert np.all(np.isnan(o[R:2 * R])) and np.all(np.isnan(l[R:2 * R]))
    good = np.r_[0:R, 2 * R:3 * R]
    ref_o, ref_l = oracle_rows(case, rows=good, indices=np.where(idx == 300, -1, idx))
    compare(o[good], l[good], ref_o, ref_l, "other lists")


# ---- capture, large batches, capacity edges -----------------------------------------------

def test_graph_capture_replays_match_eager():
    """Planner + decode (+ combine) captured in a HIP graph: nothing allocates or
    synchronises, so every replay reproduces the eager result bit for bit, with eager
    work on the stream between replays."""
    import torch
    import mla_decode_03_amd as mla
    case = _case(4, 1, 128, [700, 64, 1, 3000], seed=81)
    q, kv, bt, lens = to_device(case)
    dec = mla.Decoder(q, kv, bt, num_cus=256)
    out = torch.empty((4, 1, 128, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((4, 1, 128), dtype=torch.float32, device="cuda")
    dec(q, kv, bt, lens, case.scale, out, lse)
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=side):
        dec(q, kv, bt, lens, case.scale, out, lse)
    torch.cuda.synchronize()
    for r in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        scratch = torch.randn(1 << 20, device="cuda") * r     # unrelated eager work
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16)), r
        assert torch.equal(lse.view(torch.int32), ref_l.view(torch.int32)), r
        del scratch
    o = ref_o.float().cpu().numpy().astype(np.float64).reshape(-1, 512)
    l = ref_l.cpu().numpy().astype(np.float64).reshape(-1)
    ref = oracle_rows(case)
    compare(o, l, ref[0], ref[1], "graph")


def test_batch_beyond_the_planners_lds_path():
    """4200 sequences (the planner keeps its prefix sums in global memory past 4095),
    cost-model plan, decoded end to end; every row against the oracle."""
    rng = np.random.default_rng(82)
    lens = [int(x) for x in rng.integers(0, 130, size=4200)]
    case = _case(4200, 1, 16, lens, seed=82)
    say("batch 4200, pages", case.num_pages)
    o, l, dec = run(case)
    assert dec.plan.error() == 0
    ref_o, ref_l = oracle_rows(case)
    compare(o, l, ref_o, ref_l, "batch 4200, every row")


def test_lengths_at_and_past_the_block_table():
    """L = 64 * max_blocks_per_seq is served; one token more is an input fault: that
    sequence's rows are NaN, the flag is raised, the other sequences are untouched."""
    import mla_decode_03_amd as mla
    case = _case(3, 1, 128, [320, 100, 7], seed=83)      # block table: 5 columns
    assert case.block_table.shape[1] == 5
    ref_o, ref_l = oracle_rows(case)
    o, l, dec = run(case)
    assert dec.plan.error() == 0
    compare(o, l, ref_o, ref_l, "L at capacity")
    case.cache_seqlens[0] = 321
    q, kv, bt, lens = to_device(case)
    o2, l2, dec2 = run(case, tensors=(q, kv, bt, lens))
    assert dec2.plan.error() == mla._abi.MLA_ERR_BAD_INPUT
    assert np.all(np.isnan(o2[:128])) and np.all(np.isnan(l2[:128]))
    compare(o2[128:], l2[128:], ref_o[128:], ref_l[128:], "others")


@pytest.mark.parametrize("mode", [0, 1])
def test_hbm_read_probe_streams(mode):
    """The streaming-read probe runs in both modes (vector loads; the decode's global->LDS
    copies) over 64 MiB with the default workgroup count and with an explicit one, and
    reports a plausible rate.  Its sink is never the thing checked (unspecified)."""
    import torch
    import mla_decode_03_amd as mla
    say("hbm probe", mode)
    src = torch.arange(16 << 20, dtype=torch.int32, device="cuda")   # 64 MiB
    sink = torch.zeros(4 * 1024, dtype=torch.int32, device="cuda")
    mla.hbm_read_probe(src, mode, sink)
    mla.hbm_read_probe(src, mode, sink, num_workgroups=64)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        mla.hbm_read_probe(src, mode, sink)
    e1.record()
    torch.cuda.synchronize()
    gbs = 5 * src.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    say("  %.0f GB/s" % gbs)
    assert gbs > 200.0
