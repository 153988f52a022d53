"""Properties of the split partition rule (CPU, on the mirror in plan_mirror.py)."""
import numpy as np
import pytest

from plan_mirror import make_plan, plan_cost, segment_cost, segments


def _check(plan, seqlens, rs, max_partials):
    nblk = [(max(L, 0) + 63) // 64 for L in seqlens]
    segs = segments(plan)
    # every unit's blocks are covered exactly once
    cover = {}
    for (w, b, g, lo, hi, slot) in segs:
        assert 0 <= lo < hi <= nblk[b]
        cover.setdefault((b, g), []).append((lo, hi, w, slot))
    for b, nb in enumerate(nblk):
        for g in range(rs):
            if nb == 0:
                assert (b, g) not in cover
                continue
            parts = sorted(cover[(b, g)])
            assert parts[0][0] == 0 and parts[-1][1] == nb
            for (l0, h0, _, _), (l1, _, _, _) in zip(parts, parts[1:]):
                assert h0 == l1
            u = b * rs + g
            assert plan["num_splits"][u] == len(parts)
            slots = [p[3] for p in parts]
            if len(parts) == 1:
                assert slots == [-1]
            else:
                assert slots == list(range(plan["part_off"][u], plan["part_off"][u] + len(parts)))
    shares = [plan["wg_begin"][w + 1] - plan["wg_begin"][w] for w in range(plan["num_wg"])]
    if shares:
        assert min(shares) >= 0 and sum(shares) == plan["total"]
        if plan["rule"] == 1:
            # pages rule: shares balanced to within one block
            assert max(shares) - min(shares) <= 1
        elif plan["rule"] == 2:
            # cost rule: no workgroup exceeds its share of the cost axis by more than one
            # segment overhead plus one block (a cut rounds down by less than that)
            c = plan["seg_cost"]
            ne_units = sum(1 for L in seqlens if L > 0) * rs
            ctot = 4 * plan["total"] + c * ne_units
            n = plan["num_wg"]
            assert plan_cost(plan, c) <= -(-ctot // n) + c + 3
    # partial slots are unique and fit the workspace bound
    used = [s for (*_, s) in segs if s >= 0]
    assert len(used) == len(set(used)) == plan["num_partials"] <= max_partials


@pytest.mark.parametrize("seed", range(12))
def test_random_plans(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 40))
    seqlens = [int(x) for x in rng.integers(0, 3000, size=B)]
    rs = [1, 2, 4][seed % 3]
    grid = int(rng.integers(1, 300))
    minb = int(rng.integers(1, 9))
    plan = make_plan(seqlens, row_split=rs, grid_wg=grid, min_blocks=minb)
    _check(plan, seqlens, rs, grid + min(grid, B * rs))


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("rule", ["pages", "cost"])
def test_random_plans_each_rule(seed, rule):
    rng = np.random.default_rng(100 + seed)
    B = int(rng.integers(1, 60))
    seqlens = [int(x) for x in rng.integers(0, 5000, size=B)]
    seqlens[int(rng.integers(0, B))] = 0
    rs = [1, 2, 4][seed % 3]
    grid = int(rng.integers(1, 300))
    plan = make_plan(seqlens, row_split=rs, grid_wg=grid, min_blocks=int(rng.integers(1, 9)), rule=rule,
                     seg_q=int(rng.integers(0, 30)) or None)
    assert plan["rule"] == (1 if rule == "pages" else 2)
    _check(plan, seqlens, rs, grid + min(grid, B * rs))


@pytest.mark.parametrize("seed", range(8))
def test_auto_keeps_the_cheaper_rule(seed):
    rng = np.random.default_rng(200 + seed)
    B = int(rng.integers(2, 200))
    seqlens = [int(x) for x in rng.integers(1, 8193, size=B)]
    c = segment_cost(128)
    auto = make_plan(seqlens, grid_wg=256)
    pages = make_plan(seqlens, grid_wg=256, rule="pages")
    cost = make_plan(seqlens, grid_wg=256, rule="cost")
    wp, wc = plan_cost(pages, c), plan_cost(cost, c)
    assert (auto["cost_pages"], auto["cost_balanced"]) == (wp, wc)
    assert plan_cost(auto, c) == min(wp, wc)
    assert auto["wg_begin"] == (cost if wc < wp else pages)["wg_begin"]


@pytest.mark.parametrize("seed", range(10))
def test_aligned_even_batches_need_no_comparison(seed):
    """The shortcut's claim: with equal units and shares lined up with them, no cut of
    either rule (nor any seg cost) beats the pages rule's busiest workgroup."""
    rng = np.random.default_rng(300 + seed)
    nb = int(rng.choice([1, 2, 4, 8, 16, 64]))
    B = int(rng.integers(1, 80))
    rs = [1, 2, 4][seed % 3]
    lens = [nb * 64 if rng.random() < 0.8 else 0 for _ in range(B)]
    if not any(lens):
        lens[0] = nb * 64
    total = rs * nb * sum(1 for L in lens if L)
    shares = [d for d in range(1, total + 1) if total % d == 0 and (d % nb == 0 or nb % d == 0)]
    share = int(rng.choice(shares))
    grid = total // share
    c = int(rng.integers(1, 40))
    auto = make_plan(lens, row_split=rs, grid_wg=grid, min_blocks=1, seg_q=c)
    assert auto["rule"] == 1 and auto["num_wg"] == grid
    cost = make_plan(lens, row_split=rs, grid_wg=grid, min_blocks=1, rule="cost", seg_q=c)
    assert plan_cost(auto, c) <= plan_cost(cost, c)


def test_segment_cost_is_the_models_segment_time_in_blocks():
    # 7.61 us per segment; a block takes 2.86 us of MFMA work at 128 rows (MFMA-bound:
    # 10.6 blocks -> 11 quarters) and 2.31 us from HBM at 64 rows or fewer (13.2 -> 13)
    assert segment_cost(128) == 11 and segment_cost(64) == 13 and segment_cost(32) == 13
    assert segment_cost(16) == 13 and segment_cost(104) == 13 and segment_cost(96) == 13


def test_even_batches_keep_the_pages_cut_and_ragged_ones_take_the_cost_cut():
    even = make_plan([4096] * 64, grid_wg=256)
    assert even["rule"] == 1 and (even["cost_pages"], even["cost_balanced"]) == (0, 0)   # not compared
    c = segment_cost(128)
    assert plan_cost(make_plan([4096] * 64, grid_wg=256, rule="pages"), c) < \
        plan_cost(make_plan([4096] * 64, grid_wg=256, rule="cost"), c)
    rng = np.random.default_rng(7)
    ragged = make_plan([int(x) for x in rng.integers(1, 2049, size=256)], grid_wg=256)
    assert ragged["rule"] == 2 and ragged["cost_balanced"] < ragged["cost_pages"]


def test_headline_shape_splits_each_sequence_in_four():
    plan = make_plan([4096] * 64, grid_wg=256, min_blocks=4)
    assert plan["num_wg"] == 256 and set(plan["num_splits"]) == {4}
    assert plan["num_partials"] == 256
    _check(plan, [4096] * 64, 1, 512)


def test_small_problem_is_not_over_split_and_empty_batch():
    # 2 + 4 blocks with at least 4 per workgroup: two workgroups.  The pages rule cuts
    # at block 3 and splits the second sequence in two (busiest workgroup: 3 blocks and
    # 2 segments, 12 + 2*11 = 34 quarters); the cost rule gives each sequence its own
    # workgroup (busiest: 4 blocks and 1 segment, 27), so the cost model keeps that.
    plan = make_plan([100, 200], grid_wg=256, min_blocks=4, rule="pages")
    assert plan["num_wg"] == 2 and plan["num_splits"] == [1, 2] and plan["num_partials"] == 2
    plan = make_plan([100, 200], grid_wg=256, min_blocks=4)
    assert (plan["cost_pages"], plan["cost_balanced"]) == (34, 27)
    assert plan["rule"] == 2 and plan["num_splits"] == [1, 1] and plan["num_partials"] == 0
    plan = make_plan([100, 200], grid_wg=256, min_blocks=8)
    assert plan["num_wg"] == 1 and plan["num_splits"] == [1, 1] and plan["num_partials"] == 0
    plan = make_plan([0, 0], grid_wg=8)
    assert plan["num_wg"] == 0 and plan["num_splits"] == [0, 0] and segments(plan) == []


def test_fixed_split_plan_is_aligned_and_batch_invariant():
    """Batch-invariant mode: chunks start at each sequence's own start, hold at most C
    blocks, and a sequence's chunking is the same whatever else is in the batch."""
    C = 4
    rng = np.random.default_rng(12)
    lens = [int(x) for x in rng.integers(0, 3000, size=9)]

    def chunks_of(plan, b):
        return [(lo, hi) for (_, bb, _, lo, hi, _) in segments(plan) if bb == b]

    plan = make_plan(lens, grid_wg=10000, fixed_blocks=C)
    for b, L in enumerate(lens):
        nb = -(-L // 64)
        ch = chunks_of(plan, b)
        assert ch == [(s, min(s + C, nb)) for s in range(0, nb, C)]
        assert plan["num_splits"][b] == len(ch)
    # the same sequence in another batch, at another position
    other = [17, lens[3], 5000, 1]
    plan2 = make_plan(other, grid_wg=10000, fixed_blocks=C)
    assert chunks_of(plan2, 1) == chunks_of(plan, 3)
    # every chunk of a split sequence owns one slot, in chunk order
    for (w, b, g, lo, hi, slot) in segments(plan):
        if plan["num_splits"][b] > 1:
            assert slot == plan["part_off"][b] + lo // C
