"""Host logic of the plan sweep (mla_decode_03_amd.tune): per-workgroup costs read from a
plan's words, the launch-order makespan and the rank correlation.  The costs are checked
against the plan mirror's own segment walk on plans the mirror makes."""
import random

import numpy as np
import pytest

from mla_decode_03_amd import tune
from plan_mirror import make_plan, segments_of_range, to_words


def _blocks_in_range(plan, lo, hi):
    """Blocks of each unit the range [lo, hi) touches, from the mirror's segment walk."""
    rs, cu = plan["row_split"], plan["cu_blocks"]
    out = []
    for b, g in segments_of_range(plan, lo, hi):
        nb = cu[b + 1] - cu[b]
        start = rs * cu[b] + g * nb
        out.append(min(hi, start + nb) - max(lo, start))
    return out


@pytest.mark.parametrize("rs", [1, 2, 4])
@pytest.mark.parametrize("rule", ["pages", "cost", "fixed"])
def test_plan_segments_match_the_mirror(rule, rs):
    """Blocks per segment of every workgroup, read from a plan's words, against the mirror's
    own segment walk; a segment is split exactly when its unit spans several workgroups."""
    rng = random.Random(17 * rs + len(rule))
    for _ in range(15):
        B = rng.randint(1, 40)
        lens = [rng.choice([0, rng.randint(1, 5000), rng.randint(1, 300)]) for _ in range(B)]
        fixed = rng.choice([2, 8, 16]) if rule == "fixed" else 0
        grid = rng.choice([8, 16, 64, 256]) if not fixed else 4 * B * rs * 79 // fixed + 8
        plan = make_plan(lens, row_split=rs, grid_wg=grid, rule="pages" if fixed else rule,
                         fixed_blocks=fixed, rows=128)
        hdr, body = to_words(plan, grid, 128, max_partials=1 << 30, max_blocks=1 << 30)
        words = np.array(hdr + body, dtype=np.int64)
        segs, R = tune.plan_segments(words, B)
        assert R == 128 // rs
        for w, s in enumerate(segs):
            lo, hi = plan["wg_begin"][w], plan["wg_begin"][w + 1]
            want = [] if (w >= plan["num_wg"] or hi <= lo) else _blocks_in_range(plan, lo, hi)
            assert [n for n, _ in s] == want
        # the partial segments are the ones whose unit the plan splits
        n_split = sum(1 for s in segs for _, sp in s if sp)
        assert n_split == sum(ns for ns in plan["num_splits"] if ns > 1)


def test_dispatch_hand_cases():
    # grid 3 (not a multiple of 8): launch order = logical order, one XCD of one CU each
    assert tune.dispatch([5, 3, 2], 8) == 5
    # 16 workgroups, 8 CUs (one per XCD): launch index i runs logical (i mod 8) * 2 + i div 8
    # on XCD i mod 8, so XCD x runs logical 2x and 2x + 1
    costs = [1.0] * 16
    costs[3] = 10.0
    assert tune.dispatch(costs, 8) == 11.0
    assert tune.dispatch([4.0, 4.0, 4.0], 8) == 4.0


def test_model_terms():
    """One 128-row plan by hand: 2 sequences of 4 blocks over 2 workgroups, one each."""
    plan = make_plan([256, 256], grid_wg=2, min_blocks=1, rule="pages", rows=128)
    hdr, body = to_words(plan, 2, 128, max_partials=8, max_blocks=8)
    p = dict(t_mem=1.0, t_mfma=2.0, t_seg=3.0, t_fix=10.0, t_part=0.5)
    # each workgroup: one whole segment of 4 blocks at max(1, 2 * 128/128) = 2 us
    assert tune.model_us(p, np.array(hdr + body), 2, 256) == pytest.approx(10.0 + 3.0 + 4 * 2.0)
    # 64 rows per workgroup: blocks take max(1, 2 * 64/128) = 1 us
    plan = make_plan([256, 256], row_split=2, grid_wg=4, min_blocks=1, rule="pages", rows=128)
    hdr, body = to_words(plan, 4, 128, max_partials=8, max_blocks=8)
    assert tune.model_us(p, np.array(hdr + body), 2, 256) == pytest.approx(10.0 + 3.0 + 4 * 1.0)


def test_spearman():
    assert tune.spearman([1, 2, 3, 4], [10, 20, 30, 40]) == pytest.approx(1.0)
    assert tune.spearman([1, 2, 3, 4], [4, 3, 2, 1]) == pytest.approx(-1.0)
    # ties take the average rank: ranks (0.5, 0.5, 2) against (0, 1, 2)
    r = tune.spearman([1, 1, 2], [1, 2, 3])
    assert r == pytest.approx(np.corrcoef([0.5, 0.5, 2], [0, 1, 2])[0, 1])


def test_candidate_list():
    c = tune.candidates(128)
    assert c[0] == ("default", {})
    labels = [x[0] for x in c]
    assert len(labels) == len(set(labels))
    assert 60 <= len(c) <= 110
    # rows 32 (16 heads x 2 tokens) still takes row splits 1, 2 and 4
    assert {f.get("row_split") for _, f in tune.candidates(32)[1:]} == {1, 2, 4}
