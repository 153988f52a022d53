"""Host logic of the plan sweep (mla_decode_03_amd.tune): per-workgroup costs read from a
plan's words, the launch-order makespan and the rank correlation.  The costs are checked
against the plan mirror's own segment walk on plans the mirror makes."""
import random

import numpy as np
import pytest

from mla_decode_03_amd import tune
from plan_mirror import make_plan, segment_cost, segments_of_range, to_words


def _expected_costs(plan, c, grid):
    out = []
    for w in range(grid):
        lo, hi = plan["wg_begin"][w], plan["wg_begin"][w + 1]
        n = 0 if (w >= plan["num_wg"] or hi <= lo) else 4 * (hi - lo) + c * len(list(segments_of_range(plan, lo, hi)))
        out.append(n)
    return out


@pytest.mark.parametrize("rs", [1, 2, 4])
@pytest.mark.parametrize("rule", ["pages", "cost", "fixed"])
def test_workgroup_costs_match_the_mirror(rule, rs):
    rng = random.Random(17 * rs + len(rule))
    for _ in range(15):
        B = rng.randint(1, 40)
        lens = [rng.choice([0, rng.randint(1, 5000), rng.randint(1, 300)]) for _ in range(B)]
        fixed = rng.choice([2, 8, 16]) if rule == "fixed" else 0
        grid = rng.choice([8, 16, 64, 256]) if not fixed else 4 * B * rs * 79 // fixed + 8
        plan = make_plan(lens, row_split=rs, grid_wg=grid, rule="pages" if fixed else rule,
                         fixed_blocks=fixed, rows=128)
        c = segment_cost(128 // rs)
        hdr, body = to_words(plan, grid, 128, max_partials=1 << 30, max_blocks=1 << 30)
        words = np.array(hdr + body, dtype=np.int64)
        assert tune.workgroup_costs(words, B).tolist() == _expected_costs(plan, c, grid)


def test_makespan_hand_cases():
    # 2 CUs, launch order = logical order when the grid is not a multiple of 8
    assert tune.makespan(np.array([5, 3, 2, 2]), 2) == 7
    # grid of 16: launch index i runs logical (i mod 8) * 2 + i div 8, so the even logical
    # workgroups start first; logical 1 (cost 100) starts after eight cost-1 ones
    costs = np.ones(16, dtype=np.int64)
    costs[1] = 100
    assert tune.makespan(costs, 2) == 104
    assert tune.makespan(costs, 16) == 100
    assert tune.makespan(np.array([4, 4, 4]), 1) == 12


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
