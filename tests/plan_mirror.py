"""CPU statement of the split planner's partition rules (test helper, no product code).

Every sequence b contributes `row_split` units of nblk_b = ceil(L_b / 64) blocks; the
units are laid end to end (sequence-major, then row slice) and the block range
[0, total) is cut into num_wg = min(grid_wg, ceil(total / min_blocks)) workgroup ranges
(at least 1 when total > 0), by one of two rules:
  pages  equal block shares [floor(w*total/num_wg), floor((w+1)*total/num_wg));
  cost   equal shares of a cost axis on which every non-empty unit takes c quarter
         blocks of segment overhead and then 4 quarters per block (cuts in an
         overhead move to the unit's first block, cuts in its blocks round down).
A workgroup costs 4 per block plus c per unit it touches; rule "auto" keeps the rule
whose busiest workgroup costs less, pages on a tie.  It skips the comparison (and keeps
pages, header costs 0) when every non-empty unit holds the same nb blocks and the equal
shares line up with them (share a multiple of nb or nb of share).  c defaults to the step-time
model's time per segment over its time per block at the row count, in quarters, rounded.  A unit cut
across k > 1 workgroups owns k consecutive partial slots, numbered unit by unit.

Written from the rules, not from the kernel: the workgroup holding a position is found
by a linear search here (the kernel uses closed forms), so the bit-exact comparison of
the device plan against this mirror checks those closed forms too.
"""
from __future__ import annotations

import bisect

PAGE = 64


RULES = {"auto": 0, "pages": 1, "cost": 2, "fixed": 3}


def segment_cost(rows_per_wg):
    """Default per-segment overhead in quarter blocks (nearest): the step-time model's 7.61 us
    per segment over its time per block, max(2.31 us from HBM, 2.86 us * rows / 128 of MFMA
    work), in hundredths of a microsecond and integers."""
    blk = max(231 * 128, 286 * rows_per_wg)
    return (4 * 761 * 128 + blk // 2) // blk


def make_plan(seqlens, *, row_split=1, grid_wg=256, min_blocks=4, max_blocks=1 << 30, fixed_blocks=0,
              rule="auto", seg_q=None, rows=128):
    """rule "pages", "cost" or "auto" (see the module docstring); seg_q overrides c."""
    B = len(seqlens)
    nblk = [min((max(int(L), 0) + PAGE - 1) // PAGE, max_blocks) for L in seqlens]
    cu = [0]
    for n in nblk:
        cu.append(cu[-1] + n)
    total = row_split * cu[B]
    if fixed_blocks > 0:
        return _fixed_plan(nblk, cu, total, row_split, grid_wg, fixed_blocks)
    num_wg = 0
    if total > 0:
        num_wg = max(1, min(grid_wg, -(-total // min_blocks)))
    c = seg_q if seg_q else segment_cost(rows // row_split)
    pages = [(w * total // num_wg) if (num_wg > 0 and w <= num_wg) else total for w in range(grid_wg + 1)]
    costed = (_cost_bounds(nblk, cu, total, row_split, num_wg, c) + [total] * (grid_wg - num_wg)
              if num_wg > 0 else pages)
    worst_p = worst_c = 0
    used = [n for n in nblk if n > 0]
    aligned_even = False
    if used and num_wg > 0 and min(used) == max(used) and total % num_wg == 0:
        share, nbm = total // num_wg, max(used)
        aligned_even = share % nbm == 0 or nbm % share == 0
    if rule == "auto" and num_wg > 0 and not aligned_even:
        base = dict(cu_blocks=cu, num_wg=num_wg, row_split=row_split, batch=B)
        worst_p = plan_cost(dict(base, wg_begin=pages), c)
        worst_c = plan_cost(dict(base, wg_begin=costed), c)
    use_cost = rule == "cost" or (rule == "auto" and worst_c < worst_p)
    wg_begin = costed if use_cost else pages

    def wg_of(x):
        w = 0
        while w + 1 < num_wg and wg_begin[w + 1] <= x:
            w += 1
        return w

    units = B * row_split
    num_splits, first_wg, part_off = [], [], []
    slot = 0
    for u in range(units):
        b, g = divmod(u, row_split)
        nb = nblk[b]
        if nb == 0:
            num_splits.append(0)
            first_wg.append(-1)
        else:
            start = row_split * cu[b] + g * nb
            f, last = wg_of(start), wg_of(start + nb - 1)
            num_splits.append(last - f + 1)
            first_wg.append(f)
        part_off.append(slot)
        if num_splits[-1] > 1:
            slot += num_splits[-1]
    return dict(cu_blocks=cu, num_wg=num_wg, total=total, wg_begin=wg_begin, num_splits=num_splits,
                first_wg=first_wg, part_off=part_off, num_partials=slot, row_split=row_split, batch=B,
                rule=RULES["cost" if use_cost else "pages"], cost_pages=worst_p, cost_balanced=worst_c,
                seg_cost=c)


def _cost_bounds(nblk, cu, total, row_split, num_wg, c):
    """Workgroup boundaries (block positions, num_wg + 1 of them) that cut the cost axis
    into equal integer shares.  On that axis each non-empty unit occupies c quarters of
    overhead followed by 4 quarters per block; a cut that lands in a unit's overhead
    moves to the unit's first block, one inside its blocks rounds down to a block."""
    zones = []            # (cost start, block start, blocks) of each non-empty unit
    cost = 0
    for u in range(len(nblk) * row_split):
        b, g = divmod(u, row_split)
        nb = nblk[b]
        if nb == 0:
            continue
        zones.append((cost, row_split * cu[b] + g * nb, nb))
        cost += c + 4 * nb
    ctot = cost

    starts = [z[0] for z in zones]

    def block_at(x):
        if x >= ctot:
            return total
        s0, p0, nb = zones[bisect.bisect_right(starts, x) - 1]
        off = x - s0
        return p0 if off < c else p0 + (off - c) // 4

    return [block_at(w * ctot // num_wg) for w in range(num_wg + 1)]


def plan_cost(plan, c):
    """Largest per-workgroup cost of a plan, in quarter blocks: 4 per block plus c per
    segment (each unit a workgroup touches)."""
    worst = 0
    for w in range(plan["num_wg"]):
        lo, hi = plan["wg_begin"][w], plan["wg_begin"][w + 1]
        if hi <= lo:
            continue
        segs = sum(1 for x in segments_of_range(plan, lo, hi))
        worst = max(worst, 4 * (hi - lo) + c * segs)
    return worst


def segments_of_range(plan, lo, hi):
    rs, cu = plan["row_split"], plan["cu_blocks"]
    pos = lo
    while pos < hi:
        b = bisect.bisect_right(cu, pos // rs, 0, plan["batch"]) - 1   # last b with cu[b] <= pos / rs
        nb = cu[b + 1] - cu[b]
        g = (pos - rs * cu[b]) // nb
        unit_start = rs * cu[b] + g * nb
        yield (b, g)
        pos = unit_start + nb


def _fixed_plan(nblk, cu, total, row_split, grid_wg, fixed):
    """Batch-invariant rule: each unit cut into chunks of `fixed` blocks from its own
    start, one chunk per workgroup, chunks numbered unit by unit."""
    B = len(nblk)
    wg_begin, num_splits, first_wg, part_off = [], [], [], []
    slot = 0
    for u in range(B * row_split):
        b, g = divmod(u, row_split)
        nb = nblk[b]
        start = row_split * cu[b] + g * nb
        k = -(-nb // fixed) if nb > 0 else 0
        first_wg.append(len(wg_begin) if k > 0 else -1)
        num_splits.append(k)
        part_off.append(slot)
        if k > 1:
            slot += k
        wg_begin += [start + i * fixed for i in range(k)]
    num_wg = len(wg_begin)
    wg_begin += [total] * (grid_wg + 1 - num_wg)
    return dict(cu_blocks=cu, num_wg=num_wg, total=total, wg_begin=wg_begin, num_splits=num_splits,
                first_wg=first_wg, part_off=part_off, num_partials=slot, row_split=row_split, batch=B,
                rule=RULES["fixed"], cost_pages=0, cost_balanced=0, seg_cost=0)


def segments(plan):
    """Walk every workgroup's share the way the decode kernel does: yields
    (wg, b, g, blk_lo, blk_hi, slot)."""
    rs, cu = plan["row_split"], plan["cu_blocks"]
    out = []
    for w in range(plan["num_wg"]):
        pos, end = plan["wg_begin"][w], plan["wg_begin"][w + 1]
        while pos < end:
            b = max(i for i in range(plan["batch"]) if rs * cu[i] <= pos)
            nb = cu[b + 1] - cu[b]
            g = (pos - rs * cu[b]) // nb
            unit_start = rs * cu[b] + g * nb
            u = b * rs + g
            lo, hi = pos - unit_start, min(end - unit_start, nb)
            slot = plan["part_off"][u] + (w - plan["first_wg"][u]) if plan["num_splits"][u] > 1 else -1
            out.append((w, b, g, lo, hi, slot))
            pos = unit_start + hi
    return out


def wg_seq(plan, grid_wg):
    """The sequence holding each workgroup's first block (0 past the workgroups with work)."""
    rs, cu, total = plan["row_split"], plan["cu_blocks"], plan["total"]
    out = []
    for w in range(grid_wg):
        p = plan["wg_begin"][w]
        seq = 0
        if w < plan["num_wg"] and p < total:
            seq = max(i for i in range(plan["batch"]) if rs * cu[i] <= p)
        out.append(seq)
    return out


def to_words(plan, grid_wg, rows, max_partials, max_blocks, error=0):
    """The metadata buffer's int32 words as the device planner writes them."""
    B, rs = plan["batch"], plan["row_split"]
    hdr = [0x4D4C4150, B, rows, rs, rows // rs, plan["num_wg"], grid_wg, plan["total"],
           plan["num_partials"], error, max_partials, max_blocks, plan["rule"], plan["cost_pages"],
           plan["cost_balanced"], plan["seg_cost"]]
    return hdr, (plan["cu_blocks"] + plan["num_splits"] + plan["first_wg"] + plan["part_off"]
                      + plan["wg_begin"] + wg_seq(plan, grid_wg))
