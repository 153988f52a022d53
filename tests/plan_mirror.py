"""CPU statement of the split planner's partition rule (test helper, no product code).

Every sequence b contributes `row_split` units of nblk_b = ceil(L_b / 64) blocks; the
units are laid end to end (sequence-major, then row slice) and the block range
[0, total) is cut into num_wg shares [floor(w*total/num_wg), floor((w+1)*total/num_wg)).
num_wg = min(grid_wg, ceil(total / min_blocks)), at least 1 when total > 0.  A unit cut
across k > 1 workgroups owns k consecutive partial slots, numbered unit by unit.

Written from the rule, not from the kernel: the workgroup holding a position is found
by a linear search here (the kernel uses a closed form), so the bit-exact comparison of
the device plan against this mirror checks that closed form too.
"""
from __future__ import annotations

PAGE = 64


def make_plan(seqlens, *, row_split=1, grid_wg=256, min_blocks=4, max_blocks=1 << 30, fixed_blocks=0):
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
    wg_begin = [(w * total // num_wg) if (num_wg > 0 and w <= num_wg) else total
                for w in range(grid_wg + 1)]

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
                first_wg=first_wg, part_off=part_off, num_partials=slot, row_split=row_split, batch=B)


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
                first_wg=first_wg, part_off=part_off, num_partials=slot, row_split=row_split, batch=B)


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


def to_words(plan, grid_wg, rows, max_partials, max_blocks, error=0):
    """The metadata buffer's int32 words as the device planner writes them."""
    B, rs = plan["batch"], plan["row_split"]
    hdr = [0x4D4C4150, B, rows, rs, rows // rs, plan["num_wg"], grid_wg, plan["total"],
           plan["num_partials"], error, max_partials, max_blocks, 0, 0, 0, 0]
    return hdr[:12], (plan["cu_blocks"] + plan["num_splits"] + plan["first_wg"] + plan["part_off"]
                      + plan["wg_begin"])
