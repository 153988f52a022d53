"""Offline sweep of the split planner's options: measured step time against the cost model.

    python -m mla_decode_03_amd.tune --config 1 [--steps 40] [--out table.md]

For one seeded workload, every candidate plan (split rule x workgroup count x row split x
smallest share, plus the batch-invariant fixed-chunk plans) is made by the device planner
and timed as the whole decode path (plan, split decode, combine) with HIP events, two KV
pools alternated as in the benchmark, in round-robin passes (a new seeded order each pass)
after a settling run; the median over passes is reported.  Beside each time stands the planner's own cost model
applied to the plan it made: the TileLang notes' tile recommender ranks candidates by
traffic over bandwidth ("Key design 2: tile recommendation"), and here a workgroup costs 4
quarter blocks per 64-token block it streams plus the per-segment overhead (the header's
segment cost, or for fixed-chunk plans the default one) for each unit it touches.  Workgroups are dealt to the CUs in launch order,
each taking the first CU to come free (one resident workgroup per CU), and the busiest CU's
total is the predicted time.  The report gives the rank agreement of prediction and
measurement, and where the default plan (cost model picks the rule, one workgroup per CU)
lands.  Every candidate's output is compared with the default plan's.
"""
from __future__ import annotations

import argparse
import heapq
import json
import sys

import numpy as np

HDR_WORDS = 16
HDR_ROW_SPLIT, HDR_ROWS_PER_WG, HDR_NUM_WG, HDR_GRID_WG, HDR_RULE, HDR_SEG_COST = 3, 4, 5, 6, 12, 15
RULE_NAMES = {1: "pages", 2: "cost", 3: "fixed"}


def plan_arrays(words: np.ndarray, batch: int):
    """Split the planner's int32 words into (header, cu_blocks, wg_begin)."""
    rs = int(words[HDR_ROW_SPLIT])
    units = batch * rs
    cu = words[HDR_WORDS:HDR_WORDS + batch + 1].astype(np.int64)
    wg0 = HDR_WORDS + batch + 1 + 3 * units
    grid = int(words[HDR_GRID_WG])
    return words[:HDR_WORDS], cu, words[wg0:wg0 + grid + 1].astype(np.int64)


def workgroup_costs(words: np.ndarray, batch: int) -> np.ndarray:
    """Cost of each launched workgroup in quarter blocks: 4 per block of its range plus the
    segment cost per unit the range touches (0 for a workgroup without work)."""
    hdr, cu, wg_begin = plan_arrays(words, batch)
    rs, num_wg, c = int(hdr[HDR_ROW_SPLIT]), int(hdr[HDR_NUM_WG]), int(hdr[HDR_SEG_COST])
    if c == 0:   # fixed-chunk plans record none: the default, a segment's rows at 2180 B each
        c = (4 * int(hdr[HDR_ROWS_PER_WG]) * 2180 + 36864) // 73728   # over a 73,728 B block
    nb = np.diff(cu)
    # start of every non-empty unit on the concatenated block axis (sequence-major)
    starts = np.array([rs * cu[b] + g * nb[b] for b in range(batch) if nb[b] > 0 for g in range(rs)],
                      dtype=np.int64)
    cost = np.zeros(len(wg_begin) - 1, dtype=np.int64)
    for w in range(min(num_wg, len(cost))):
        lo, hi = wg_begin[w], wg_begin[w + 1]
        if hi <= lo:
            continue
        first = np.searchsorted(starts, lo, side="right") - 1
        last = np.searchsorted(starts, hi - 1, side="right") - 1
        cost[w] = 4 * (hi - lo) + c * (last - first + 1)
    return cost


def makespan(costs: np.ndarray, num_cus: int) -> int:
    """Busiest CU when the grid's workgroups are started in launch order, each on the first CU
    to come free.  Launch index i runs logical workgroup (i mod 8) * (G / 8) + i div 8 when the
    grid G is a multiple of 8 (the decode's XCD-aware numbering), else i."""
    G = len(costs)
    order = ([(i & 7) * (G >> 3) + (i >> 3) for i in range(G)] if G % 8 == 0 else list(range(G)))
    free = [0] * max(1, num_cus)
    for w in order:
        t = heapq.heappop(free)
        heapq.heappush(free, t + int(costs[w]))
    return max(free)


def spearman(x, y) -> float:
    """Rank correlation (average ranks for ties)."""
    def ranks(a):
        a = np.asarray(a, dtype=np.float64)
        order = np.argsort(a, kind="stable")
        r = np.empty(len(a))
        i = 0
        while i < len(a):
            j = i
            while j + 1 < len(a) and a[order[j + 1]] == a[order[i]]:
                j += 1
            r[order[i:j + 1]] = 0.5 * (i + j)
            i = j + 1
        return r
    rx, ry = ranks(x), ranks(y)
    if rx.std() == 0 or ry.std() == 0:
        return float("nan")
    return float(np.corrcoef(rx, ry)[0, 1])


def candidates(rows: int):
    """The sweep: (label, PlanOptions fields) pairs; the default plan first."""
    out = [("default", {})]
    for rs in (1, 2, 4):
        if rows % rs or rows // rs < 1:
            continue
        for nwg in (128, 192, 256, 384, 512):
            for minb in (4, 16):
                for rule in (1, 2):
                    out.append(("%s rs%d wg%d min%d" % (RULE_NAMES[rule], rs, nwg, minb),
                                dict(row_split=rs, num_workgroups=nwg, min_blocks_per_wg=minb, split_rule=rule)))
        for chunk in (4, 8, 16, 32, 64):
            out.append(("fixed%d rs%d" % (chunk, rs), dict(row_split=rs, fixed_split_blocks=chunk)))
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--config", type=int, default=1, help="seeded workload index (bf16 ones: 1..4)")
    ap.add_argument("--steps", type=int, default=100, help="timed steps per candidate and round")
    ap.add_argument("--warmup", type=int, default=10, help="untimed steps before each timing")
    ap.add_argument("--rounds", type=int, default=5, help="round-robin passes; the median is reported")
    ap.add_argument("--settle", type=int, default=1000, help="untimed steps before the first round")
    ap.add_argument("--out", default=None, help="also write the table (markdown) here")
    args = ap.parse_args(argv)

    import torch
    import mla_decode_03_amd as mla
    from mla_inputs import CONFIGS, make_config

    case = make_config(args.config)
    if case.dtype != "bf16":
        sys.exit("the split planner serves the bf16 workloads (1..4)")
    dev = torch.device("cuda:0")
    q = torch.from_numpy(case.q_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    kv_a = torch.from_numpy(case.kv_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    pools = (kv_a, kv_a.clone())
    bt = torch.from_numpy(case.block_table).to(dev)
    lens = torch.from_numpy(case.cache_seqlens).to(dev)
    B, T, H = case.batch, case.q_len, case.num_heads
    rows = T * H
    num_cus = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = torch.cuda.current_stream()

    # every candidate's plan and buffers, made once
    runs = []
    for label, fields in candidates(rows):
        opts = mla.PlanOptions(**fields) if fields else None
        dec = mla.Decoder(q, kv_a, bt, causal=case.causal, split=True, options=opts)
        out = torch.empty((B, T, H, 512), dtype=q.dtype, device=dev)
        lse = torch.empty((B, T, H), dtype=torch.float32, device=dev)
        runs.append((label, dec, out, lse))

    def step(run, i):
        _, dec, out, lse = run
        plan = dec.plan_for(lens, stream)
        mla.decode(dec.problem, q, pools[i & 1], bt, lens, case.scale, out, lse, plan, dec.workspace, stream)

    def time_steps(run, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(n):
            step(run, i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    time_steps(runs[0], args.settle)   # clocks and caches settle before anything is timed
    times = [[] for _ in runs]
    # round-robin in a fresh seeded order each round, so drift, and what the candidate before
    # left behind (clock, caches), spread over every candidate
    for r in range(args.rounds):
        for k in np.random.default_rng(r).permutation(len(runs)):
            run = runs[k]
            for i in range(args.warmup):
                step(run, i)
            times[k].append(time_steps(run, args.steps))
        print("round %d of %d done" % (r + 1, args.rounds), flush=True)

    ref_out = runs[0][2].float()
    results = []
    for k, (label, dec, out, lse) in enumerate(runs):
        if dec.plan.error(stream):
            raise RuntimeError("planner flagged an input fault for %s" % label)
        words = dec.metadata.view(torch.int32).cpu().numpy()
        d = (out.float() - ref_out).abs()
        if not bool((d <= 2e-2 + 1e-2 * ref_out.abs()).all()):
            raise RuntimeError("%s: output differs from the default plan's beyond tolerance" % label)
        rec = {"label": label, "rule": RULE_NAMES.get(int(words[HDR_RULE]), "?"),
               "row_split": int(words[HDR_ROW_SPLIT]), "num_wg": int(words[HDR_NUM_WG]),
               "grid_wg": int(words[HDR_GRID_WG]), "model": makespan(workgroup_costs(words, B), num_cus),
               "us": round(float(np.median(times[k])), 2), "spread_us": round(max(times[k]) - min(times[k]), 2),
               "max_abs_vs_default": float(d.max())}
        results.append(rec)
        print(json.dumps(rec), flush=True)

    best = min(results, key=lambda r: r["us"])
    default = results[0]
    rank = 1 + sum(r["us"] < default["us"] for r in results)
    rho = spearman([r["model"] for r in results], [r["us"] for r in results])
    by_model = min(results, key=lambda r: (r["model"], r["us"]))
    lines = ["Workload: %s (%d candidate plans; µs per step = planner + decode + combine, median of %d "
             "shuffled round-robin rounds of %d timed steps)" % (CONFIGS[args.config]["name"], len(results), args.rounds,
                                                          args.steps), "",
             "Default plan: %.2f µs, rank %d of %d; fastest: %s at %.2f µs (default / fastest = %.3f)."
             % (default["us"], rank, len(results), best["label"], best["us"], default["us"] / best["us"]),
             "Model's pick (lowest busiest-CU cost): %s at %.2f µs.  Spearman rank correlation of "
             "model cost and measured time: %.3f." % (by_model["label"], by_model["us"], rho), "",
             "| plan | rule used | row split | workgroups with work / launched | model (quarter blocks, busiest CU) "
             "| µs per step | spread over rounds | max abs diff vs default |", "|---|---|---|---|---|---|---|---|"]
    for r in sorted(results, key=lambda r: r["us"]):
        lines.append("| %s | %s | %d | %d / %d | %d | %.2f | %.2f | %.3g |" % (
            r["label"], r["rule"], r["row_split"], r["num_wg"], r["grid_wg"], r["model"], r["us"],
            r["spread_us"], r["max_abs_vs_default"]))
    text = "\n".join(lines)
    print(text, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text + "\n")


if __name__ == "__main__":
    main()
