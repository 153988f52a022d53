"""Offline sweep of the split planner's options: measured step time against the step-time model.

    python -m mla_decode_03_amd.tune --config 1 [--steps 40] [--out table.md] [--dump sweep.json]
    python -m mla_decode_03_amd.tune fit sweep1.json sweep2.json ... [--out profiles/plan_cost_model.json]

For one seeded workload, every candidate plan (split rule x workgroup count x row split x
smallest share, plus the batch-invariant fixed-chunk plans) is made by the device planner
and timed as the whole decode path (plan, split decode, combine) with HIP events, two KV
pools alternated as in the benchmark, in round-robin passes (a new seeded order each pass)
after a settling run; the median over passes is reported.  Beside each time stands the
step-time model's prediction for the plan (see PARAM_NAMES below: the TileLang notes' tile
recommender, "Key design 2: tile recommendation", in its roofline form: per block the larger
of memory and MFMA time, plus intrinsic per-segment and per-step terms; workgroups dealt to
XCDs and CUs in launch order).  The report gives the rank agreement of prediction and
measurement, and where the default plan (cost model picks the rule, one workgroup per CU)
lands.  Every candidate's output is compared with the default plan's.  `fit` measures the
model's parameters from sweep dumps, with the rank agreement of each workload also checked
with that workload left out of the fit.
"""
from __future__ import annotations

import argparse
import heapq
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
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


# The step-time model, in the form of the TileLang notes' tile recommender ("Key design
# 2: tile recommendation"): a kernel's time is the largest of its traffic over bandwidth
# and its compute over throughput, plus an intrinsic term for launch, prologue and
# epilogue.  For the split decode:
#   block     each 64-token KV block a workgroup streams takes max(t_mem, t_mfma * R / 128):
#             the HBM time of its 73,728 B at one CU's share of the stream, or the MFMA time
#             of its two products for R rows (R = rows per workgroup);
#   segment   each unit a workgroup touches adds t_seg (its Q rows and first pages in, its
#             output or partial rows out);
#   launch    workgroups go to the XCDs in launch order (index i to XCD i mod 8, the
#             decode's own numbering maps it to a logical workgroup) and there to the CU
#             that comes free first; the decode ends with the busiest CU;
#   step      + t_fix (the planner, the launches, the combine's fixed part)
#             + t_part * R / 128 per partial segment the combine merges.
# The parameters are measured: fitted (least squares on log time) to the sweep's timings,
# the figures in profiles/plan_cost_model.json.
PARAM_NAMES = ("t_mem", "t_mfma", "t_seg", "t_fix", "t_part")
MODEL_FILE = os.path.join(ROOT, "profiles", "plan_cost_model.json")


def plan_segments(words: np.ndarray, batch: int):
    """Per launched workgroup, its segments as (blocks, split) pairs (split: the unit is cut
    across workgroups, so this segment writes a partial); rows per workgroup."""
    hdr, cu, wg_begin = plan_arrays(words, batch)
    rs, num_wg = int(hdr[HDR_ROW_SPLIT]), int(hdr[HDR_NUM_WG])
    nb = np.diff(cu)
    starts, lens = [], []
    for b in range(batch):
        if nb[b] > 0:
            for g in range(rs):
                starts.append(rs * cu[b] + g * nb[b])
                lens.append(nb[b])
    starts = np.array(starts, dtype=np.int64)
    out = []
    for w in range(len(wg_begin) - 1):
        lo, hi = wg_begin[w], wg_begin[w + 1]
        segs = []
        if w < num_wg and hi > lo:
            i = int(np.searchsorted(starts, lo, side="right")) - 1
            while i < len(starts) and starts[i] < hi:
                s0, s1 = max(lo, starts[i]), min(hi, starts[i] + lens[i])
                segs.append((int(s1 - s0), bool(s0 > starts[i] or s1 < starts[i] + lens[i])))
                i += 1
        out.append(segs)
    return out, int(hdr[HDR_ROWS_PER_WG])


def dispatch(costs, num_cus: int) -> float:
    """Busiest CU when launch index i goes to XCD i mod 8 and there to the CU that comes free
    first; launch index i runs logical workgroup (i mod 8) * (G / 8) + i div 8 when the grid
    G is a multiple of 8 (the decode's XCD-aware numbering), else i."""
    G = len(costs)
    order = [(i & 7) * (G >> 3) + (i >> 3) for i in range(G)] if G % 8 == 0 else list(range(G))
    xcds = [[0.0] * max(1, num_cus // 8) for _ in range(8)]
    for i, w in enumerate(order):
        h = xcds[i & 7]
        t = heapq.heappop(h)
        heapq.heappush(h, t + float(costs[w]))
    return max(max(h) for h in xcds)


def model_us(params: dict, words: np.ndarray, batch: int, num_cus: int) -> float:
    """Predicted microseconds per step (planner + decode + combine) of a plan."""
    segs, R = plan_segments(words, batch)
    blk = max(params["t_mem"], params["t_mfma"] * R / 128.0)
    costs = [sum(params["t_seg"] + n * blk for n, _ in s) for s in segs]
    parts = sum(1 for s in segs for _, split in s if split)
    return params["t_fix"] + dispatch(costs, num_cus) + params["t_part"] * parts * R / 128.0


def load_params(path: str = MODEL_FILE) -> dict:
    with open(path) as f:
        return json.load(f)["params"]


def fit(dumps, out=None):
    """Fit the model's parameters to sweep dumps (`--dump` files): least squares on the log
    of the step time over every candidate of every workload, and the rank agreement per
    workload, with all workloads in the fit and with the workload left out of it."""
    from scipy.optimize import least_squares
    data = []
    for path in dumps:
        with open(path) as f:
            d = json.load(f)
        for c in d["candidates"]:
            segs_R = np.array(c["words"], dtype=np.int64)
            data.append((d["workload"], segs_R, d["batch"], d["num_cus"], c["us"]))
    names = sorted({w for w, *_ in data}, key=lambda w: [x[0] for x in data].index(w))

    def solve(rows):
        def resid(p):
            prm = dict(zip(PARAM_NAMES, p))
            return [np.log(model_us(prm, wd, b, n)) - np.log(us) for _, wd, b, n, us in rows]
        r = least_squares(resid, [2.5, 2.5, 6.0, 15.0, 0.1], bounds=([0.1] * 2 + [0.0] * 3, [50.0] * 2 + [100.0] * 3))
        return dict(zip(PARAM_NAMES, (round(float(x), 4) for x in r.x))), float(np.sqrt(np.mean(np.square(r.fun))))

    params, rms = solve(data)
    report = {"params": params, "rms_log_error": round(rms, 4), "workloads": {}}
    for w in names:
        rows = [x for x in data if x[0] == w]
        rho = spearman([model_us(params, wd, b, n) for _, wd, b, n, _ in rows], [us for *_, us in rows])
        held, _ = solve([x for x in data if x[0] != w])
        rho_held = spearman([model_us(held, wd, b, n) for _, wd, b, n, _ in rows], [us for *_, us in rows])
        report["workloads"][w] = {"candidates": len(rows), "spearman": round(rho, 4),
                                  "spearman_left_out_of_fit": round(rho_held, 4), "params_without_it": held}
    text = json.dumps(report, indent=1)
    if out:
        with open(out, "w") as f:
            f.write(text + "\n")
    print(text)
    return report


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
    argv = sys.argv[1:] if argv is None else argv
    if argv and argv[0] == "fit":
        fp = argparse.ArgumentParser(prog="tune fit", description="fit the step-time model to sweep dumps")
        fp.add_argument("dumps", nargs="+")
        fp.add_argument("--out", default=None)
        fa = fp.parse_args(argv[1:])
        fit(fa.dumps, fa.out)
        return
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--config", type=int, default=1, help="seeded workload index (bf16 ones: 1..4)")
    ap.add_argument("--steps", type=int, default=100, help="timed steps per candidate and round")
    ap.add_argument("--warmup", type=int, default=10, help="untimed steps before each timing")
    ap.add_argument("--rounds", type=int, default=5, help="round-robin passes; the median is reported")
    ap.add_argument("--settle", type=int, default=1000, help="untimed steps before the first round")
    ap.add_argument("--out", default=None, help="also write the table (markdown) here")
    ap.add_argument("--dump", default=None, help="also write every candidate's plan words and times (JSON)")
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

    params = load_params() if os.path.exists(MODEL_FILE) else None
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
               "grid_wg": int(words[HDR_GRID_WG]),
               "model": round(model_us(params, words, B, num_cus), 2) if params else float("nan"),
               "us": round(float(np.median(times[k])), 2), "spread_us": round(max(times[k]) - min(times[k]), 2),
               "max_abs_vs_default": float(d.max())}
        results.append(rec)
        print(json.dumps(rec), flush=True)
        rec["times_us"] = [round(x, 3) for x in times[k]]
        rec["words"] = words.tolist()

    best = min(results, key=lambda r: r["us"])
    default = results[0]
    rank = 1 + sum(r["us"] < default["us"] for r in results)
    rho = spearman([r["model"] for r in results], [r["us"] for r in results])
    by_model = min(results, key=lambda r: r["model"])   # the first of equal predictions, in sweep order
    lines = ["Workload: %s (%d candidate plans; µs per step = planner + decode + combine, median of %d "
             "shuffled round-robin rounds of %d timed steps)" % (CONFIGS[args.config]["name"], len(results), args.rounds,
                                                          args.steps), "",
             "Default plan: %.2f µs, rank %d of %d; fastest: %s at %.2f µs (default / fastest = %.3f)."
             % (default["us"], rank, len(results), best["label"], best["us"], default["us"] / best["us"]),
             "Model's pick (lowest predicted step time): %s at %.2f µs measured.  Spearman rank correlation "
             "of predicted and measured time: %.3f." % (by_model["label"], by_model["us"], rho), "",
             "| plan | rule used | row split | workgroups with work / launched | model (µs per step) "
             "| µs per step | spread over rounds | max abs diff vs default |", "|---|---|---|---|---|---|---|---|"]
    for r in sorted(results, key=lambda r: r["us"]):
        lines.append("| %s | %s | %d | %d / %d | %.1f | %.2f | %.2f | %.3g |" % (
            r["label"], r["rule"], r["row_split"], r["num_wg"], r["grid_wg"], r["model"], r["us"],
            r["spread_us"], r["max_abs_vs_default"]))
    text = "\n".join(lines)
    print(text, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text + "\n")
    if args.dump:
        with open(args.dump, "w") as f:
            json.dump({"workload": CONFIGS[args.config]["name"], "config": args.config, "num_cus": num_cus,
                       "batch": B, "rows": rows, "seqlens": case.cache_seqlens.tolist(), "candidates": results}, f)


if __name__ == "__main__":
    main()
