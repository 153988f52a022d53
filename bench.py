#!/usr/bin/env python3
"""Benchmark of MLA decode on one MI355X.

Workload (default): batch 64, 128 query heads, q_len 1, every sequence 4096 cached
tokens, 576-wide bf16 latent rows (512 latent + 64 rope) in 64-token pages, block
table a seeded page permutation, scale 192^-0.5; seeded N(0, 1) synthetic inputs.

One step = the whole decode path on one batch: the split plan, the split-KV decode kernel
and the log-sum-exp combine.  The plan is computed inside the decode launch from the
step's lengths (plan_in_decode: one mla_get_metadata up front, then every decode launch
re-plans, each workgroup taking its own share); --planner-kernel plans with a planner
launch every step instead.  Inputs are resident in HBM
before timing starts.  Two KV pools with identical contents are alternated step by
step, so no step can be served from the 256 MB memory-side cache left warm by the
step before it.

Timed passes hold the stream with a short spin kernel while the host enqueues the
whole pass, so the device runs the steps back to back: the figures are device time,
with no host enqueue gaps inside them (a serving loop gets the same by enqueueing
ahead or replaying a captured graph).  Each timed pass starts with --settle-ms of
untimed whole steps, back to back with the timed ones: when the device goes from idle
to this load, its power management first runs the shader clock about 10 percent
below its sustained rate for some milliseconds, and the settle steps carry the timed
ones past that into the sustained rate a serving loop runs at.  The decode kernel's own
duration comes from a second pass of whole steps whose decode launches carry events bound
to the kernel's start and end (mla_decode_splits_timed: no timing packet between the
launches); the planner and the combine are timed in passes of their own (back to back,
after settle steps).

Prints one JSON line: throughput in TFLOP/s (algorithmic FLOPs: 2*(576+512) per
visible key per query row), KV GB/s, roofline fractions, the decode kernel's own
duration from HIP events, the device's streaming-read rate from the library's probe
(context for the roofline), and the CPU oracle's rate on the host as a reported baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CU x 4096 FLOP/clk x 2.4 GHz)
METRIC = "MLA decode TFLOP/s + KV GB/s (% roofline), 128 heads, B=64, seqlen 4096"
DECODE_KERNEL = "mla_decode_bf16_kernel"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_%s_traffic.json")   # per workload name


def workload_sizes(case, indices=None):
    """Algorithmic FLOPs and bytes of one decode of `case` (each visible key once; with
    sparse `indices`, each listed entry once, plus the lists themselves)."""
    import numpy as np
    T, H = case.q_len, case.num_heads
    elem = 2 if case.dtype == "bf16" else 4
    rows = case.batch * T * H
    if indices is not None:
        keys = int(np.sum(indices != -1))
        other = rows * 576 * elem + rows * 512 * elem + rows * 4 + indices.size * 4 + case.batch * 4
        return keys * H * 2 * (576 + 512), keys * 576 * elem, keys * 576 * elem + other
    flops = 0
    for L in case.cache_seqlens.tolist():
        for t in range(T):
            n = (L - T + 1 + t) if (case.causal and T > 1) else L
            flops += max(n, 0) * H * 2 * (576 + 512)
    kv_bytes = int(np.sum(np.maximum(case.cache_seqlens, 0))) * 576 * elem
    other = rows * 576 * elem + rows * 512 * elem + rows * 4 + case.block_table.size * 4 + case.batch * 4
    return flops, kv_bytes, kv_bytes + other


def traffic_from_profile(workload):
    """HBM bytes per decode launch from the workload's committed counter profile, if it was
    taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE % workload) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    from mla_decode_03_amd.profiling import kernel_source_hash
    if rec.get("kernel_source_sha") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def hbm_probe(torch, mla, dev, nbytes=512 << 20, reps=10):
    """The device's streaming-read rate, as context for the roofline fraction: 512 MiB (twice
    the 256 MB memory-side cache, so the passes stream from HBM) read once per pass by the
    library's probe, with plain vector loads and with the decode's global->LDS copies."""
    src = torch.zeros(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(4096, dtype=torch.int32, device=dev)
    res = {"bytes": nbytes}
    for mode, key in ((0, "vector_loads_gbs"), (1, "lds_copies_gbs")):
        for _ in range(3):
            mla.hbm_read_probe(src, mode, sink)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            mla.hbm_read_probe(src, mode, sink)
        e1.record()
        torch.cuda.synchronize()
        res[key] = round(nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del src, sink
    return res


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(case, flops, indices=None):
    import oracle
    t0 = time.perf_counter()
    oracle.decode_case(case, indices=indices)
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.max_threads(),
            "cpu_model": cpu_model(), "kind": "oracle", "seconds": round(dt, 3),
            "sample": "the whole workload once: all %d query rows x %d keys, float64 two-pass "
                      "softmax on the host" % (case.batch * case.q_len * case.num_heads,
                                               int(case.cache_seqlens.max()))}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", type=int, default=1, help="workload index 0..4 (default: the headline one)")
    ap.add_argument("--settle-ms", type=float, default=50.0,
                    help="untimed whole steps run back to back right before each timed pass, in ms "
                         "of device time (carries the timed steps past the clock dip after idle)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--num-workgroups", type=int, default=0)
    ap.add_argument("--min-blocks", type=int, default=0)
    ap.add_argument("--planner-kernel", action="store_true",
                    help="plan with a planner launch every step (mla_get_metadata), instead of inside the "
                         "decode launch (plan_in_decode, the default here)")
    ap.add_argument("--row-split", type=int, default=0)
    ap.add_argument("--fixed-split-blocks", type=int, default=0,
                    help="batch-invariant plan: fixed chunks of this many 64-token blocks")
    ap.add_argument("--sinks", action="store_true",
                    help="attention-sink variant (seeded per-head sink logits)")
    ap.add_argument("--sparse-topk", type=int, default=0,
                    help="sparse variant: every (b, t) attends to this many seeded distinct positions")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the HBM streaming-read probe (reported as context beside the roofline)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="after timing, copy BYTES device to device 3 times (the reference "
                         "dispatch that scales the HBM byte counters of a profiled run)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the decode runs on a single MI355X and this build "
              "has no multi-GPU path (asked for --gpus %d, WORLD_SIZE %d)" % (args.gpus, world),
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import mla_decode_03_amd as mla
    from mla_inputs import CONFIGS, make_config, make_sinks, make_topk_indices

    mla.lib()
    dev = torch.device("cuda:0")
    case = make_config(args.config)
    indices_np = None
    if args.sparse_topk > 0:
        if case.causal or case.dtype != "bf16":
            sys.exit("--sparse-topk needs a bf16 workload without causal masking")
        indices_np = make_topk_indices(case.cache_seqlens, case.q_len, args.sparse_topk, seed=11)
    flops, kv_bytes, total_bytes = workload_sizes(case, indices_np)

    if case.dtype == "bf16":
        q = torch.from_numpy(case.q_bits.view(np.int16)).to(dev).view(torch.bfloat16)
        kv_a = torch.from_numpy(case.kv_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        q = torch.from_numpy(case.q).to(dev)
        kv_a = torch.from_numpy(case.kv).to(dev)
    kv_b = kv_a.clone()
    bt = torch.from_numpy(case.block_table).to(dev)
    lens = torch.from_numpy(case.cache_seqlens).to(dev)
    B, T, H = case.batch, case.q_len, case.num_heads
    out = torch.empty((B, T, H, 512), dtype=q.dtype, device=dev)
    lse = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    sinks = torch.from_numpy(make_sinks(H, seed=1)).to(dev) if args.sinks else None
    indices = torch.from_numpy(indices_np).to(dev) if indices_np is not None else None
    split = case.dtype == "bf16"
    # bf16 batches of at most 4095 (units of) sequences plan inside the decode launch: the plan
    # is made once and every decode re-plans from the lengths it is given
    in_decode = split and not args.planner_kernel and case.batch * (case.q_len if args.sparse_topk > 0 else 1) <= 4095
    opts = mla.PlanOptions(num_workgroups=args.num_workgroups, min_blocks_per_wg=args.min_blocks,
                           row_split=args.row_split, fixed_split_blocks=args.fixed_split_blocks,
                           plan_in_decode=1 if in_decode else 0)
    dec = mla.Decoder(q, kv_a, bt, causal=case.causal, split=split, options=opts, topk=args.sparse_topk)
    pools = (kv_a, kv_b)
    stream = torch.cuda.current_stream()

    def step(i, dec_ev=None):
        """One whole step; dec_ev: a (start, stop) event pair bound to the decode kernel's own
        start and end (no timing packet between the step's launches)."""
        kv = pools[i & 1]
        if not split:
            mla.decode(dec.problem, q, kv, bt, lens, case.scale, out, lse, None, None, stream, sinks)
            return
        plan = dec.plan_for(lens, stream)
        mla.decode_splits(dec.problem, q, kv, bt, lens, case.scale, out, lse, plan, dec.workspace, stream,
                          sinks, indices, events=dec_ev)
        mla.combine(dec.problem, out, lse, plan, dec.workspace, stream, sinks)

    t_host = time.perf_counter()
    for i in range(args.warmup):
        step(i)
    t_host = (time.perf_counter() - t_host) / max(args.warmup, 1)   # host seconds to enqueue a step
    torch.cuda.synchronize()

    # the spin kernel's rate, to hold the stream while a whole pass is enqueued
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    torch.cuda._sleep(1 << 20)
    c1.record(stream)
    torch.cuda.synchronize()
    cycles_per_ms = (1 << 20) / max(c0.elapsed_time(c1), 1e-3)

    def hold(n_steps):
        ms = 2.0 + 3.0 * n_steps * t_host * 1e3 + 5e-3 * n_steps   # enqueue time, with margin
        torch.cuda._sleep(int(min(ms, 2000.0) * cycles_per_ms))

    # untimed steps that fill --settle-ms of device time, from one step's duration
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    hold(10)
    s0.record(stream)
    for i in range(10):
        step(i)
    s1.record(stream)
    torch.cuda.synchronize()
    settle = max(10, int(args.settle_ms / max(s0.elapsed_time(s1) / 10, 1e-3)))

    # timed region: exactly `steps` whole-path steps, back to back on the device, right
    # behind the settle steps
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    hold(settle + args.steps)
    for i in range(settle):
        step(i)
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1)
    ms_per_step = total_ms / args.steps

    # Per-kernel durations.  Events recorded between the launches of a step would change
    # them (each is a stream packet that waits for and releases the work before it, and the
    # kernel after it starts cold).  So the decode kernel is timed with events bound to its
    # own start and end (mla_decode_splits_timed), over `steps` whole steps after `settle`
    # untimed ones, and the planner and the combine in passes of their own, `steps`
    # launches back to back between two events, each after `settle` whole steps.  A
    # kernel trace of the same command agrees with the decode figure (the timed steps'
    # dispatches).

    def timed_pass(fn):
        torch.cuda.synchronize()
        hold(settle + args.steps)
        for i in range(settle):
            step(i)
        p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        p0.record(stream)
        for i in range(args.steps):
            fn(i)
        p1.record(stream)
        torch.cuda.synchronize()
        return p0.elapsed_time(p1) / args.steps

    if split:
        dev_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.steps)]
        for a_, b_ in dev_ev:             # creates the events
            a_.record(stream)
            b_.record(stream)
        torch.cuda.synchronize()
        hold(settle + args.steps)
        for i in range(settle):
            step(i)
        for i in range(args.steps):
            step(i, dev_ev[i])
        torch.cuda.synchronize()
        dec_ms = sum(a_.elapsed_time(b_) for a_, b_ in dev_ev) / args.steps
        # (planning inside the decode: plan_for launches nothing after the first call)
        plan_ms = timed_pass(lambda i: dec.plan_for(lens, stream)) if not in_decode else 0.0
        plan = dec.plan_for(lens, stream)
        comb_ms = timed_pass(lambda i: mla.combine(dec.problem, out, lse, plan, dec.workspace, stream, sinks))
        kernel_ms = dec_ms
        launches = {"method": "decode: events bound to the kernel's own start and end, over whole steps; plan "
                              "and combine: passes of their own",
                    "plan_in_decode": bool(in_decode),
                    "first_timed_step": args.warmup + 10 + settle,
                    "decode_us": round(kernel_ms * 1e3, 2), "plan_us": round(plan_ms * 1e3, 2),
                    "step_minus_plan_combine_us": round((ms_per_step - plan_ms - comb_ms) * 1e3, 2),
                    "combine_us": round(comb_ms * 1e3, 2), "step_us": round(ms_per_step * 1e3, 2)}
    else:
        kernel_ms = ms_per_step
        launches = {"method": "decode = step (one launch per step)", "first_timed_step": args.warmup + 10 + settle,
                    "decode_us": round(kernel_ms * 1e3, 2)}

    t = ms_per_step * 1e-3
    tflops = flops / t / 1e12
    kv_gbs = kv_bytes / t / 1e9
    frac_hbm = (total_bytes / t / 1e9) / HBM_PEAK_GBS
    frac_mfma = tflops / MFMA_BF16_PEAK_TFLOPS

    roofline = None
    # The committed counter profiles were taken on the plain decode with the default plan;
    # any other launch (a variant or a plan override) has no traffic figure.
    profiled = not (args.sinks or args.sparse_topk or args.num_workgroups or args.min_blocks or args.row_split
                    or args.fixed_split_blocks or args.planner_kernel)
    if kernel_ms is not None:
        achieved = total_bytes / (kernel_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_from_profile(CONFIGS[args.config]["name"]) if profiled else None,
                    "kernel": DECODE_KERNEL if split else "mla_decode_f32_kernel", "kernel_ms": round(kernel_ms, 5),
                    "algorithmic_bytes_per_launch": total_bytes}

    probe = None
    if not args.no_probe:
        probe = hbm_probe(torch, mla, dev)
        if roofline is not None:
            probe["decode_frac_of_lds_copies"] = round(roofline["achieved"] / probe["lds_copies_gbs"], 4)

    if args.calibrate_copy > 0:
        src = torch.empty(args.calibrate_copy, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(case, flops, indices_np)

    rec = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settle,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dtype,
        "data": "synthetic",
        "config": {"workload": CONFIGS[args.config]["name"], "batch": B, "heads": H, "q_len": T,
                   "seqlen": int(case.cache_seqlens.max()), "page": 64, "d_qk": 576, "d_v": 512,
                   "causal": case.causal, "kv_pools_alternated": 2,
                   "variant": "+".join(v for v, on in (("attention_sink", args.sinks),
                                                       ("sparse_top%d" % args.sparse_topk, args.sparse_topk > 0))
                                       if on) or "plain",
                   "plan": {"num_workgroups": dec.plan.grid_wg if dec.plan else None,
                            "fixed_split_blocks": args.fixed_split_blocks or None,
                            "in_decode": bool(in_decode)}},
        "kv_gb_per_s": round(kv_gbs, 1),
        "frac_hbm_total_bytes": round(frac_hbm, 4),
        "frac_mfma_bf16": round(frac_mfma, 4),
        "frac_roofline": round(max(frac_hbm, frac_mfma), 4),
        "algorithmic": {"flop": flops, "kv_bytes": kv_bytes, "total_bytes": total_bytes},
        "roofline": roofline,
        "launches": launches,
        "hbm_probe": probe,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
