"""Summaries of rocprofv3 output for the decode kernels (the files under profiles/).

    python -m mla_decode_03_amd.profiling traffic FETCH_CSV WRITE_CSV --copy-bytes N [--out FILE]
        HBM bytes per decode launch from a FETCH_SIZE pass and a WRITE_SIZE pass
        (rocprofv3 --pmc ... --output-format csv, *_counter_collection.csv) over a
        `bench.py --calibrate-copy N` run.  Each counter is scaled by what it reads for
        the plain device copy of N bytes the same run makes, so the figure does not
        depend on the counter's unit.  Writes JSON with the decode kernel's source hash
        (bench.py reports the figure only while that hash matches).
    python -m mla_decode_03_amd.profiling stats KERNEL_STATS_CSV
        Markdown table of a --kernel-trace --stats run (calls, average/min/max us).
    python -m mla_decode_03_amd.profiling trace KERNEL_TRACE_CSV --steps K --skip N
        Per-kernel durations of a traced `bench.py --steps K` run whose line gives
        first_timed_step N (the whole steps enqueued before the timed ones): over every
        dispatch, and over the dispatches of the K timed steps (what bench.py's step time
        and its decode figure, step minus planner minus combine, cover).
    python -m mla_decode_03_amd.profiling counters CSV [CSV ...]
        Median per dispatch of every counter in SQ/TCC passes, per kernel.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DECODE_KERNEL = "mla_decode_bf16_kernel"
COPY_KERNEL = "__amd_rocclr_copyBuffer"
KERNEL_SOURCES = ["mla_decode_03_amd/csrc/mla_decode_bf16.hip", "mla_decode_03_amd/csrc/mla_device.h",
                  "mla_decode_03_amd/csrc/mla_args.h"]


def kernel_source_hash() -> str:
    """Hash of the decode kernel's sources: a traffic figure is valid for this hash only."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _per_dispatch(path):
    """{(kernel name, counter): {dispatch id: summed value}} of a counter-collection CSV."""
    out = collections.defaultdict(lambda: collections.defaultdict(float))
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            name = row.get("Kernel_Name", "")
            out[(name, row["Counter_Name"])][int(row["Dispatch_Id"])] += float(row["Counter_Value"])
    return out


def _median_for(table, kernel_substr, counter, pick=None):
    vals = []
    for (name, ctr), by in table.items():
        if ctr == counter and kernel_substr in name:
            vals.extend(by.values())
    if pick is not None:
        vals = [v for v in vals if pick(v)]
    if not vals:
        raise SystemExit("no %s dispatches with %s in the profile" % (kernel_substr, counter))
    return statistics.median(vals), len(vals)


def traffic(fetch_csv, write_csv, copy_bytes, out=None):
    res = {"kernel": DECODE_KERNEL, "kernel_source_sha": kernel_source_hash(), "copy_bytes": copy_bytes}
    total = 0.0
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        tab = _per_dispatch(path)
        # the calibration copy is the copy dispatch that moves the most data
        copies = [v for (name, ctr), by in tab.items() if ctr == counter and COPY_KERNEL in name
                  for v in by.values()]
        if not copies:
            raise SystemExit("no %s dispatch in %s" % (COPY_KERNEL, path))
        big = max(copies)
        cal, ncal = _median_for(tab, COPY_KERNEL, counter, pick=lambda v: v > 0.5 * big)
        dec, ndec = _median_for(tab, DECODE_KERNEL, counter)
        factor = copy_bytes / cal
        key = "fetch" if counter == "FETCH_SIZE" else "write"
        res[key] = {"counter_per_launch": dec, "launches": ndec, "copy_counter": cal, "copy_launches": ncal,
                    "bytes_per_count": factor, "bytes_per_launch": round(dec * factor)}
        total += dec * factor
    res["hbm_bytes_per_launch"] = round(total)
    text = json.dumps(res, indent=1)
    if out:
        with open(out, "w") as f:
            f.write(text + "\n")
    print(text)


def stats(path):
    with open(path, newline="") as f:
        rows = list(csv.DictReader(f))
    print("| kernel | calls | avg us | min us | max us |")
    print("|---|---|---|---|---|")
    for r in rows:
        name = r["Name"]
        short = name.split("(")[0].replace("void ", "").replace("mla::", "")
        print("| %s | %s | %.2f | %.2f | %.2f |" % (short, r["Calls"], float(r["AverageNs"]) / 1e3,
                                                   float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))


def trace(path, steps, skip, decode=DECODE_KERNEL):
    """Markdown table of per-kernel durations from a kernel-trace CSV of a `bench.py
    --steps K` run: over every dispatch, and over the dispatches of the K timed steps (the
    decode launches skip+1 .. skip+K and, in launch order, the dispatch just before and
    just after each: that step's planner and combine).  `skip` is the number of whole
    steps the run enqueued before its timed ones (`first_timed_step` in bench.py's line).
    Returns {kernel: {"all": us, "timed": us}}."""
    allds = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            allds.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]))
    allds.sort()
    dec_pos = [i for i, d in enumerate(allds) if decode in d[2]]
    timed = set()
    if len(dec_pos) >= skip + steps:
        for p in dec_pos[skip:skip + steps]:
            timed.update(q for q in (p - 1, p, p + 1) if 0 <= q < len(allds))
    per = collections.defaultdict(lambda: ([], []))
    for i, (b, e, name) in enumerate(allds):
        per[name][0].append((e - b) / 1e3)
        if i in timed:
            per[name][1].append((e - b) / 1e3)
    print("| kernel | calls | avg us | timed steps: calls | timed steps: avg us |")
    print("|---|---|---|---|---|")
    res = {}
    for name, (us, tus) in sorted(per.items(), key=lambda kv: -len(kv[1][0])):
        short = name.split("(")[0].replace("void ", "").replace("mla::", "")
        res[short] = {"all": sum(us) / len(us)}
        if tus:
            res[short]["timed"] = sum(tus) / len(tus)
        print("| %s | %d | %.2f | %d | %s |" % (short, len(us), sum(us) / len(us), len(tus),
                                                "%.2f" % (sum(tus) / len(tus)) if tus else "-"))
    return res


def counters(paths):
    for path in paths:
        tab = _per_dispatch(path)
        kernels = sorted({name for name, _ in tab})
        for k in kernels:
            short = k.split("(")[0].replace("void ", "").replace("mla::", "")
            for (name, ctr), by in sorted(tab.items()):
                if name == k:
                    vals = sorted(by.values())
                    print("%-40s %-28s dispatches %3d  median %.6g" % (short[:40], ctr, len(vals),
                                                                      vals[len(vals) // 2]))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_csv")
    t.add_argument("write_csv")
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--out")
    s = sub.add_parser("stats")
    s.add_argument("csv")
    tr = sub.add_parser("trace")
    tr.add_argument("csv")
    tr.add_argument("--steps", type=int, required=True)
    tr.add_argument("--skip", type=int, required=True, help="whole steps before the timed ones")
    c = sub.add_parser("counters")
    c.add_argument("csv", nargs="+")
    a = ap.parse_args(argv)
    if a.cmd == "traffic":
        traffic(a.fetch_csv, a.write_csv, a.copy_bytes, a.out)
    elif a.cmd == "stats":
        stats(a.csv)
    elif a.cmd == "trace":
        trace(a.csv, a.steps, a.skip)
    else:
        counters(a.csv)


if __name__ == "__main__":
    sys.exit(main())
