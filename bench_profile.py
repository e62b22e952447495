"""Turn rocprofv3 output of bench.py runs into the summaries kept under profiles/.

  python bench_profile.py trace  <kernel-trace dir> <out.md> "<command that made it>"
  python bench_profile.py traffic <fetch dir> <write dir> <copy-fetch dir> <copy-write dir> \
                          <out.json> "<commands>"
  python bench_profile.py mfma <pmc dir> <probe pmc dir> <out.json> "<commands>" [extra json]

trace: per-kernel calls / average / total duration from a
  `rocprofv3 --kernel-trace --stats --output-format csv` run.
traffic: HBM bytes per decode step from two `--pmc FETCH_SIZE` / `--pmc WRITE_SIZE`
  runs (KiB per dispatch), each scaled by the factor the same counter shows for
  a plain 1 GiB device copy (`bench.py --copy-calibration`): factor = copied
  bytes / (counter KiB * 1024). One step = every library kernel launched by one
  mla_decode call. The JSON carries the source hash bench.py checks, so a
  stale measurement is never reported for a changed kernel.
"""
from __future__ import annotations

import csv
import glob
import json
import os
import sys
from collections import defaultdict

import bench

LIB_KERNELS = ("mla_decode", "mla_split_combine", "mla_combine")
COPY_BYTES = 1 << 30


def _find(d: str, suffix: str) -> str:
    hits = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return hits[0]


def _short(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "")
    return name.split("(")[0].replace("void ", "")


def trace(kt_dir: str, out_md: str, command: str) -> None:
    rows = list(csv.DictReader(open(_find(kt_dir, "kernel_stats.csv"))))
    lines = [f"# Kernel trace: {os.path.basename(out_md)[:-3]}", "", "Command:", "",
             "```", command, "```", "",
             "| kernel | calls | average (us) | total (us) | share |",
             "|---|---|---|---|---|"]
    for r in rows:
        avg_ns = float(r["AverageNs"])
        tot_ns = float(r["TotalDurationNs"])
        lines.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {avg_ns / 1e3:.2f} | "
                     f"{tot_ns / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    open(out_md, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _per_kernel(d: str, counter: str):
    vals = defaultdict(list)
    for r in csv.DictReader(open(_find(d, "counter_collection.csv"))):
        if r["Counter_Name"] == counter:
            vals[_short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return vals


def _copy_factor(d: str, counter: str) -> float:
    v = _per_kernel(d, counter)
    copies = [x for k, xs in v.items() if "copyBuffer" in k for x in xs]
    if not copies:
        raise RuntimeError(f"no copy kernel in {d}")
    kib = sorted(copies)[len(copies) // 2]
    return COPY_BYTES / (kib * 1024.0)


def traffic(fetch_dir, write_dir, cfetch_dir, cwrite_dir, out_json, command) -> None:
    ff = _copy_factor(cfetch_dir, "FETCH_SIZE")
    wf = _copy_factor(cwrite_dir, "WRITE_SIZE")
    fetch = _per_kernel(fetch_dir, "FETCH_SIZE")
    write = _per_kernel(write_dir, "WRITE_SIZE")
    per = {}
    for k in sorted(set(fetch) | set(write)):
        if not any(t in k for t in LIB_KERNELS):
            continue
        f = fetch.get(k, [0.0])
        w = write.get(k, [0.0])
        per[k] = {"fetch_bytes": sum(f) / len(f) * 1024 * ff,
                  "write_bytes": sum(w) / len(w) * 1024 * wf, "launches_seen": len(f)}
    total = sum(v["fetch_bytes"] + v["write_bytes"] for v in per.values())
    rec = {"source_hash": bench.source_hash(), "command": command,
           "fetch_factor": round(ff, 4), "write_factor": round(wf, 4),
           "per_kernel": per, "bytes_per_launch": int(total)}
    if len(sys.argv) > 8:
        rec.update(json.loads(sys.argv[8]))
    json.dump(rec, open(out_json, "w"), indent=1)
    print(json.dumps(rec, indent=1))


def _counters(d: str):
    """-> {kernel: {counter: [(value, duration ns) per dispatch]}}"""
    vals = defaultdict(lambda: defaultdict(list))
    for r in csv.DictReader(open(_find(d, "counter_collection.csv"))):
        dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        vals[_short(r["Kernel_Name"])][r["Counter_Name"]].append((float(r["Counter_Value"]), dur))
    return vals


def _median(xs):
    xs = sorted(xs)
    return xs[len(xs) // 2]


def mfma(pmc_dir, probe_dir, out_json, command, extra=None) -> None:
    """Per kernel, medians over its dispatches:
      mfma_busy_frac  (SQ_VALU_MFMA_BUSY_CYCLES / GRBM_GUI_ACTIVE) of the kernel
                      divided by the same ratio of the probe, which keeps every
                      matrix core busy: the share of the kernel's time the matrix
                      cores are busy, at the kernel's own clock;
      executed_bf16_flops  SQ_INSTS_VALU_MFMA_MOPS_BF16 * 512 (padding and
                      idle-step MFMAs included);
      executed_tflops  those flops over the dispatch's duration under the
                      profiler, next to the probe's sustained rate."""
    probe = _counters(probe_dir)
    pk = [k for k in probe if "mfma_probe" in k]
    if not pk:
        raise RuntimeError(f"no probe kernel in {probe_dir}")
    pc = probe[pk[0]]
    # the probe's long dispatch (the short first one only warms it up)
    i = max(range(len(pc["GRBM_GUI_ACTIVE"])), key=lambda j: pc["GRBM_GUI_ACTIVE"][j][0])
    probe_ratio = pc["SQ_VALU_MFMA_BUSY_CYCLES"][i][0] / pc["GRBM_GUI_ACTIVE"][i][0]
    probe_tflops = pc["SQ_INSTS_VALU_MFMA_MOPS_BF16"][i][0] * 512 / (pc["GRBM_GUI_ACTIVE"][i][1] * 1e-9) / 1e12
    per = {}
    for k, c in _counters(pmc_dir).items():
        if not any(t in k for t in LIB_KERNELS) or not c.get("GRBM_GUI_ACTIVE"):
            continue
        n = len(c["GRBM_GUI_ACTIVE"])
        ratios = [b[0] / g[0] for b, g in zip(c["SQ_VALU_MFMA_BUSY_CYCLES"], c["GRBM_GUI_ACTIVE"]) if g[0] > 0]
        rec = {"dispatches": n, "mfma_busy_frac": round(_median(ratios) / probe_ratio, 4)}
        if c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16"):
            fl = [m[0] * 512 for m in c["SQ_INSTS_VALU_MFMA_MOPS_BF16"]]
            rates = [m[0] * 512 / (m[1] * 1e-9) / 1e12 for m in c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] if m[1] > 0]
            rec["executed_bf16_flops"] = _median(fl)
            rec["executed_tflops"] = round(_median(rates), 1)
            rec["executed_frac_of_probe"] = round(_median(rates) / probe_tflops, 4)
        rec["median_duration_us"] = round(_median([g[1] for g in c["GRBM_GUI_ACTIVE"]]) / 1e3, 2)
        per[k] = rec
    out = {"source_hash": bench.source_hash(), "command": command,
           "probe_busy_ratio": round(probe_ratio, 3), "probe_tflops": round(probe_tflops, 1),
           "per_kernel": per}
    if extra:
        out.update(json.loads(extra))
    json.dump(out, open(out_json, "w"), indent=1)
    print(json.dumps(out, indent=1))


if __name__ == "__main__":
    if sys.argv[1] == "trace":
        trace(sys.argv[2], sys.argv[3], sys.argv[4])
    elif sys.argv[1] == "traffic":
        traffic(*sys.argv[2:8])
    elif sys.argv[1] == "mfma":
        mfma(*sys.argv[2:7])
    else:
        raise SystemExit(__doc__)
