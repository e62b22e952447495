"""Benchmark: MLA decode over a paged latent cache on one MI355X.

A step is one libmla.mla_decode call (split plan, split-KV decode kernel and,
where sequences are split, the LSE combine kernel) over the whole batch of
the DeepSeek-V3-shaped decode workload: 64 sequences x 128 heads x 4096
cached tokens, 576-wide bf16 latent rows in 64-token blocks, one query token
per sequence. Inputs are synthetic (seeded N(0,1), see workload/) and resident
in HBM before timing; the cache is rotated over enough copies that no step
can be served from the 256 MB MALL left behind by the previous one.

Each step is one library call from Python; --graph replays the steps from
HIP graphs (several consecutive steps per graph) instead.

Prints one JSON line (rank 0): throughput in algorithmic GB/s (every visible
cached token read once per sequence, plus q, out, lse, block table, seqlens),
TFLOP/s, the roofline of the step measured with HIP events on the launch
stream, and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
METRIC = "MLA decode latent-KV GB/s + TFLOP/s and % of MI355X roofline (128 heads, 4K ctx)"
WORKLOAD_CFG = 2                 # 64 x 128 heads x 4096 tokens, bf16 cache


def source_hash() -> str:
    h = hashlib.sha256()
    for rel in ("mla_latent_kv_10_amd/csrc/libmla.hip", "include/mla.h"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=WORKLOAD_CFG, help="workload index 1..5")
    ap.add_argument("--num-parts", type=int, default=0)
    ap.add_argument("--m-tile", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="replay the steps from HIP graphs instead of launching each from Python")
    ap.add_argument("--cpu-seqs", type=int, default=64, help="sequences in the oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (HBM counter calibration)")
    return ap.parse_args()


def copy_calibration():
    import torch
    n = 1 << 30
    x = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "launches": 3}))


def cpu_baseline(w, n_seqs: int):
    """Oracle on the first n_seqs sequences (all their heads), host threads."""
    import oracle
    import workload as wl
    n_seqs = max(1, min(n_seqs, w.B))
    rows = np.arange(n_seqs * w.s_q * w.H, dtype=np.int64)
    t0 = time.perf_counter()
    oracle.decode_absorbed(w.q, w.kv, w.block_table, w.seqlens, w.softmax_scale,
                           kv_scales=w.kv_scales, rows=rows)
    dt = time.perf_counter() - t0
    sub = wl.Workload(**{**w.__dict__, "B": n_seqs, "q": w.q[:n_seqs],
                         "seqlens": w.seqlens[:n_seqs], "block_table": w.block_table[:n_seqs]})
    nbytes, flops, _ = wl.config_flops_bytes(sub)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"first {n_seqs} of {w.B} sequences (all {w.H} heads, {int(w.seqlens[0])} "
                      f"tokens each), fp64 two-pass oracle, same seeded inputs"}


def roofline(nbytes: int, flops: int, avg_ms: float, traffic) -> dict:
    """The binding roofline of one step: HBM (algorithmic bytes at 8 TB/s) or
    MFMA (algorithmic flops at the dense bf16 peak), whichever takes longer at
    its peak; the other one's fraction is reported beside it."""
    gbs = nbytes / (avg_ms * 1e-3) / 1e9
    tfs = flops / (avg_ms * 1e-3) / 1e12
    hbm = {"achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": round(gbs / HBM_PEAK_GBS, 4)}
    mfma = {"achieved": round(tfs, 2), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tfs / BF16_MFMA_PEAK_TFLOPS, 4)}
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (BF16_MFMA_PEAK_TFLOPS * 1e12)
    bound, main_, other, other_name = (("hbm", hbm, mfma, "mfma") if t_hbm >= t_mfma
                                       else ("mfma", mfma, hbm, "hbm"))
    return {"bound": bound, **main_, "traffic": traffic,
            "kernel": "one mla_decode step (decode kernel + LSE combine), HIP events "
                      "on the launch stream",
            f"{other_name}_achieved": other["achieved"], f"{other_name}_frac": other["frac"]}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU path is a design, not a build)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    import torch
    import mla_latent_kv_10_amd as mla
    import workload as wl

    mla.lib()   # raises if libmla.so is missing: there is no other path
    w = wl.config_workload(args.config)
    nbytes, flops, _ = wl.config_flops_bytes(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q = torch.from_numpy(w.q.view(np.int16)).view(torch.bfloat16).to(dev)
    bt = torch.from_numpy(w.block_table).to(dev)
    sl = torch.from_numpy(w.seqlens).to(dev)
    if w.kv_dtype == "bf16":
        kv0 = torch.from_numpy(w.kv.view(np.int16)).view(torch.bfloat16).to(dev)
        sc0 = None
    else:
        kv0 = torch.from_numpy(w.kv).to(dev)
        sc0 = torch.from_numpy(w.kv_scales.view(np.int16)).view(torch.float16).to(dev)
    cache_bytes = kv0.numel() * kv0.element_size() + (0 if sc0 is None else sc0.numel() * 2)
    copies = max(1, int(np.ceil(3 * 256e6 / cache_bytes)) + 1)
    kvs = [kv0] + [kv0.clone() for _ in range(copies - 1)]
    scs = [sc0] + [None if sc0 is None else sc0.clone() for _ in range(copies - 1)]
    out = torch.empty((w.B, w.s_q, w.H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.s_q, w.H), dtype=torch.float32, device=dev)
    prob = mla.make_problem(q, kv0, bt, kv_dtype=mla.KV_Q8_0 if sc0 is not None else mla.KV_BF16,
                            max_seqlen=w.max_seqlen, num_parts=args.num_parts,
                            m_tile=args.m_tile)
    ws = torch.empty(max(16, mla.workspace_size(prob)), dtype=torch.uint8, device=dev)
    parts = mla.problem_num_parts(prob)

    def step(i):
        mla.mla_decode(q, kvs[i % copies], bt, sl, w.softmax_scale, out, lse,
                       kv_scales=scs[i % copies], max_seqlen=w.max_seqlen,
                       num_parts=args.num_parts, m_tile=args.m_tile, workspace=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    if not args.graph:
        # eager: one library call per step from Python
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        runs = [1] * args.steps
        t0 = time.perf_counter()
        for i in range(args.steps):
            ev[i][0].record(stream)
            step(i)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    else:
        # HIP graphs: G consecutive steps (rotating over the cache copies) are
        # captured once and replayed, the way a serving loop issues decode
        # steps; a second graph holds the K mod G remaining steps, so exactly
        # K steps run in the timed region. The library makes no allocation,
        # memset or synchronisation inside a step, so a step captures as its
        # kernel launches alone.
        G = min(args.steps, 2 * copies)
        graphs = []
        for n_in in (G, args.steps % G):
            if n_in == 0:
                continue
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(n_in):
                    step(i)
            graphs.append((g, n_in))
        for g, _ in graphs:          # untimed first replays
            g.replay()
        torch.cuda.synchronize()
        plan = [graphs[0]] * (args.steps // G) + ([graphs[1]] if len(graphs) > 1 else [])
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in plan]
        runs = [n_in for _, n_in in plan]
        t0 = time.perf_counter()
        for (g, _), (e0, e1) in zip(plan, ev):
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    per_launch_ms = [a.elapsed_time(b) / n for (a, b), n in zip(ev, runs)]
    avg_ms = float(np.mean(per_launch_ms))
    ms_per_step = wall / args.steps * 1e3
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (avg_ms * 1e-3) / 1e9

    traffic = None
    tfile = os.path.join(ROOT, "profiles", f"hbm_traffic_{w.name}.json")
    if os.path.exists(tfile):
        rec = json.load(open(tfile))
        if rec.get("source_hash") == source_hash() and rec.get("num_parts") == parts:
            traffic = rec.get("bytes_per_launch")

    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "heads": w.H, "seqlen": int(w.seqlens[0]),
                   "seqlen_q": w.s_q, "kv_cache": f"{w.kv_dtype}, paged 64-token blocks, "
                   "576 = 512 latent + 64 rope", "d_latent": 512, "d_rope": 64,
                   "num_parts": parts, "m_tile": args.m_tile or "auto",
                   "cache_copies_rotated": copies,
                   "launch": "hip_graph" if args.graph else "eager"},
        "tflops": round(flops / (avg_ms * 1e-3) / 1e12, 2),
        "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
        "event_ms": {"mean": round(avg_ms, 5), "p10": round(float(np.percentile(per_launch_ms, 10)), 5),
                     "p90": round(float(np.percentile(per_launch_ms, 90)), 5)},
        "roofline": roofline(nbytes, flops, avg_ms, traffic),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seqs)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
