"""Benchmark: MLA decode over a paged latent cache on one MI355X.

A step is one libmla.mla_decode call (split plan, split-KV decode kernel and,
where sequences are split, the LSE combine kernel) over the whole batch of
the DeepSeek-V3-shaped decode workload: 64 sequences x 128 heads x 4096
cached tokens, 576-wide bf16 latent rows in 64-token blocks, one query token
per sequence. Inputs are synthetic (seeded N(0,1), see workload/) and resident
in HBM before timing; the cache is rotated over enough copies that no step
can be served from the 256 MB MALL left behind by the previous one.

Each step is one library call from Python; --graph replays the steps from
HIP graphs (several consecutive steps per graph) instead. Before the W
warmup steps the step is repeated, untimed, for --settle-ms (default 100 ms)
so that the timed steps run at the GPU's sustained clocks rather than while
they ramp up from idle; the JSON line reports how many steps that took.

Prints one JSON line (rank 0): throughput in algorithmic GB/s (every visible
cached token read once per sequence, plus q, out, lse, block table, seqlens),
TFLOP/s, the roofline of the step measured with one HIP event pair on the
launch stream around the timed steps, and the CPU oracle timed on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import re
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
    """Hash of the decode kernels' code (libmla.hip and mla.h) with comments
    and blank space left out, so that a profile stays matched to the code
    it measured across edits of comments only."""
    h = hashlib.sha256()
    for rel in ("mla_latent_kv_10_amd/csrc/libmla.hip", "include/mla.h"):
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)   # block comments
        text = re.sub(r"//[^\n]*", " ", text)                 # line comments
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=WORKLOAD_CFG,
                    help="workload index 1..5 (6: the bench shape over an fp8 cache; 7: the "
                         "q8_0 workload's shape over a q4_0 cache in Hadamard rotation)")
    ap.add_argument("--num-parts", type=int, default=0)
    ap.add_argument("--m-tile", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="untimed repetitions of the step for this long before the warmup "
                         "steps, so that the timed steps run at the GPU's sustained clocks "
                         "(0: none)")
    ap.add_argument("--graph", action="store_true",
                    help="replay the steps from HIP graphs instead of launching each from Python")
    ap.add_argument("--cpu-seqs", type=int, default=0,
                    help="sequences in the oracle sample (0: 64, or 2 for the q4_0 cache, "
                         "whose rows the oracle rotates back from the matrix entries)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (HBM counter calibration and "
                         "measured copy bandwidth)")
    ap.add_argument("--layer-steps", action="store_true",
                    help="time the steps either side of the decode instead (query absorption, "
                         "output projection, cache append) at the bench shape")
    ap.add_argument("--lds-probe", action="store_true",
                    help="the LDS read rate per CU with 1, 2, 4 and 8 waves (probe library)")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="run only the MFMA probe kernel (sustained dense bf16 MFMA rate; "
                         "the MFMA-busy counter calibration)")
    return ap.parse_args()


def copy_calibration():
    """A plain 1 GiB device-to-device copy, three times: the reference the HBM
    counters are scaled by, and the copy bandwidth the chip sustains."""
    import torch
    n = 1 << 30
    x = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    y.copy_(x)
    e0.record()
    for _ in range(2):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 2
    print(json.dumps({"copy_bytes": n, "launches": 3, "copy_ms": round(ms, 4),
                      "read_plus_write_gbs": round(2 * n / (ms * 1e-3) / 1e9, 1)}))


def layer_steps(steps: int):
    """The steps either side of the decode at the bench workload's shape (64
    query rows x 128 heads): query absorption, output projection and the
    cache append (bf16, q8_0, fp8, rotated q4_0), each replayed `steps` times from a HIP
    graph so that host launch cost stays out; HIP events on the launch stream.
    Algorithmic bytes: every weight once plus the activations in and out."""
    import torch
    import mla_latent_kv_10_amd as mla
    import workload as wl
    mla.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = torch.Generator(device=dev).manual_seed(7)
    rows, H = 64, 128

    def rnd(*shape):
        return torch.randn(*shape, device=dev, generator=g).to(torch.bfloat16)

    qn, qr = rnd(rows, 1, H, 128), rnd(rows, 1, H, 64)
    wk, wv = rnd(H, 512, 128) * 0.05, rnd(H, 128, 512) * 0.05
    qa = torch.empty(rows, 1, H, 576, dtype=torch.bfloat16, device=dev)
    ol = rnd(rows, 1, H, 512)
    o = torch.empty(rows, 1, H, 128, dtype=torch.bfloat16, device=dev)
    w = wl.config_workload(WORKLOAD_CFG)
    bt = torch.from_numpy(w.block_table).to(dev)
    sl = torch.from_numpy(w.seqlens).to(dev)
    new = rnd(w.B, 1, 576)
    caches = {"bf16": (torch.empty(w.kv.shape, dtype=torch.bfloat16, device=dev), None),
              "q8_0": (torch.empty(w.kv.shape, dtype=torch.int8, device=dev),
                       torch.empty(w.kv.shape[:2] + (18,), dtype=torch.float16, device=dev)),
              "fp8": (torch.empty(w.kv.shape, dtype=torch.uint8, device=dev),
                      torch.empty(w.kv.shape[:2], dtype=torch.float32, device=dev)),
              "q4_0h": (torch.empty(w.kv.shape[:2] + (288,), dtype=torch.uint8, device=dev),
                        torch.empty(w.kv.shape[:2] + (18,), dtype=torch.float16, device=dev))}
    wbytes = H * 128 * 512 * 2
    cases = [("absorb_query", lambda: mla.mla_absorb_query(qn, qr, wk, qa),
              wbytes + qn.numel() * 2 + qr.numel() * 2 + qa.numel() * 2),
             ("project_output", lambda: mla.mla_project_output(ol, wv, o),
              wbytes + ol.numel() * 2 + o.numel() * 2)]
    per_row = {"bf16": 1152, "q8_0": 612, "fp8": 580, "q4_0h": 324}
    for kvd, (kv, sc) in caches.items():
        cases.append((f"cache_append_{kvd}",
                      lambda kv=kv, sc=sc: mla.mla_cache_append(new, bt, sl, kv, sc),
                      new.numel() * 2 + w.B * per_row[kvd]))
    out = {}
    stream = torch.cuda.current_stream(dev)
    for name, fn, nbytes in cases:
        fn()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(steps):
                fn()
        # untimed replays for about 50 ms first, so that the timed replay
        # runs at the GPU's sustained clocks
        t_settle = time.perf_counter()
        while time.perf_counter() - t_settle < 0.05:
            graph.replay()
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / steps * 1e3
        out[name] = {"us": round(us, 2), "algorithmic_bytes": nbytes,
                     "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
                     "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    print(json.dumps({"layer_steps": out, "rows": rows, "heads": H, "launches_per_graph": steps}))


def mfma_probe():
    """Independent bf16 MFMAs on every SIMD (mla_latent_kv_10_amd/csrc/mla_probe.hip):
    the dense bf16 MFMA rate the chip sustains, next to the 2.5 PFLOP/s peak."""
    import ctypes
    import torch
    from mla_latent_kv_10_amd._build import PROBE_PATH
    lib = ctypes.CDLL(PROBE_PATH)
    lib.mla_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.mla_probe_mfma.restype = ctypes.c_int
    wgs = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 20000
    out = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.mla_probe_mfma(ctypes.c_void_p(out.data_ptr()), wgs, 200, stream) == 0
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    assert lib.mla_probe_mfma(ctypes.c_void_p(out.data_ptr()), wgs, iters, stream) == 0
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    flops = wgs * 4 * iters * 8 * 32768
    tfs = flops / (ms * 1e-3) / 1e12
    # each SIMD retires one 32x32x16 MFMA per 32 cycles at full rate
    clock_ghz = wgs * 4 * iters * 8 * 32 / (ms * 1e-3) / wgs / 4 / 1e9
    print(json.dumps({"probe": "mfma_bf16_32x32x16", "workgroups": wgs, "iters": iters,
                      "ms": round(ms, 4), "tflops": round(tfs, 1),
                      "frac_of_peak": round(tfs / BF16_MFMA_PEAK_TFLOPS, 4),
                      "implied_clock_ghz": round(clock_ghz, 3)}))


def lds_probe():
    """ds_read_b128 from conflict-free addresses by 1, 2, 4 and 8 waves per CU
    (mla_latent_kv_10_amd/csrc/mla_probe.hip): the rate at which one wave,
    and a CU, receive LDS data, in bytes per shader cycle."""
    import ctypes
    import torch
    from mla_latent_kv_10_amd._build import PROBE_PATH
    lib = ctypes.CDLL(PROBE_PATH)
    lib.mla_probe_lds.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_void_p]
    lib.mla_probe_lds.restype = ctypes.c_int
    wgs = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 2000
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    res = {}
    for waves in (1, 2, 4, 8):
        out = torch.zeros(wgs * waves * 4, dtype=torch.int32, device="cuda")
        for _ in range(2):   # the second launch is the one read
            assert lib.mla_probe_lds(ctypes.c_void_p(out.data_ptr()), wgs, waves, iters, stream) == 0
        torch.cuda.synchronize()
        cyc = out.view(-1, 4)[:, 0].to(torch.int64).cpu().numpy().astype(np.float64)
        per_wave = 8 * 1024 * iters / cyc
        res[str(waves)] = {"bytes_per_cycle_per_wave": round(float(per_wave.mean()), 2),
                           "bytes_per_cycle_per_cu": round(float(per_wave.mean()) * waves, 1)}
    print(json.dumps({"probe": "lds_read_b128", "workgroups": wgs, "iters": iters,
                      "waves_per_cu": res}))


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_gbs(w, n_seqs: int, rows_per_seq=None):
    """Time the oracle on the first n_seqs sequences (all their query rows, or
    the first rows_per_seq of each) -> (GB/s, seconds, algorithmic bytes)."""
    import oracle
    import workload as wl
    n_seqs = max(1, min(n_seqs, w.B))
    per = w.s_q * w.H
    take = per if rows_per_seq is None else min(per, rows_per_seq)
    rows = np.concatenate([np.arange(b * per, b * per + take, dtype=np.int64)
                           for b in range(n_seqs)])
    t0 = time.perf_counter()
    oracle.decode_absorbed(w.q, w.kv, w.block_table, w.seqlens, w.softmax_scale,
                           kv_scales=w.kv_scales, rows=rows)
    dt = time.perf_counter() - t0
    sub = wl.Workload(**{**w.__dict__, "B": n_seqs, "q": w.q[:n_seqs],
                         "seqlens": w.seqlens[:n_seqs], "block_table": w.block_table[:n_seqs]})
    nbytes, _, _ = wl.config_flops_bytes(sub)
    if take < per:   # the cache of a sequence counts once; per-row q/out/lse for the rows run
        nbytes -= n_seqs * (per - take) * (576 * 2 + 512 * 2 + 4)
    return nbytes / dt / 1e9, dt, nbytes


def cpu_baseline(w, n_seqs: int):
    """The fp64 oracle, untuned, on the host: a bounded sample of the same
    workload on all host threads, plus single-thread figures (the tiny
    workload whole, and one sequence's first 16 rows of this workload)."""
    import oracle
    import workload as wl
    threads = oracle.max_threads()
    gbs, dt, _ = _oracle_gbs(w, n_seqs)
    oracle.set_threads(1)
    try:
        g1, d1, _ = _oracle_gbs(wl.config_workload(1), 1)
        g2, d2, _ = _oracle_gbs(w, 1, rows_per_seq=16)
    finally:
        oracle.set_threads(threads)
    n_seqs = max(1, min(n_seqs, w.B))
    lens = w.seqlens[:n_seqs]
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "seconds": round(dt, 3), "cpu_model": _cpu_model(), "nproc": os.cpu_count(),
            "sample": f"first {n_seqs} of {w.B} sequences (all {w.s_q * w.H} query rows, "
                      f"{int(lens.min())}..{int(lens.max())} tokens), fp64 two-pass oracle, "
                      "same seeded inputs",
            "single_thread": {
                "tiny_b1_h16_l256": {"value": round(g1, 4), "unit": "GB/s",
                                     "seconds": round(d1, 4)},
                f"{w.name}_one_seq_16_rows": {"value": round(g2, 4), "unit": "GB/s",
                                              "seconds": round(d2, 4)}}}


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
            "kernel": "one mla_decode step (decode kernel + LSE combine): one HIP event "
                      "pair on the launch stream around the K timed steps, divided by K",
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
    if args.mfma_probe:
        mfma_probe()
        return
    if args.lds_probe:
        lds_probe()
        return
    if args.layer_steps:
        layer_steps(args.steps)
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
    elif w.kv_dtype == "fp8":
        kv0 = torch.from_numpy(w.kv).to(dev)
        sc0 = torch.from_numpy(w.kv_scales).to(dev)
    else:
        kv0 = torch.from_numpy(w.kv).to(dev)
        sc0 = torch.from_numpy(w.kv_scales.view(np.int16)).view(torch.float16).to(dev)
    cache_bytes = kv0.numel() * kv0.element_size() + (
        0 if sc0 is None else sc0.numel() * sc0.element_size())
    # enough copies that the 256 MB MALL cannot hold the cache of a step; a
    # cache of a few MB (the 256-token workload) is rotated over 64 copies,
    # which leaves it MALL-resident as it would be in use
    copies = min(64, max(1, int(np.ceil(3 * 256e6 / cache_bytes)) + 1)) if cache_bytes < 16e6 \
        else max(1, int(np.ceil(3 * 256e6 / cache_bytes)) + 1)
    kvs = [kv0] + [kv0.clone() for _ in range(copies - 1)]
    scs = [sc0] + [None if sc0 is None else sc0.clone() for _ in range(copies - 1)]
    out = torch.empty((w.B, w.s_q, w.H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.s_q, w.H), dtype=torch.float32, device=dev)
    prob = mla.make_problem(q, kv0, bt, kv_dtype={"bf16": mla.KV_BF16, "q8_0": mla.KV_Q8_0,
                                                  "fp8": mla.KV_FP8,
                                                  "q4_0h": mla.KV_Q4_0H}[w.kv_dtype],
                            max_seqlen=w.max_seqlen, num_parts=args.num_parts,
                            m_tile=args.m_tile)
    ws = torch.empty(max(16, mla.workspace_size(prob)), dtype=torch.uint8, device=dev)
    parts = mla.problem_num_parts(prob)

    def step(i):
        mla.mla_decode(q, kvs[i % copies], bt, sl, w.softmax_scale, out, lse,
                       kv_scales=scs[i % copies], max_seqlen=w.max_seqlen,
                       num_parts=args.num_parts, m_tile=args.m_tile, workspace=ws)

    # Clock settling: from idle, the decode kernel of the bench workload runs
    # at about 99 us over its first hundred launches, 91 us over the next
    # hundred and 82-84 us from about 20 ms of back-to-back work on (rocprofv3
    # trace, one box), as the GPU's clocks come up. The same step is repeated,
    # untimed, for settle_ms before the W warmup steps, so that the K timed
    # steps measure the sustained rate; the JSON line reports it.
    settle_steps = 0
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(20):
            step(settle_steps)
            settle_steps += 1
        torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - t_settle) * 1e3
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    # One HIP event pair on the launch stream brackets the whole timed region:
    # an event recorded between steps is a barrier packet of its own, and
    # bracketing every step that way added about 20 us to a 90 us step of the
    # bench workload (measured on one box: 90-91 us a step without per-step
    # events, 107-114 us with them).
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if not args.graph:
        # eager: one library call per step from Python
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for i in range(args.steps):
            step(i)
        e1.record(stream)
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
        t0 = time.perf_counter()
        e0.record(stream)
        for g, _ in plan:
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    avg_ms = e0.elapsed_time(e1) / args.steps
    ms_per_step = wall / args.steps * 1e3
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (avg_ms * 1e-3) / 1e9

    traffic = None
    tfile = os.path.join(ROOT, "profiles", f"hbm_traffic_{w.name}.json")
    if os.path.exists(tfile):
        rec = json.load(open(tfile))
        if rec.get("source_hash") == source_hash() and rec.get("num_parts") == parts:
            traffic = rec.get("bytes_per_launch")

    # matrix-core counters of the same workload and source (rocprofv3 run
    # summarised under profiles/), reported beside the algorithmic fractions
    mfma_counters = None
    mfile = os.path.join(ROOT, "profiles", f"mfma_{w.name}.json")
    if os.path.exists(mfile):
        rec = json.load(open(mfile))
        if rec.get("source_hash") == source_hash():
            mfma_counters = {"probe_tflops": rec.get("probe_tflops"),
                             "per_kernel": {k: {"busy_frac": v["mfma_busy_frac"],
                                                "executed_frac_of_probe": v["executed_frac_of_probe"],
                                                "median_duration_us": v["median_duration_us"]}
                                            for k, v in rec["per_kernel"].items()
                                            if v.get("executed_bf16_flops", 0) > 0}}
            if w.kv_dtype == "fp8":
                # its scores run on fp8 MFMAs, which the bf16 MOPS counter
                # does not count; the busy fraction covers both kinds
                mfma_counters["executed_counts"] = "bf16 value MFMAs only (fp8 score MFMAs not counted)"

    lo, hi = int(w.seqlens.min()), int(w.seqlens.max())
    seqlen_desc = lo if lo == hi else f"{lo}..{hi} (mean {float(w.seqlens.mean()):.1f})"
    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"bf16": "bf16", "q8_0": "q8_0 cache, bf16 MFMA",
                  "fp8": "fp8 (e4m3) cache, bf16 MFMA",
                  "q4_0h": "q4_0 cache in Hadamard rotation, bf16 MFMA"}[w.kv_dtype],
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "heads": w.H, "seqlen": seqlen_desc,
                   "seqlen_q": w.s_q, "kv_cache": f"{w.kv_dtype}, paged 64-token blocks, "
                   "576 = 512 latent + 64 rope", "d_latent": 512, "d_rope": 64,
                   "num_parts": parts, "m_tile": args.m_tile or "auto",
                   "cache_copies_rotated": copies,
                   "launch": "hip_graph" if args.graph else "eager"},
        "tflops": round(flops / (avg_ms * 1e-3) / 1e12, 2),
        "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
        "event_ms": {"mean": round(avg_ms, 5)},
        "clock_settle": {"untimed_steps": settle_steps, "ms": round(settle_ms, 1)},
        "roofline": roofline(nbytes, flops, avg_ms, traffic),
    }
    if mfma_counters:
        res["roofline"]["mfma_counters"] = mfma_counters
    if not args.no_cpu_baseline:
        n_cpu = args.cpu_seqs or (2 if w.kv_dtype == "q4_0h" else 64)
        res["cpu_baseline"] = cpu_baseline(w, n_cpu)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
