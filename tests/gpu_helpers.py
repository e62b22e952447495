"""Shared helpers of the GPU parity tests: move a workload to the device,
run libmla through its C ABI binding, compare with the CPU oracle."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

import mla_latent_kv_10_amd as mla
import oracle
import workload as wl

# Parity bar: bf16 inputs, fp32 accumulation, bf16 output.
#   |gpu - ref| <= 2e-2 + 2^-7 A per element, where A = sum_t p_t |V_t| (from
#     the oracle) is the magnitude of the terms behind the value: 2e-2
#     absolute, plus the two bf16 roundings the arithmetic implies, each at most
#     2^-8 relative to the terms: the probabilities entering the value product
#     and the stored output. (A bf16 output cannot even hold values above 8 to
#     2e-2; the long-context workload's x8 rows reach |out| = 30, and terms of
#     +-30 partly cancel.) For unit-scale data A is about 1 and the bound is
#     about 2.8e-2;
#   max |gpu - ref| <= 1e-2 * max |ref| over the tensor;
#   |lse_gpu - lse_ref| <= 1e-3.
OUT_ABS_TOL = 2e-2
OUT_QUANTUM = 2.0 ** -7
OUT_REL_TOL = 1e-2
LSE_ABS_TOL = 1e-3


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def require_library():
    if not os.path.exists(mla.LIB_PATH):
        raise RuntimeError("libmla.so is not built; run __graft_entry__.build() first")
    mla.lib()


def device_inputs(w: wl.Workload, dev="cuda"):
    t = {}
    t["q"] = torch.from_numpy(w.q.view(np.int16)).view(torch.bfloat16).to(dev)
    if w.kv_dtype == "bf16":
        t["kv"] = torch.from_numpy(w.kv.view(np.int16)).view(torch.bfloat16).to(dev)
        t["kv_scales"] = None
    else:
        t["kv"] = torch.from_numpy(w.kv).to(dev)
        t["kv_scales"] = torch.from_numpy(w.kv_scales.view(np.int16)).view(torch.float16).to(dev)
    t["bt"] = torch.from_numpy(w.block_table).to(dev)
    t["sl"] = torch.from_numpy(w.seqlens).to(dev)
    return t


def run_gpu(w: wl.Workload, t=None, **kw):
    """-> (out float64 [B, s_q, H, 512], lse float64 [B, s_q, H], out bf16 bits)."""
    if t is None:
        t = device_inputs(w)
    out, lse = mla.mla_decode(t["q"], t["kv"], t["bt"], t["sl"], w.softmax_scale,
                              kv_scales=t["kv_scales"], max_seqlen=w.max_seqlen, **kw)
    torch.cuda.synchronize()
    bits = out.view(torch.int16).cpu().numpy().view(np.uint16)
    return (out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
            bits)


def oracle_rows(w: wl.Workload, rows=None):
    """-> (out, lse, out_abs) from the oracle (all rows, or the listed ones)."""
    return oracle.decode_absorbed(w.q, w.kv, w.block_table, w.seqlens, w.softmax_scale,
                                  kv_scales=w.kv_scales, rows=rows, with_abs=True)


def compare(out, lse, ref_out, ref_lse, ref_abs=None, what=""):
    """Assert the parity bar; NaN / -inf must match exactly in place.
    ref_abs: the oracle's term magnitudes (defaults to |ref_out|)."""
    out = np.asarray(out, np.float64).reshape(-1, 512)
    ref_out = np.asarray(ref_out, np.float64).reshape(-1, 512)
    ref_abs = (np.abs(ref_out) if ref_abs is None
               else np.asarray(ref_abs, np.float64).reshape(-1, 512))
    lse = np.asarray(lse, np.float64).reshape(-1)
    ref_lse = np.asarray(ref_lse, np.float64).reshape(-1)
    assert out.shape == ref_out.shape and lse.shape == ref_lse.shape
    nan_ref = np.isnan(ref_lse)
    assert np.array_equal(np.isnan(lse), nan_ref), f"{what}: NaN rows differ"
    assert np.all(np.isnan(out[nan_ref])), f"{what}: poisoned rows must be NaN"
    ninf = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), ninf), f"{what}: empty rows differ"
    assert np.all(out[ninf] == 0), f"{what}: empty rows must be zero"
    ok = ~nan_ref & ~ninf
    if not ok.any():
        return dict(max_abs=0.0, lse_abs=0.0)
    diff = np.abs(out[ok] - ref_out[ok])
    err = diff.max()
    excess = (diff - OUT_QUANTUM * ref_abs[ok]).max()
    ref_max = np.abs(ref_out[ok]).max()
    lerr = np.abs(lse[ok] - ref_lse[ok]).max()
    log(f"  {what}: out max|err| {err:.3e} (max|ref| {ref_max:.3e}, beyond bf16 steps "
        f"{excess:.3e}), lse max|err| {lerr:.3e}")
    assert excess <= OUT_ABS_TOL, f"{what}: out error {excess} beyond the bf16 steps > {OUT_ABS_TOL}"
    assert err <= OUT_REL_TOL * ref_max, f"{what}: out error {err} > 1e-2 * {ref_max}"
    assert lerr <= LSE_ABS_TOL, f"{what}: lse error {lerr}"
    return dict(max_abs=float(err), lse_abs=float(lerr))


def sample_rows(w: wl.Workload, n: int, seed: int = 0):
    """Seeded sample of row ids, always including the first and last rows and,
    for every sampled sequence, its last head of the last query token."""
    total = w.rows
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(total, size=min(n, total), replace=False).tolist())
    rows.update([0, total - 1])
    return np.array(sorted(rows), np.int64)
