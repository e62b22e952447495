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

# Parity bar (bf16 inputs, fp32 accumulation, bf16 output), per element e of
# an output row:
#
#   |gpu - ref| <= 2e-2 + k * 2^-8 * A_e,    A_e = sum_t p_t |V_t[e]|
#
# A_e (from the oracle) is the size of the terms behind the value; |out_e| <=
# A_e. 2^-8 is the unit roundoff of bf16 (8 significant bits, round to
# nearest even): rounding x to bf16 moves it by at most 2^-8 |x|. k counts the
# bf16 roundings the kernel's arithmetic puts on the value path, each of which
# moves out_e by at most 2^-8 A_e:
#   1. the probabilities p_t, rounded to bf16 before the value product (the
#      normaliser l sums the unrounded fp32 values);
#   2. the output, rounded to bf16;
#   3. a sequence cut into several KV parts: each part's normalised output is
#      held in bf16 until the parts are merged (merge weights sum to 1, so the
#      parts' A_e average to A_e);
#   4. a q8_0 cache: the dequantised value scale * int8 (exact in fp32) is
#      rounded to bf16 for the value product (the scores use it unrounded);
#      a q4_0 cache in Hadamard rotation likewise: the rotated-back value
#      d / sqrt(32) * n (n the integer Hadamard sum of the codes, exact) is
#      rounded to bf16 for the value product, the scores use n exactly and
#      d in fp32.
# So k = 3 for a bf16 cache and 4 for a q8_0 or q4_0 cache (the split case
# bounds the unsplit one). An fp8 (E4M3) cache converts to bf16 exactly and its
# per-token scale multiplies the score and the probability in fp32 before
# rounding (1), so k = 3 as for bf16. The 2e-2 term absorbs what is left:
# fp32 accumulation, the exp2 approximation and score rounding, all orders of
# magnitude smaller.
# A flat 2e-2 cannot hold in general: bf16 cannot hold values above 8 to
# within 2e-2, and the long-context workload's x8 rows reach |out| = 30.
# Where the workload keeps A_e small enough for the flat bound to be
# attainable, the flat bound is asserted as well (flat=True).
#   max |gpu - ref| <= 1e-2 * max |ref| over the tensor;
#   |lse_gpu - lse_ref| <= 1e-3 (absolute).
OUT_ABS_TOL = 2e-2
BF16_U = 2.0 ** -8
ROUNDINGS = {"bf16": 3, "q8_0": 4, "fp8": 3, "q4_0h": 4}
OUT_REL_TOL = 1e-2
LSE_ABS_TOL = 1e-3

# (what, max|err|, max|ref|, margin left under the bar, lse max|err|) of every
# comparison, printed in the terminal summary (tests/conftest.py)
REPORT: list = []


def out_quantum(kv_dtype: str) -> float:
    return ROUNDINGS[kv_dtype] * BF16_U


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
    elif w.kv_dtype == "fp8":
        t["kv"] = torch.from_numpy(w.kv).to(dev)
        t["kv_scales"] = torch.from_numpy(w.kv_scales).to(dev)
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


def compare(out, lse, ref_out, ref_lse, ref_abs=None, what="", kv_dtype="bf16", flat=False):
    """Assert the parity bar; NaN / -inf must match exactly in place.
    ref_abs: the oracle's term magnitudes A_e (defaults to |ref_out|).
    kv_dtype: the cache type of the run (sets k in the bar above).
    flat: also assert the flat bound max|err| <= 2e-2."""
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
    quantum = out_quantum(kv_dtype)
    diff = np.abs(out[ok] - ref_out[ok])
    assert np.all(np.isfinite(diff)), f"{what}: non-finite output where the oracle is finite"
    err = float(diff.max())
    excess = float((diff - quantum * ref_abs[ok]).max())
    ref_max = float(np.abs(ref_out[ok]).max())
    lerr = float(np.abs(lse[ok] - ref_lse[ok]).max())
    margin = OUT_ABS_TOL - excess
    REPORT.append((what, err, ref_max, margin, lerr, int(ok.sum())))
    log(f"  {what}: rows {int(ok.sum())}, out max|err| {err:.3e} (max|ref| {ref_max:.3e}; "
        f"beyond {ROUNDINGS[kv_dtype]}x2^-8 A: {excess:.3e}, margin {margin:.3e}), "
        f"lse max|err| {lerr:.3e}")
    assert excess <= OUT_ABS_TOL, (f"{what}: out error {excess} beyond the bf16 roundings "
                                   f"> {OUT_ABS_TOL}")
    assert err <= OUT_REL_TOL * ref_max, f"{what}: out error {err} > 1e-2 * {ref_max}"
    assert lerr <= LSE_ABS_TOL, f"{what}: lse error {lerr}"
    if flat:
        assert err <= OUT_ABS_TOL, f"{what}: out error {err} > flat {OUT_ABS_TOL}"
    return dict(max_abs=err, lse_abs=lerr, margin=margin)


def sample_rows(w: wl.Workload, n: int, seed: int = 0):
    """Seeded sample of row ids, always including the first and last rows."""
    total = w.rows
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(total, size=min(n, total), replace=False).tolist())
    rows.update([0, total - 1])
    return np.array(sorted(rows), np.int64)
