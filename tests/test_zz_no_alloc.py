"""The allocation-free decode entry point (mla_decode_noalloc) through the C
ABI: on the library's own per-device workspace it gives mla_decode's result
bit for bit (same kernels, same plan), and the oracle's within the parity
bar, on two calls in a row (the second smaller, so it runs over what the
first left in the shared workspace); problems whose workspace exceeds the
array are refused before anything is enqueued."""
import ctypes

import pytest
import torch

import mla_latent_kv_10_amd as mla
import workload as wl
from gpu_helpers import compare, device_inputs, log, oracle_rows, require_library

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    require_library()
    assert torch.cuda.is_available()


def _both(w, **kw):
    """-> (noalloc out, lse, reference-entry-point out, lse) as host arrays."""
    t = device_inputs(w)
    shape = (w.B, w.s_q, w.H)
    out_n = torch.full(shape + (512,), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse_n = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    mla.mla_decode_noalloc(t["q"], t["kv"], t["bt"], t["sl"], w.softmax_scale, out_n, lse_n,
                           kv_scales=t["kv_scales"], max_seqlen=w.max_seqlen, **kw)
    torch.cuda.synchronize()
    out_r, lse_r = mla.mla_decode(t["q"], t["kv"], t["bt"], t["sl"], w.softmax_scale,
                                  kv_scales=t["kv_scales"], max_seqlen=w.max_seqlen, **kw)
    torch.cuda.synchronize()
    return out_n, lse_n, out_r, lse_r


def _check(w, what, **kw):
    out_n, lse_n, out_r, lse_r = _both(w, **kw)
    assert torch.equal(out_n.view(torch.int16), out_r.view(torch.int16)), f"{what}: out differs"
    assert torch.equal(lse_n, lse_r), f"{what}: lse differs"
    compare(out_n.float().cpu().numpy(), lse_n.cpu().numpy(), *oracle_rows(w), what=what,
            kv_dtype=w.kv_dtype)


def test_noalloc_matches_decode_on_two_calls_in_a_row():
    # first call: 128 heads, sequences split over several parts (partials and
    # the merge run in the shared array)
    w1 = wl.make_workload("noalloc1", 6, 1, 128, [4096, 3000, 1, 2500, 4000, 777], seed=41,
                          table="permuted")
    log("noalloc call 1: 6 x 128 heads, ragged up to 4096 tokens")
    _check(w1, "noalloc 1")
    # second call, smaller: 16 heads, two sequences, forced split
    w2 = wl.make_workload("noalloc2", 2, 1, 16, [900, 130], seed=42, table="permuted")
    log("noalloc call 2: 2 x 16 heads, 5 parts")
    _check(w2, "noalloc 2", num_parts=5)


@pytest.mark.parametrize("kvd,H", [("q8_0", 64), ("fp8", 128), ("q4_0h", 128)])
def test_noalloc_quantised_cache_and_causal_pair(kvd, H):
    w = wl.make_workload(f"noalloc_{kvd}", 3, 2, H, [700, 2100, 65], seed=43, table="permuted",
                         kv_dtype=kvd)
    log(f"noalloc {kvd}, {H} heads, causal pairs")
    _check(w, f"noalloc {kvd}")


def test_noalloc_refuses_a_workspace_beyond_the_array():
    w = wl.make_workload("noalloc_big", 2, 1, 128, [2000, 64], seed=44)
    t = device_inputs(w)
    out = torch.zeros((w.B, 1, w.H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((w.B, 1, w.H), dtype=torch.float32, device="cuda")
    prob = mla.make_problem(t["q"], t["kv"], t["bt"], kv_dtype=mla.KV_BF16,
                            max_seqlen=w.max_seqlen, num_parts=400000)
    assert mla.workspace_size(prob) > mla.NOALLOC_SCRATCH_BYTES
    vp = ctypes.c_void_p
    st = mla.lib().mla_decode_noalloc(ctypes.byref(prob), vp(t["q"].data_ptr()),
                                      vp(t["kv"].data_ptr()), None, vp(t["bt"].data_ptr()),
                                      vp(t["sl"].data_ptr()), ctypes.c_float(w.softmax_scale),
                                      vp(out.data_ptr()), vp(lse.data_ptr()),
                                      vp(torch.cuda.current_stream().cuda_stream))
    assert st == 2, mla.lib().mla_last_error().decode()
    assert "MLA_NOALLOC_SCRATCH_BYTES" in mla.lib().mla_last_error().decode()
    torch.cuda.synchronize()
    assert torch.count_nonzero(out.view(torch.int16)) == 0 and torch.count_nonzero(lse) == 0
