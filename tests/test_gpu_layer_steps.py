"""GPU parity of the steps either side of the decode kernel (query absorption,
output projection, cache append) against the CPU oracle, through the C ABI,
and the whole chain q_nope -> absorb -> decode -> project against the
decompressed per-head definition, stage by stage."""
import math

import numpy as np
import pytest
import torch

import mla_latent_kv_10_amd as mla
import oracle
import workload as wl
from gpu_helpers import compare, device_inputs, log, oracle_rows, require_library, run_gpu

pytestmark = pytest.mark.gpu

# Bar of a bf16-in, fp32-accumulate, bf16-out product over n terms:
#   |gpu - ref| <= 2^-8 |ref| + n * 2^-24 * sum |terms|
# (output rounding to bf16, unit roundoff 2^-8; each bf16 x bf16 product is
# exact in fp32 and each of the n-1 fp32 additions rounds by at most 2^-24 of
# the partial sum, bounded by sum |terms|).
BF16_U = 2.0 ** -8


@pytest.fixture(scope="module", autouse=True)
def _lib():
    require_library()
    assert torch.cuda.is_available()


def _bf16_tensor(bits, dev="cuda"):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def _bits_of(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _weights(H, seed):
    """W_UK, W_UV [H, 128, 512] ~ N(0, 1/512), rounded to bf16 (bits, float64)."""
    bk = wl.normal_bf16(H * 128 * 512, seed, wl.S_WUK, stddev=1 / math.sqrt(512)).reshape(H, 128, 512)
    bv = wl.normal_bf16(H * 128 * 512, seed, wl.S_WUV, stddev=1 / math.sqrt(512)).reshape(H, 128, 512)
    return bk, bv, wl.bf16_bits_to_f32(bk).astype(np.float64), wl.bf16_bits_to_f32(bv).astype(np.float64)


def _product_bar(ref, mag, n):
    return BF16_U * np.abs(ref) + n * 2.0 ** -24 * mag


def _absorb_gpu(qn_bits, qr_bits, wk_bits):
    wk_t = np.ascontiguousarray(np.swapaxes(wk_bits, 1, 2))   # layout of the entry point
    q_abs = mla.mla_absorb_query(_bf16_tensor(qn_bits), _bf16_tensor(qr_bits), _bf16_tensor(wk_t))
    torch.cuda.synchronize()
    return _bits_of(q_abs)


@pytest.mark.parametrize("B,s_q,H", [(1, 1, 16), (64, 1, 128), (3, 2, 40), (70, 1, 8)])
def test_absorb_query_matches_the_oracle(B, s_q, H):
    seed = 500 + B + H
    wk_bits, _, wk, _ = _weights(H, seed)
    qn_bits = wl.normal_bf16(B * s_q * H * 128, seed, wl.S_QNOPE).reshape(B, s_q, H, 128)
    qr_bits = wl.normal_bf16(B * s_q * H * 64, seed, wl.S_QROPE).reshape(B, s_q, H, 64)
    got = _absorb_gpu(qn_bits, qr_bits, wk_bits)
    qn = wl.bf16_bits_to_f32(qn_bits).astype(np.float64)
    qr = wl.bf16_bits_to_f32(qr_bits).astype(np.float64)
    ref = oracle.absorb_query(qn, qr, wk)
    # the RoPE slice is copied bit for bit
    assert np.array_equal(got[..., 512:], qr_bits)
    g = wl.bf16_bits_to_f32(got[..., :512]).astype(np.float64)
    # sum_j |W_UK[h][j][d] q_nope[j]| per output value
    mag = np.einsum("bihj,hjd->bihd", np.abs(qn), np.abs(wk))
    err = np.abs(g - ref[..., :512])
    log(f"absorb B={B} s_q={s_q} H={H}: max|err| {err.max():.3e}, max|ref| {np.abs(ref).max():.3e}")
    assert np.all(err <= _product_bar(ref[..., :512], mag, 128))


@pytest.mark.parametrize("B,s_q,H", [(1, 1, 16), (64, 1, 128), (3, 2, 40), (70, 1, 8)])
def test_project_output_matches_the_oracle(B, s_q, H):
    seed = 600 + B + H
    _, wv_bits, _, wv = _weights(H, seed)
    ol_bits = wl.normal_bf16(B * s_q * H * 512, seed, 30).reshape(B, s_q, H, 512)
    o = mla.mla_project_output(_bf16_tensor(ol_bits), _bf16_tensor(wv_bits))
    torch.cuda.synchronize()
    g = wl.bf16_bits_to_f32(_bits_of(o)).astype(np.float64)
    ol = wl.bf16_bits_to_f32(ol_bits).astype(np.float64)
    ref = oracle.project_output(ol, wv)
    mag = np.einsum("bihd,hjd->bihj", np.abs(ol), np.abs(wv))
    err = np.abs(g - ref)
    log(f"project B={B} s_q={s_q} H={H}: max|err| {err.max():.3e}, max|ref| {np.abs(ref).max():.3e}")
    assert np.all(err <= _product_bar(ref, mag, 512))


@pytest.mark.parametrize("kvd", ["bf16", "q8_0", "fp8", "q4_0h"])
def test_cache_append_is_bit_exact(kvd):
    """Every byte of the cache after an append equals the oracle's: the new
    rows land at their positions (q8_0: quantised by the same rule), rows
    outside the table or in an invalid block are skipped, nothing else moves."""
    w = wl.make_workload("append", 5, 2, 16, [130, 1, 64, 200, 70], seed=71, table="permuted",
                         kv_dtype=kvd, max_blocks=4)
    w.block_table[4, 1] = w.num_blocks + 2          # positions 68, 69 land in a bad block
    new_bits = wl.normal_bf16(5 * 2 * 576, 71, 41).reshape(5, 2, 576)
    t = device_inputs(w)
    mla.mla_cache_append(_bf16_tensor(new_bits), t["bt"], t["sl"], t["kv"], t["kv_scales"])
    torch.cuda.synchronize()
    kv_ref = w.kv.copy()
    sc_ref = None if kvd == "bf16" else w.kv_scales.copy()
    n = oracle.cache_append(new_bits, w.block_table, w.seqlens, kv_ref, sc_ref)
    assert n == 2 + 1 + 2 + 2 + 0
    if kvd == "bf16":
        assert np.array_equal(_bits_of(t["kv"]), kv_ref)
    elif kvd == "fp8":
        assert np.array_equal(t["kv"].cpu().numpy(), kv_ref)
        assert np.array_equal(t["kv_scales"].cpu().numpy().view(np.uint32), sc_ref.view(np.uint32))
    else:
        assert np.array_equal(t["kv"].cpu().numpy(), kv_ref)
        assert np.array_equal(t["kv_scales"].view(torch.int16).cpu().numpy().view(np.uint16), sc_ref)


@pytest.mark.parametrize("kvd", ["bf16", "q8_0", "fp8", "q4_0h"])
def test_append_then_decode(kvd):
    """A decode step after the append reads the appended rows: it matches the
    oracle's decode of the oracle-appended cache."""
    w = wl.make_workload("app_dec", 3, 2, 128, [300, 2, 1000], seed=72, table="permuted",
                         kv_dtype=kvd)
    new_bits = wl.normal_bf16(3 * 2 * 576, 72, 41).reshape(3, 2, 576)
    t = device_inputs(w)
    mla.mla_cache_append(_bf16_tensor(new_bits), t["bt"], t["sl"], t["kv"], t["kv_scales"])
    out, lse = mla.mla_decode(t["q"], t["kv"], t["bt"], t["sl"], w.softmax_scale,
                              kv_scales=t["kv_scales"], max_seqlen=w.max_seqlen)
    torch.cuda.synchronize()
    oracle.cache_append(new_bits, w.block_table, w.seqlens, w.kv, w.kv_scales)
    compare(out.float().cpu().numpy(), lse.cpu().numpy(), *oracle_rows(w),
            what=f"append+decode {kvd}", kv_dtype=kvd)


@pytest.mark.parametrize("cfg_B,H,L", [(1, 16, 256), (2, 128, 200)])
def test_layer_chain_matches_the_decompressed_definition(cfg_B, H, L):
    """q_nope -> GPU absorb -> GPU decode -> GPU project, each stage checked
    against the oracle on that stage's own inputs at its own bar, then the
    whole chain against the per-head decompressed definition (explicit
    k = W_UK c, v = W_UV c, standard softmax) in fp64."""
    seed = 700 + H
    w = wl.make_workload("chain", cfg_B, 1, H, L, seed=seed, table="permuted")
    wk_bits, wv_bits, wk, wv = _weights(H, seed)
    qn_bits = wl.normal_bf16(cfg_B * H * 128, seed, wl.S_QNOPE).reshape(cfg_B, 1, H, 128)
    qr_bits = wl.normal_bf16(cfg_B * H * 64, seed, wl.S_QROPE).reshape(cfg_B, 1, H, 64)
    qn = wl.bf16_bits_to_f32(qn_bits).astype(np.float64)
    qr = wl.bf16_bits_to_f32(qr_bits).astype(np.float64)
    # stage 1: absorption
    q_abs = _absorb_gpu(qn_bits, qr_bits, wk_bits)
    ref_abs = oracle.absorb_query(qn, qr, wk)
    g = wl.bf16_bits_to_f32(q_abs).astype(np.float64)
    mag = np.einsum("bihj,hjd->bihd", np.abs(qn), np.abs(wk))
    assert np.all(np.abs(g[..., :512] - ref_abs[..., :512]) <= _product_bar(ref_abs[..., :512], mag, 128))
    # stage 2: decode on the GPU's absorbed query, against the oracle on the same bits
    w.q = q_abs.reshape(cfg_B, 1, H, 576)
    out, lse, out_bits = run_gpu(w)
    compare(out, lse, *oracle_rows(w), what=f"chain decode H={H}")
    # stage 3: output projection on the GPU's latent output
    o = mla.mla_project_output(_bf16_tensor(out_bits), _bf16_tensor(wv_bits))
    torch.cuda.synchronize()
    og = wl.bf16_bits_to_f32(_bits_of(o)).astype(np.float64)
    ol = wl.bf16_bits_to_f32(out_bits).astype(np.float64)
    ref_o = oracle.project_output(ol, wv)
    magv = np.einsum("bihd,hjd->bihj", np.abs(ol), np.abs(wv))
    assert np.all(np.abs(og - ref_o) <= _product_bar(ref_o, magv, 512))
    # the chain against the decompressed definition: what remains is the bf16
    # rounding of q~ (scores move by at most scale * 2^-8 * sum_d |q~_d x_d|),
    # of the decode's arithmetic (bar above) and of o_lat and o
    o_ref, lse_ref = oracle.decode_decompressed(qn, qr, wk, wv, w.kv, w.block_table, w.seqlens,
                                                w.softmax_scale)
    kv = wl.bf16_bits_to_f32(w.kv).astype(np.float64).reshape(-1, 576)
    ds = w.softmax_scale * BF16_U * (np.abs(ref_abs.reshape(-1, 576)) @ np.abs(kv).T).max()
    lerr = np.abs(lse - lse_ref).max()
    oerr = np.abs(og - o_ref).max()
    log(f"chain H={H}: lse max|err| {lerr:.3e} (score shift bound {ds:.3e}), "
        f"o max|err| {oerr:.3e}, max|o| {np.abs(o_ref).max():.3e}")
    assert lerr <= ds + 1e-3
    # output: the weights move by a factor within exp(+-2 ds), so o by at most
    # (e^{2 ds} - 1) * sum_t p_t |v_t|, bounded by that factor times
    # max_j sum_d |W_UV[h][j][d]| * max |c|
    v_max = np.abs(wv).sum(-1).max() * np.abs(kv[:, :512]).max()
    assert oerr <= (math.exp(2 * ds) - 1) * v_max + 2e-2 * max(1.0, np.abs(o_ref).max())
