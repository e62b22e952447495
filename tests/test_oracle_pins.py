"""Pins of the CPU oracle to facts outside itself (CPU only).

Each test checks the oracle against something the pages or the mathematics
fix: closed forms of softmax attention, the absorption identity of MLA, exact
rows under a one-hot probe, the LSE merge of a token partition, IEEE
bfloat16 / binary16 bit patterns, and the partition rule's invariants. A
plausible mistake in the oracle (a dropped RoPE slice, a wrong block index,
a transposed W, a log base, an off-by-one in the causal rule) fails at least
one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import workload as wl

HERE = os.path.dirname(os.path.abspath(__file__))


def _bf16(x):
    return wl.f32_to_bf16_bits(np.asarray(x, np.float32))


def _bf16s(x):
    return int(_bf16([x])[0])


def _rows_f64(w):
    """Dequantized cache as float64 [num_blocks, 64, 576] (bf16 only)."""
    return wl.bf16_bits_to_f32(w.kv).astype(np.float64).reshape(w.kv.shape)


def _seq_rows(w, b):
    """The cache rows of sequence b in logical order, float64 [L, 576]."""
    kvf = _rows_f64(w)
    L = int(w.seqlens[b])
    ids = w.block_table[b, : (L + 63) // 64]
    return kvf[ids].reshape(-1, 576)[:L]


# ----------------------------------------------------------- number formats
def test_bf16_bit_patterns():
    # bfloat16 = top half of binary32: sign, 8-bit exponent (bias 127), 7-bit fraction
    cases = {0x3F80: 1.0, 0xC000: -2.0, 0x3E80: 0.25, 0x4049: 3.140625,
             0x0001: 2.0 ** -133, 0x0080: 2.0 ** -126, 0x7F7F: (2 - 2 ** -7) * 2.0 ** 127,
             0x8000: -0.0}
    for bits, val in cases.items():
        assert oracle.bf16_value(bits) == val


def test_fp16_bit_patterns():
    # IEEE 754 binary16: 5-bit exponent (bias 15), 10-bit fraction, subnormals m * 2^-24
    cases = {0x3C00: 1.0, 0xC000: -2.0, 0x0001: 2.0 ** -24, 0x03FF: 1023 * 2.0 ** -24,
             0x0400: 2.0 ** -14, 0x7BFF: 65504.0, 0x3555: 0.333251953125, 0x2C00: 0.0625}
    for bits, val in cases.items():
        assert oracle.fp16_value(bits) == val
    assert math.isinf(oracle.fp16_value(0x7C00))
    assert math.isnan(oracle.fp16_value(0x7E00))


def test_fp16_decoding_matches_numpy_for_all_finite_patterns():
    bits = np.arange(0, 0x7C00, 37, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.fp16_value(int(b)) for b in bits])
    assert np.array_equal(got, ref)


def test_q8_value_is_scale_times_int():
    assert oracle.q8_value(-127, 0x2C00) == -7.9375
    assert oracle.q8_value(0, 0x7BFF) == 0.0
    assert oracle.q8_value(5, 0x0001) == 5 * 2.0 ** -24


# ----------------------------------------------------- generator (shared) pins
def test_generator_fp16_rounding_matches_ieee_rne():
    x = wl.normal_f32(20000, 7, 1, stddev=3.0) * np.float32(0.01)
    x = np.concatenate([x, np.float32([6.1e-5, 5.96e-8, 2.98e-8, 3.0e-8, 65519.0, 65520.0])])
    got = np.array([wl._load().gen_f32_to_fp16(float(v)) for v in x], np.uint16)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)  # numpy rounds to nearest even
    assert np.array_equal(got, ref)


def test_generator_bf16_rounding_is_rne():
    # ties: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> even (1.0); 1 + 3*2^-8 -> up
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 1 + 2 ** -9], np.float32)
    assert list(wl.f32_to_bf16_bits(x)) == [0x3F80, 0x3F82, 0xBF80, 0x3F80]
    assert wl._load().gen_f32_to_bf16(float(x[1])) == 0x3F82


def test_generator_is_counter_based_and_normal():
    a = wl.normal_f64(4096, 11, 2)
    b = wl.normal_f64(1000, 11, 2, offset=3000)
    assert np.array_equal(a[3000:4000], b)
    big = wl.normal_f64(1 << 18, 5, 3)
    assert abs(big.mean()) < 0.01 and abs(big.std() - 1.0) < 0.01


def test_q8_writer_error_bound():
    x = wl.normal_f32(64 * 576, 3, 2).reshape(64, 576)
    q, d = wl.quantize_q8_0(x)
    for r in range(0, 64, 7):
        for g in range(18):
            scale = oracle.fp16_value(int(d[r, g]))
            d32 = float(np.abs(x[r, g * 32:(g + 1) * 32]).max()) / 127.0
            for k in range(32):
                xv = float(x[r, g * 32 + k])
                xh = oracle.q8_value(int(q[r, g * 32 + k]), int(d[r, g]))
                # half a step, plus the fp16 rounding of the scale times |q| <= 127
                assert abs(xv - xh) <= d32 / 2 + 127 * abs(scale - d32) + 1e-7


# ----------------------------------------------------------- closed forms
def test_zero_query_gives_mean_of_visible_rows_and_log_n():
    w = wl.make_workload("t", 2, 1, 3, [130, 64], seed=21, table="permuted")
    w.q[:] = 0
    out, lse = oracle.decode_absorbed(w.q, w.kv, w.block_table, w.seqlens, w.softmax_scale)
    for b in range(2):
        rows = _seq_rows(w, b)
        mean = rows[:, :512].mean(axis=0)
        for h in range(3):
            np.testing.assert_allclose(out[b, 0, h], mean, rtol=0, atol=1e-13)
            assert abs(lse[b, 0, h] - math.log(rows.shape[0])) < 1e-13


def test_zero_scale_equals_zero_query():
    w = wl.make_workload("t", 1, 1, 2, [97], seed=22)
    o1, l1 = oracle.decode_absorbed(w.q, w.kv, w.block_table, w.seqlens, 0.0)
    mean = _seq_rows(w, 0)[:, :512].mean(axis=0)
    np.testing.assert_allclose(o1[0, 0, 1], mean, atol=1e-13)
    assert abs(l1[0, 0, 0] - math.log(97)) < 1e-13


def test_single_token_returns_the_latent_row_exactly():
    w = wl.make_workload("t", 3, 1, 4, [1, 1, 1], seed=23, table="permuted")
    out, lse = oracle.decode_absorbed(w.q, w.kv, w.block_table, w.seqlens, w.softmax_scale)
    qf = wl.bf16_bits_to_f32(w.q).astype(np.float64).reshape(w.q.shape)
    for b in range(3):
        row = _seq_rows(w, b)[0]
        for h in range(4):
            assert np.array_equal(out[b, 0, h], row[:512])  # p = 1 exactly
            s0 = w.softmax_scale * float(np.dot(qf[b, 0, h], row))
            assert abs(lse[b, 0, h] - s0) < 1e-12


def test_term_magnitude_closed_forms():
    # one token: out_abs = |row|; zero query: out_abs = mean |row|; always >= |out|
    w = wl.make_workload("t", 2, 1, 3, [1, 150], seed=35, table="permuted")
    out, lse, oabs = oracle.decode_absorbed(w.q, w.kv, w.block_table, w.seqlens,
                                            w.softmax_scale, with_abs=True)
    assert np.array_equal(oabs[0, 0, 1], np.abs(_seq_rows(w, 0)[0, :512]))
    assert np.all(oabs >= np.abs(out) - 1e-15)
    w.q[:] = 0
    out, lse, oabs = oracle.decode_absorbed(w.q, w.kv, w.block_table, w.seqlens,
                                            w.softmax_scale, with_abs=True)
    np.testing.assert_allclose(oabs[1, 0, 2], np.abs(_seq_rows(w, 1)[:, :512]).mean(axis=0),
                               atol=1e-13)
    o2, l2 = oracle.decode_absorbed(w.q, w.kv, w.block_table, w.seqlens, w.softmax_scale)
    assert np.array_equal(o2, out) and np.array_equal(l2, lse)


def test_two_tokens_is_a_logistic_mix():
    w = wl.make_workload("t", 1, 1, 5, [2], seed=24)
    out, lse = oracle.decode_absorbed(w.q, w.kv, w.block_table, w.seqlens, w.softmax_scale)
    qf = wl.bf16_bits_to_f32(w.q).astype(np.float64).reshape(w.q.shape)
    r = _seq_rows(w, 0)
    for h in range(5):
        s0 = w.softmax_scale * float(qf[0, 0, h] @ r[0])
        s1 = w.softmax_scale * float(qf[0, 0, h] @ r[1])
        p0 = 1.0 / (1.0 + math.exp(s1 - s0))
        exp_out = p0 * r[0, :512] + (1 - p0) * r[1, :512]
        np.testing.assert_allclose(out[0, 0, h], exp_out, atol=1e-12)
        assert abs(lse[0, 0, h] - (max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1))))) < 1e-12


def _one_hot_workload(B, H, seqlens, targets, seed, s_q=1, d_probe=7):
    """Rope columns zero except rope[d_probe] = 64 at each target token; the
    probed query row is zero except rope[d_probe] = 64; scale 1. The target
    logit is 4096 and every other logit is 0, so p = 1 on the target."""
    w = wl.make_workload("probe", B, s_q, H, seqlens, seed=seed, table="permuted")
    w.kv[:, :, 512:] = 0
    w.q[:] = 0
    w.q[..., 512 + d_probe] = _bf16s(64.0)
    for b, t in targets:
        phys = w.block_table[b, t // 64]
        w.kv[phys, t % 64, 512 + d_probe] = _bf16s(64.0)
    w.softmax_scale = 1.0
    return w


def test_one_hot_probe_returns_the_target_row_through_the_block_table():
    seqlens = [300, 64, 129]
    targets = [(0, 299), (1, 0), (2, 128)]
    w = _one_hot_workload(3, 2, seqlens, targets, seed=25)
    out, lse = oracle.decode_absorbed(w.q, w.kv, w.block_table, w.seqlens, 1.0)
    kvf = _rows_f64(w)
    for b, t in targets:
        phys = w.block_table[b, t // 64]
        for h in range(2):
            assert np.array_equal(out[b, 0, h], kvf[phys, t % 64, :512])
            assert lse[b, 0, h] == 4096.0


def test_rope_slice_takes_part_in_the_scores():
    # same probe, but moving the rope peak moves the output row: a dropped
    # RoPE slice would give the uniform mean instead
    w = _one_hot_workload(1, 1, [200], [(0, 77)], seed=26)
    out, _ = oracle.decode_absorbed(w.q, w.kv, w.block_table, w.seqlens, 1.0)
    assert np.array_equal(out[0, 0, 0], _seq_rows(w, 0)[77, :512])


def test_causal_pair_first_query_does_not_see_the_last_token():
    L = 150
    w = _one_hot_workload(1, 2, [L], [(0, L - 1)], seed=27, s_q=2)
    out, lse = oracle.decode_absorbed(w.q, w.kv, w.block_table, w.seqlens, 1.0)
    rows = _seq_rows(w, 0)
    # query 1 sees the probe row; query 0 sees L-1 tokens, all with logit 0
    assert np.array_equal(out[0, 1, 0], rows[L - 1, :512])
    np.testing.assert_allclose(out[0, 0, 0], rows[: L - 1, :512].mean(axis=0), atol=1e-13)
    assert abs(lse[0, 0, 1] - math.log(L - 1)) < 1e-12


def test_causal_pair_first_query_equals_single_token_decode_one_shorter():
    w = wl.make_workload("t", 2, 2, 3, [100, 65], seed=28)
    out2, lse2 = oracle.decode_absorbed(w.q, w.kv, w.block_table, w.seqlens, w.softmax_scale)
    q1 = np.ascontiguousarray(w.q[:, :1])
    out1, lse1 = oracle.decode_absorbed(q1, w.kv, w.block_table, w.seqlens - 1, w.softmax_scale)
    assert np.array_equal(out2[:, 0], out1[:, 0])
    assert np.array_equal(lse2[:, 0], lse1[:, 0])


def test_empty_rows_are_zero_with_minus_inf_lse():
    w = wl.make_workload("t", 3, 2, 2, [0, 1, 5], seed=29)
    out, lse = oracle.decode_absorbed(w.q, w.kv, w.block_table, w.seqlens, w.softmax_scale)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    # seqlen 1 with a pair: query 0 sees nothing, query 1 sees token 0
    assert np.all(out[1, 0] == 0) and np.all(np.isneginf(lse[1, 0]))
    assert np.array_equal(out[1, 1, 0], _seq_rows(w, 1)[0, :512])
    assert np.all(np.isfinite(lse[2]))


def test_invalid_block_ids_poison_only_their_sequence():
    w = wl.make_workload("t", 2, 1, 2, [70, 70], seed=30)
    ok_out, ok_lse = oracle.decode_absorbed(w.q, w.kv, w.block_table, w.seqlens, w.softmax_scale)
    bt = w.block_table.copy()
    bt[0, 1] = w.num_blocks  # out of range
    out, lse = oracle.decode_absorbed(w.q, w.kv, bt, w.seqlens, w.softmax_scale)
    assert np.all(np.isnan(out[0])) and np.all(np.isnan(lse[0]))
    assert np.array_equal(out[1], ok_out[1]) and np.array_equal(lse[1], ok_lse[1])


def test_seqlens_clamp_to_table_capacity():
    w = wl.make_workload("t", 1, 1, 2, [128], seed=31, max_blocks=2)
    a, la = oracle.decode_absorbed(w.q, w.kv, w.block_table, w.seqlens, w.softmax_scale)
    b, lb = oracle.decode_absorbed(w.q, w.kv, w.block_table, w.seqlens + 1000, w.softmax_scale)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_block_permutation_is_bit_invariant():
    w = wl.make_workload("t", 2, 1, 3, [200, 90], seed=32)
    out, lse = oracle.decode_absorbed(w.q, w.kv, w.block_table, w.seqlens, w.softmax_scale)
    perm = wl.permutation(w.num_blocks, 99, 1)
    kv2 = np.empty_like(w.kv)
    kv2[perm] = w.kv
    bt2 = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    out2, lse2 = oracle.decode_absorbed(w.q, kv2, bt2, w.seqlens, w.softmax_scale)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_row_subset_matches_full_run():
    w = wl.make_workload("t", 2, 2, 3, [70, 9], seed=33)
    out, lse = oracle.decode_absorbed(w.q, w.kv, w.block_table, w.seqlens, w.softmax_scale)
    rows = np.array([11, 0, 5, 7], np.int64)
    o2, l2 = oracle.decode_absorbed(w.q, w.kv, w.block_table, w.seqlens, w.softmax_scale,
                                    rows=rows)
    assert np.array_equal(o2, out.reshape(-1, 512)[rows])
    assert np.array_equal(l2, lse.reshape(-1)[rows])


def test_q8_cache_reads_scale_times_int():
    w = wl.make_workload("t", 1, 1, 2, [1], seed=34, kv_dtype="q8_0")
    out, _ = oracle.decode_absorbed(w.q, w.kv, w.block_table, w.seqlens, w.softmax_scale,
                                    kv_scales=w.kv_scales)
    phys = w.block_table[0, 0]
    exp_row = [oracle.q8_value(int(w.kv[phys, 0, d]), int(w.kv_scales[phys, 0, d // 32]))
               for d in range(512)]
    assert np.array_equal(out[0, 0, 1], np.array(exp_row))


# ------------------------------------------------------ absorption identity
@pytest.mark.parametrize("B,s_q,H,seqlens,seed", [
    (1, 1, 16, [256], 1001),            # the tiny decode shape
    (2, 2, 3, [70, 5], 41),
    (3, 1, 2, [1, 64, 130], 42),
])
def test_absorbed_equals_decompressed(B, s_q, H, seqlens, seed):
    """MLA's up-projections fold into the query and the output projection:
    attention over the latent with q~ = [W_UK^T q_nope; q_rope], followed by
    W_UV, equals explicit per-head attention with k = [W_UK c; k_rope] and
    v = W_UV c."""
    w = wl.make_workload("absorb", B, s_q, H, seqlens, seed=seed)
    w_uk = wl.normal_f64(H * 128 * 512, seed, wl.S_WUK, stddev=1 / math.sqrt(512)).reshape(H, 128, 512)
    w_uv = wl.normal_f64(H * 128 * 512, seed, wl.S_WUV, stddev=1 / math.sqrt(512)).reshape(H, 128, 512)
    q_nope = wl.normal_f64(B * s_q * H * 128, seed, wl.S_QNOPE).reshape(B, s_q, H, 128)
    q_rope = wl.normal_f64(B * s_q * H * 64, seed, wl.S_QROPE).reshape(B, s_q, H, 64)
    o_ref, lse_ref = oracle.decode_decompressed(q_nope, q_rope, w_uk, w_uv, w.kv, w.block_table,
                                                w.seqlens, w.softmax_scale)
    q_abs = oracle.absorb_query(q_nope, q_rope, w_uk)
    o_lat, lse_abs = oracle.decode_absorbed_f64q(q_abs, w.kv, w.block_table, w.seqlens,
                                                 w.softmax_scale)
    o_abs = oracle.project_output(o_lat, w_uv)
    scale = max(1.0, np.abs(o_ref).max())
    assert np.abs(o_abs - o_ref).max() <= 1e-10 * scale
    fin = np.isfinite(lse_ref)
    assert np.array_equal(fin, np.isfinite(lse_abs))
    assert np.abs(lse_abs[fin] - lse_ref[fin]).max() <= 1e-10 * max(1.0, np.abs(lse_ref[fin]).max())


def test_absorption_catches_a_missing_rope_slice():
    # the identity is sensitive: zeroing q_rope on one side breaks it
    B, s_q, H, seed = 1, 1, 2, 43
    w = wl.make_workload("absorb", B, s_q, H, [80], seed=seed)
    w_uk = wl.normal_f64(H * 128 * 512, seed, wl.S_WUK, stddev=1 / math.sqrt(512)).reshape(H, 128, 512)
    w_uv = wl.normal_f64(H * 128 * 512, seed, wl.S_WUV, stddev=1 / math.sqrt(512)).reshape(H, 128, 512)
    q_nope = wl.normal_f64(B * s_q * H * 128, seed, wl.S_QNOPE).reshape(B, s_q, H, 128)
    q_rope = wl.normal_f64(B * s_q * H * 64, seed, wl.S_QROPE).reshape(B, s_q, H, 64)
    o_ref, _ = oracle.decode_decompressed(q_nope, q_rope, w_uk, w_uv, w.kv, w.block_table,
                                          w.seqlens, w.softmax_scale)
    q_abs = oracle.absorb_query(q_nope, np.zeros_like(q_rope), w_uk)
    o_lat, _ = oracle.decode_absorbed_f64q(q_abs, w.kv, w.block_table, w.seqlens, w.softmax_scale)
    assert np.abs(oracle.project_output(o_lat, w_uv) - o_ref).max() > 1e-4


# ------------------------------------------------------------ LSE combine
def _partial(w, b, blk_lo, blk_hi):
    """Oracle attention of sequence b restricted to its blocks [blk_lo, blk_hi)."""
    bt = np.full((1, w.max_blocks), -1, np.int32)
    n = blk_hi - blk_lo
    bt[0, :n] = w.block_table[b, blk_lo:blk_hi]
    L = min(int(w.seqlens[b]), blk_hi * 64) - blk_lo * 64
    q = np.ascontiguousarray(w.q[b:b + 1])
    return oracle.decode_absorbed(q, w.kv, bt, np.array([max(L, 0)], np.int32), w.softmax_scale)


@pytest.mark.parametrize("cuts", [[2], [1, 3], [1, 2, 3, 4]])
def test_combine_of_a_token_partition_equals_unsplit(cuts):
    w = wl.make_workload("t", 1, 1, 4, [300], seed=44, table="permuted")
    full_o, full_l = oracle.decode_absorbed(w.q, w.kv, w.block_table, w.seqlens, w.softmax_scale)
    edges = [0] + cuts + [5]
    po, pl = [], []
    for lo, hi in zip(edges[:-1], edges[1:]):
        o, l = _partial(w, 0, lo, hi)
        po.append(o.reshape(-1, 512))
        pl.append(l.reshape(-1))
    po = np.stack(po).astype(np.float32)
    pl = np.stack(pl).astype(np.float32)
    out, lse = oracle.combine(po, pl)
    np.testing.assert_allclose(out, full_o.reshape(-1, 512), rtol=0, atol=2e-6)
    np.testing.assert_allclose(lse, full_l.reshape(-1), rtol=0, atol=2e-6)


def test_combine_ignores_empty_parts_and_handles_all_empty():
    po = wl.normal_f32(3 * 2 * 512, 1, 1).reshape(3, 2, 512)
    pl = np.array([[0.5, -np.inf], [-np.inf, -np.inf], [1.5, -np.inf]], np.float32)
    po[1] = 0
    po[:, 1] = 0
    out, lse = oracle.combine(po, pl)
    # row 0: weights e^0.5 : e^1.5 over parts 0 and 2
    w0 = 1 / (1 + math.e)
    np.testing.assert_allclose(out[0], w0 * po[0, 0] + (1 - w0) * po[2, 0], atol=1e-6)
    assert abs(lse[0] - (1.5 + math.log1p(math.exp(-1.0)))) < 1e-6
    assert np.all(out[1] == 0) and np.isneginf(lse[1])


def test_combine_single_part_is_identity():
    po = wl.normal_f32(1 * 3 * 512, 2, 1).reshape(1, 3, 512)
    pl = np.float32([[0.25, -3.0, 7.0]])
    out, lse = oracle.combine(po, pl)
    assert np.array_equal(out, po[0].astype(np.float64))
    assert np.array_equal(lse, pl[0].astype(np.float64))


# ---------------------------------------------------------------- the plan
def _part_of(part_start, x):
    return int(np.searchsorted(part_start, x, side="right") - 1)


@pytest.mark.parametrize("B,P,seed", [(1, 1, 1), (5, 3, 2), (128, 256, 3), (64, 256, 4),
                                      (7, 40, 5), (300, 17, 6)])
def test_plan_partition_invariants(B, P, seed):
    sl = wl.uniform_int(B, seed, 7, 0, 3000)
    sl[::5] = 0
    max_blocks = 40  # clamps lengths above 2560
    pl = oracle.plan(sl, max_blocks, P)
    pre, ps = pl["seq_prefix"], pl["part_start"]
    nb = (np.clip(sl.astype(np.int64), 0, max_blocks * 64) + 63) // 64
    assert np.array_equal(np.diff(pre), nb) and pre[0] == 0
    T = int(pre[-1])
    assert ps[0] == 0 and ps[-1] == T
    sizes = np.diff(ps)
    assert sizes.min() >= 0 and sizes.max() - sizes.min() <= 1
    slots = set()
    for b in range(B):
        f, l = int(pl["seq_first_part"][b]), int(pl["seq_last_part"][b])
        if nb[b] > 0:
            assert f == _part_of(ps, pre[b]) and l == _part_of(ps, pre[b + 1] - 1)
            assert ps[f] <= pre[b] < ps[f + 1] and ps[l] < pre[b + 1] <= ps[l + 1]
            if l > f:  # split: one partial slot per (sequence, part), unique, < 2P
                for p in range(f, l + 1):
                    s = 2 * p + (1 if (p == f and pre[b] > ps[p]) else 0)
                    assert s not in slots and s < 2 * P
                    slots.add(s)
        else:
            assert f == l and 0 <= f < P
            if pre[b] < T:
                assert f == _part_of(ps, pre[b])
            else:
                assert f == P - 1


# ------------------------------------------------------ the pages' numbers
def test_byte_arithmetic_of_the_pages():
    g = json.load(open(os.path.join(HERE, "golden", "page_numbers.json")))
    per_tok_elems = g["mla_latent_dims"] + g["mla_rope_dims"]
    assert per_tok_elems == wl.D_K
    assert per_tok_elems * 1 == g["mla_bytes_per_token_layer_fp8"]
    mla = per_tok_elems * g["layers"]
    assert abs(mla - g["mla_stack_bytes_per_token_approx"]) / g["mla_stack_bytes_per_token_approx"] < 0.05
    gqa = g["gqa_kv_heads"] * g["gqa_head_dim"] * 2 * 2
    assert gqa == g["gqa_bytes_per_token_layer_fp16"]
    assert abs(gqa * g["layers"] - g["gqa_stack_bytes_per_token_approx"]) / g["gqa_stack_bytes_per_token_approx"] < 0.05
    assert round(gqa / per_tok_elems) == g["ratio_approx"]
    assert gqa * g["gqa_context_tokens"] == g["gqa_bytes_per_layer_128k_fp16"]
    # the workload's per-token byte count at bf16 is 2 x the page's fp8 figure
    w = wl.make_workload("t", 1, 1, 1, [64], seed=1)
    kv_bytes = wl.config_flops_bytes(w)[0] - (576 * 2 + 512 * 2 + 4) - 4 - 4
    assert kv_bytes == 64 * 2 * g["mla_bytes_per_token_layer_fp8"]
