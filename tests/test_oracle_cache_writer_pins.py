"""Pins of the oracle's cache writers (CPU only): the binary16 encoder, the
q8_0 quantiser and the paged append, checked against IEEE facts, closed-form
cases, numpy's own float16 rounding and invariants of the paging."""
import numpy as np
import pytest

import oracle
import workload as wl


def test_fp16_encoder_round_trips_every_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16).astype(np.float32)
    for b, v in zip(bits, vals):
        if np.isnan(v):
            continue
        assert oracle.fp16_bits(float(v)) == int(b), hex(int(b))


def test_fp16_encoder_ties_and_overflow():
    # midpoint of 1 and its successor 1 + 2^-10 rounds to the even one (1)
    assert oracle.fp16_bits(1.0 + 2.0 ** -11) == 0x3C00
    # midpoint of 1 + 2^-10 and 1 + 2^-9 rounds up to the even one
    assert oracle.fp16_bits(1.0 + 3 * 2.0 ** -11) == 0x3C02
    assert oracle.fp16_bits(65504.0) == 0x7BFF
    assert oracle.fp16_bits(65519.99) == 0x7BFF
    assert oracle.fp16_bits(65520.0) == 0x7C00
    assert oracle.fp16_bits(-1e9) == 0xFC00
    assert oracle.fp16_bits(2.0 ** -24) == 0x0001        # smallest subnormal
    assert oracle.fp16_bits(2.0 ** -25) == 0x0000        # tie between 0 and it: even
    assert oracle.fp16_bits(3 * 2.0 ** -25) == 0x0002    # tie between 1 and 2 units: even
    assert oracle.fp16_bits(-0.0) == 0x8000


def test_fp16_encoder_matches_numpy_rounding():
    x = wl.normal_f32(20000, 5, 3) * np.float32(3.0) ** wl.uniform_int(20000, 5, 4, -12, 12)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    got = np.array([oracle.fp16_bits(float(v)) for v in x], np.uint16)
    assert np.array_equal(got, ref)


def _row(groups):
    x = np.zeros(576, np.float32)
    for g, vals in groups.items():
        x[32 * g:32 * g + len(vals)] = vals
    return x


def test_q8_0_closed_forms():
    # group 0: integers with max |x| = 127 -> scale 1, codes are the values
    ints = np.array([127, -3, 0, 5, -127, 64, 1, -1], np.float32)
    # group 1: scale 1 with exact halves -> rounded away from zero
    halves = np.array([127, 2.5, -2.5, 0.5, -0.5, 1.5, -1.5, 126.5], np.float32)
    # group 2 stays zero: scale 0, codes 0; group 3: max 254 -> scale 2
    twos = np.array([-254, 10, 11, 3], np.float32)
    q, sc = oracle.quantize_q8_0(_row({0: ints, 1: halves, 3: twos}))
    assert sc[0] == 0x3C00 and sc[1] == 0x3C00 and sc[2] == 0 and sc[3] == 0x4000
    assert list(q[:8]) == [127, -3, 0, 5, -127, 64, 1, -1]
    assert list(q[32:40]) == [127, 3, -3, 1, -1, 2, -2, 127]
    assert np.all(q[64:96] == 0)
    assert list(q[96:100]) == [-127, 5, 6, 2]     # 11/2 = 5.5 -> 6, 3/2 = 1.5 -> 2
    assert np.all(q[100:] == 0)


def test_q8_0_error_bound_and_extremes():
    x = wl.normal_f32(576 * 200, 9, 2).reshape(200, 576) * np.float32(1.7)
    q, sc = oracle.quantize_q8_0(x)
    d = np.abs(x.reshape(200, 18, 32)).max(-1) / np.float32(127.0)
    d16 = sc.view(np.float16).astype(np.float64)
    deq = q.reshape(200, 18, 32) * d16[..., None]
    err = np.abs(x.reshape(200, 18, 32) - deq)
    bound = d[..., None] / 2 + 127 * np.abs(d - d16)[..., None] + 1e-6 * np.abs(x).max()
    assert np.all(err <= bound)
    assert np.all(np.abs(q.reshape(200, 18, 32)).max(-1) == 127)
    assert q.min() >= -127


def test_cache_append_bf16_writes_exactly_the_new_rows():
    w = wl.make_workload("app", 3, 2, 16, [130, 2, 64], seed=31, table="permuted")
    kv0 = w.kv.copy()
    new = wl.normal_bf16(3 * 2 * 576, 31, 40).reshape(3, 2, 576)
    kv = w.kv.copy()
    n = oracle.cache_append(new, w.block_table, w.seqlens, kv)
    assert n == 6
    touched = np.zeros(kv.shape[:2], bool)
    for b in range(3):
        for i in range(2):
            t = int(w.seqlens[b]) - 2 + i
            blk = w.block_table[b, t // 64]
            assert np.array_equal(kv[blk, t % 64], new[b, i])
            touched[blk, t % 64] = True
    assert np.array_equal(kv[~touched], kv0[~touched])


def test_cache_append_skips_positions_and_blocks_outside_the_cache():
    w = wl.make_workload("app2", 3, 2, 16, [1, 70, 64], seed=32, table="sequential")
    w.block_table[1, 1] = w.num_blocks + 3       # invalid block for positions 68, 69
    new = wl.normal_bf16(3 * 2 * 576, 32, 40).reshape(3, 2, 576)
    kv = w.kv.copy()
    n = oracle.cache_append(new, w.block_table, w.seqlens, kv)
    # sequence 0: positions -1 (skipped) and 0; sequence 1: both in the bad block
    assert n == 1 + 0 + 2
    assert np.array_equal(kv[w.block_table[0, 0], 0], new[0, 1])


def test_cache_append_q8_0_is_the_quantiser_on_the_new_rows():
    w = wl.make_workload("app3", 2, 1, 16, [100, 64], seed=33, table="permuted", kv_dtype="q8_0")
    new = wl.normal_bf16(2 * 576, 33, 40).reshape(2, 1, 576)
    kv, sc = w.kv.copy(), w.kv_scales.copy()
    assert oracle.cache_append(new, w.block_table, w.seqlens, kv, sc) == 2
    q_ref, s_ref = oracle.quantize_q8_0(wl.bf16_bits_to_f32(new.reshape(2, 576)))
    for b in range(2):
        t = int(w.seqlens[b]) - 1
        blk = w.block_table[b, t // 64]
        assert np.array_equal(kv[blk, t % 64], q_ref[b])
        assert np.array_equal(sc[blk, t % 64], s_ref[b])


# ------------------------------------------------------------ fp8 (E4M3)

def test_fp8_decoder_fixed_points():
    # OCP E4M3: bias 7, 3 fraction bits, subnormals below 2^-6, max 448, one NaN pattern
    assert oracle.fp8_value(0x00) == 0.0
    assert oracle.fp8_value(0x01) == 2.0 ** -9            # smallest subnormal
    assert oracle.fp8_value(0x07) == 7 * 2.0 ** -9        # largest subnormal
    assert oracle.fp8_value(0x08) == 2.0 ** -6            # smallest normal
    assert oracle.fp8_value(0x38) == 1.0
    assert oracle.fp8_value(0x39) == 1.125
    assert oracle.fp8_value(0x7E) == 448.0
    assert oracle.fp8_value(0xFE) == -448.0
    assert oracle.fp8_value(0xC0) == -2.0
    assert np.isnan(oracle.fp8_value(0x7F)) and np.isnan(oracle.fp8_value(0xFF))
    vals = [oracle.fp8_value(b) for b in range(0x7F)]
    assert all(a < b for a, b in zip(vals, vals[1:]))   # codes 0..126 increase


def test_fp8_encoder_round_trips_and_rounds_to_even():
    for b in range(256):
        if b in (0x7F, 0xFF):
            continue
        assert oracle.fp8_bits(oracle.fp8_value(b)) == b, hex(b)
    assert oracle.fp8_bits(1.0625) == 0x38      # halfway 1 .. 1.125 -> even (1)
    assert oracle.fp8_bits(1.1875) == 0x3A      # halfway 1.125 .. 1.25 -> even (1.25)
    assert oracle.fp8_bits(2.0 ** -10) == 0x00  # halfway 0 .. 2^-9 -> even (0)
    assert oracle.fp8_bits(3 * 2.0 ** -10) == 0x02
    assert oracle.fp8_bits(460.0) == 0x7E       # saturates at 448
    assert oracle.fp8_bits(1e30) == 0x7E and oracle.fp8_bits(-1e30) == 0xFE


def test_fp8_writer_matches_the_generators_independent_writer_and_bounds():
    x = wl.normal_f32(576 * 100, 11, 2).reshape(100, 576) * np.float32(3.0)
    x[7] = 0.0
    q, sc = oracle.quantize_fp8(x)
    q2, sc2 = wl.quantize_fp8(x)
    assert np.array_equal(q, q2) and np.array_equal(sc, sc2)
    assert sc[7] == 0 and np.all(q[7] == 0)
    dec = np.array([oracle.fp8_value(b) for b in range(256)])
    xh = dec[q] * sc[:, None]
    # relative spacing of E4M3 normals is 2^-3, so rounding moves a value by at
    # most 2^-4 of itself; subnormals (below 2^-6 d) by at most 2^-10 d
    bound = np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * sc[:, None]) + 1e-12
    assert np.all(np.abs(x - xh) <= bound)
    assert np.all(np.abs(dec[q]).max(1)[sc > 0] == 448.0)   # the largest value maps to +-448


def test_cache_append_fp8_is_the_writer_on_the_new_rows():
    w = wl.make_workload("app4", 2, 1, 16, [100, 64], seed=34, table="permuted", kv_dtype="fp8")
    new = wl.normal_bf16(2 * 576, 34, 40).reshape(2, 1, 576)
    kv, sc = w.kv.copy(), w.kv_scales.copy()
    assert oracle.cache_append(new, w.block_table, w.seqlens, kv, sc) == 2
    q_ref, s_ref = oracle.quantize_fp8(wl.bf16_bits_to_f32(new.reshape(2, 576)))
    for b in range(2):
        t = int(w.seqlens[b]) - 1
        blk = w.block_table[b, t // 64]
        assert np.array_equal(kv[blk, t % 64], q_ref[b]) and sc[blk, t % 64] == s_ref[b]
