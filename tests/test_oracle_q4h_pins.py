"""Pins of the oracle's q4_0 cache in Hadamard rotation (CPU only).

The rotation is checked against the Sylvester construction of the Hadamard
matrix (Kronecker powers of [[1, 1], [1, -1]], built here in numpy, not from
the oracle's sign rule), the cache writer against closed forms (a one-hot
row, blocks whose rotated values are exactly representable) and its error
bound, the reader against an independent numpy dequantisation, and decoding
over such a cache against brute-force softmax attention in numpy.
"""
import math

import numpy as np
import pytest

import oracle
import workload as wl


def _sylvester(n=32):
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.kron(np.array([[1.0, 1.0], [1.0, -1.0]]), h)
    return h


H = _sylvester()
R = H / math.sqrt(32.0)


def _fp16_value(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def _codes(packed):
    """uint8 [..., 288] -> int codes [..., 576] (low nibble first)."""
    p = np.asarray(packed, np.uint8).astype(np.int64)
    return np.stack([p & 0xF, p >> 4], axis=-1).reshape(p.shape[:-1] + (576,))


def _rows(packed, scales):
    """Dequantised rows in double, independently of the oracle: per block
    d * (code - 8), rotated back with the Sylvester matrix."""
    c = _codes(packed)
    d = _fp16_value(scales)
    y = (c - 8) * np.repeat(d, 32, axis=-1)
    yb = y.reshape(y.shape[:-1] + (18, 32))
    return (yb @ R.T).reshape(y.shape)


# ------------------------------------------------------------------ rotation
def test_rotation_is_the_sylvester_hadamard_matrix():
    cols = np.stack([oracle.hadamard32(np.eye(32)[j]) for j in range(32)], axis=1)
    assert np.allclose(cols, R, rtol=0, atol=1e-15)
    # first Walsh function constant, second alternating, sixteenth a step
    assert np.allclose(cols[0] * math.sqrt(32), 1.0)
    assert np.allclose(cols[1] * math.sqrt(32), [(-1) ** j for j in range(32)])
    assert np.allclose(cols[16] * math.sqrt(32), [1] * 16 + [-1] * 16)


def test_rotation_is_orthogonal_and_its_own_inverse():
    x = wl.normal_f64(32 * 40, 7, 1).reshape(40, 32)
    y = oracle.hadamard32(x)
    assert np.allclose(oracle.hadamard32(y), x, rtol=0, atol=1e-13)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)


def test_q4_value_is_scale_times_code_minus_8():
    assert oracle.q4_value(0, 0x3C00) == -8.0
    assert oracle.q4_value(15, 0x3C00) == 7.0
    assert oracle.q4_value(8, 0x7BFF) == 0.0
    assert oracle.q4_value(9, 0x0001) == 2.0 ** -24
    assert oracle.q4_value(3, 0xC000) == 10.0     # -2 * (3 - 8)


# -------------------------------------------------------------------- writer
def test_writer_zero_block_and_one_hot_closed_forms():
    # block 0: x = e_k (k = 5): R e_k = H[:, k] / sqrt(32), all of one
    # magnitude; the first (m = 0, sign +) sets d = -1 / (8 sqrt(32)), so
    # codes are 0 where H[m][k] = +1 and min(15, 16) = 15 where it is -1.
    # block 1 stays zero: d = 0 / -8 = -0 (binary16 0x8000), every code 8.
    k = 5
    x = np.zeros(576, np.float32)
    x[k] = 1.0
    q, sc = oracle.quantize_q4h(x)
    c = _codes(q)
    expect = np.where(H[:, k] > 0, 0, 15)
    assert np.array_equal(c[:32], expect)
    d32 = np.float32(np.float32(1.0) / np.sqrt(np.float32(32.0))) / np.float32(-8.0)
    assert int(sc[0]) == int(np.float16(d32).view(np.uint16))
    assert int(sc[1]) == 0x8000 and np.all(c[32:64] == 8)
    assert np.all(q[16:32] == 0x88)


def test_writer_recovers_exactly_representable_rotated_blocks():
    rng_codes = wl.uniform_int(18 * 32 * 6, 11, 2, 1, 15).reshape(6, 18, 32)
    pos0 = wl.uniform_int(18 * 6, 11, 3, 0, 31).reshape(6, 18)
    for r in range(6):
        for g in range(18):
            rng_codes[r, g, pos0[r, g]] = 0          # unique largest magnitude: -8 d
    expo = wl.uniform_int(18 * 6, 11, 4, -6, 3).reshape(6, 18)
    d = np.ldexp(1.0, expo)                        # powers of two: exact in fp16
    y = (rng_codes - 8) * d[..., None]
    x = (y @ R.T).reshape(6, 576).astype(np.float32)   # R y (R symmetric)
    q, sc = oracle.quantize_q4h(x)
    assert np.array_equal(_codes(q).reshape(6, 18, 32), rng_codes)
    assert np.array_equal(_fp16_value(sc), d)


def test_writer_error_bound_on_gaussian_rows_with_outliers():
    x = wl.normal_f32(576 * 50, 13, 5).reshape(50, 576)
    x[::7, 3] *= 40.0                              # one large value in some blocks
    q, sc = oracle.quantize_q4h(x)
    xh = _rows(q, sc)
    err = (xh - x.astype(np.float64)).reshape(50, 18, 32)
    d32 = np.abs(_fp16_value(sc))                  # |fp16(d)|, d = m / -8
    # rotated error per value <= |d| (rounding 1/2, the clamp at code 15 one
    # step) plus 8 |fp16(d) - d|; the rotation keeps the Euclidean norm
    bound = math.sqrt(32) * (d32 * (1 + 8 * 2.0 ** -11) + 1e-6)
    assert np.all(np.linalg.norm(err, axis=2) <= bound)
    # what the rotation is for: a lone large value no longer sets a scale that
    # flattens the rest of its block. On the blocks holding one, plain q4_0 of
    # the same values (the generator's writer, no rotation) errs more.
    qp, sp = wl.quantize_q4_0(x)
    plain = (_codes(qp) - 8) * np.repeat(_fp16_value(sp), 32, axis=-1)
    err_plain = (plain - x.astype(np.float64)).reshape(50, 18, 32)
    rot = np.linalg.norm(err[::7, 0], axis=1)
    pln = np.linalg.norm(err_plain[::7, 0], axis=1)
    assert rot.mean() < 0.6 * pln.mean()


# -------------------------------------------------------------------- reader
def test_reader_matches_an_independent_dequantisation():
    w = wl.make_workload("t", 2, 1, 4, [70, 33], seed=17, kv_dtype="q4_0h", table="permuted")
    assert np.allclose(oracle.q4h_rows(w.kv, w.kv_scales), _rows(w.kv, w.kv_scales),
                       rtol=0, atol=1e-12)


def test_single_token_decode_returns_the_rotated_back_row():
    # one token whose blocks are all code 8 except code k_g = 9 (value d_g):
    # its cached row is d_g * H[:, k_g] / sqrt(32) per block
    w = wl.make_workload("t", 1, 1, 3, [1], seed=19, kv_dtype="q4_0h")
    kv = np.full_like(w.kv, 0x88)
    sc = np.zeros_like(w.kv_scales)
    phys = int(w.block_table[0, 0])
    expect = np.zeros(576)
    for g in range(18):
        kg = (5 * g + 3) % 32
        byte = 16 * g + kg // 2
        kv[phys, 0, byte] = (9 << 4 | 8) if kg & 1 else (8 << 4 | 9)
        dg = 2.0 ** (g % 5 - 2)
        sc[phys, 0, g] = np.float16(dg).view(np.uint16)
        expect[32 * g:32 * g + 32] = dg * H[:, kg] / math.sqrt(32)
    out, lse = oracle.decode_absorbed(w.q, kv, w.block_table, w.seqlens, w.softmax_scale,
                                      kv_scales=sc)
    qf = wl.bf16_bits_to_f32(w.q).astype(np.float64).reshape(3, 576)
    for h in range(3):
        assert np.allclose(out[0, 0, h], expect[:512], rtol=1e-15, atol=0)
        assert abs(lse[0, 0, h] - w.softmax_scale * float(qf[h] @ expect)) < 1e-12


@pytest.mark.parametrize("seqlens,s_q", [([1, 64, 65, 130], 1), ([40, 3], 2)])
def test_decode_equals_brute_force_softmax_over_the_dequantised_rows(seqlens, s_q):
    B, H = len(seqlens), 4
    w = wl.make_workload("t", B, s_q, H, seqlens, seed=23, kv_dtype="q4_0h", table="permuted")
    out, lse = oracle.decode_absorbed(w.q, w.kv, w.block_table, w.seqlens, w.softmax_scale,
                                      kv_scales=w.kv_scales)
    rows = _rows(w.kv, w.kv_scales)
    qf = wl.bf16_bits_to_f32(w.q).astype(np.float64).reshape(B, s_q, H, 576)
    for b in range(B):
        L = int(w.seqlens[b])
        ids = w.block_table[b, :(L + 63) // 64]
        X = rows[ids].reshape(-1, 576)[:L]
        for i in range(s_q):
            n = L - s_q + 1 + i
            s = w.softmax_scale * (X[:n] @ qf[b, i].T)          # [n, H]
            mx = s.max(axis=0)
            p = np.exp(s - mx)
            ref_lse = mx + np.log(p.sum(axis=0))
            ref = (p / p.sum(axis=0)).T @ X[:n, :512]
            assert np.allclose(out[b, i], ref, rtol=1e-12, atol=1e-12)
            assert np.allclose(lse[b, i], ref_lse, rtol=0, atol=1e-12)


# -------------------------------------------------------------------- append
def test_cache_append_q4h_is_the_writer_on_the_new_rows():
    w = wl.make_workload("t", 3, 2, 1, [5, 64, 130], seed=29, kv_dtype="q4_0h", table="permuted")
    rows = wl.normal_bf16(3 * 2 * 576, 29, 9).reshape(3, 2, 576)
    kv, sc = w.kv.copy(), w.kv_scales.copy()
    n = oracle.cache_append(rows, w.block_table, w.seqlens, kv, sc)
    assert n == 6
    qx, sx = oracle.quantize_q4h(wl.bf16_bits_to_f32(rows))
    touched = np.zeros(kv.shape[:2], bool)
    for b in range(3):
        for i in range(2):
            t = int(w.seqlens[b]) - 2 + i
            blk, slot = int(w.block_table[b, t // 64]), t % 64
            assert np.array_equal(kv[blk, slot], qx[b, i])
            assert np.array_equal(sc[blk, slot], sx[b, i])
            touched[blk, slot] = True
    assert np.array_equal(kv[~touched], w.kv[~touched])
    assert np.array_equal(sc[~touched], w.kv_scales[~touched])


def test_workload_writer_matches_the_oracle_writer_on_rotated_values():
    # the generator quantises values it takes as already rotated; the oracle's
    # writer rotates first: fed R x, the generator must give the oracle's codes
    x = wl.normal_f32(576 * 20, 31, 1).reshape(20, 576)
    qo, so = oracle.quantize_q4h(x)
    xr = oracle.hadamard32(x.astype(np.float64)).astype(np.float32)
    qg, sg = wl.quantize_q4_0(xr)
    # the single-precision transform and the double one round differently, so
    # a value at a code boundary may land one code apart; nothing else differs
    cg, co = _codes(qg), _codes(qo)
    assert np.mean(cg == co) > 0.999 and np.max(np.abs(cg - co)) <= 1
    assert np.max(np.abs(_fp16_value(sg) / _fp16_value(so) - 1)) < 2.0 ** -10


# ---------------------------------------------- read back once, decode as rows
def test_bulk_read_back_equals_the_independent_dequantisation():
    w = wl.make_workload("t", 3, 1, 4, [70, 33, 200], seed=37, kv_dtype="q4_0h", table="permuted")
    rows = oracle.q4h_dequantize(w.kv, w.kv_scales)
    assert rows.shape == w.kv.shape[:2] + (576,)
    assert np.allclose(rows, _rows(w.kv, w.kv_scales), rtol=0, atol=1e-12)


def test_decode_over_fp64_rows_is_the_decode_over_the_cache_they_hold():
    # rows given as doubles: exactly the bf16 decode when they are the bf16
    # values, and the q4_0 decode when they are its read-back rows
    w = wl.make_workload("t", 3, 2, 4, [1, 70, 130], seed=41, table="permuted")
    as_f64 = wl.bf16_bits_to_f32(w.kv).astype(np.float64).reshape(w.kv.shape)
    o0, l0 = oracle.decode_absorbed(w.q, w.kv, w.block_table, w.seqlens, w.softmax_scale)
    o4, l4 = oracle.decode_absorbed(w.q, as_f64, w.block_table, w.seqlens, w.softmax_scale)
    assert np.array_equal(o0, o4) and np.array_equal(l0, l4)
    w = wl.make_workload("t", 3, 2, 4, [1, 70, 130], seed=41, table="permuted", kv_dtype="q4_0h")
    o3, l3 = oracle.decode_absorbed(w.q, w.kv, w.block_table, w.seqlens, w.softmax_scale,
                                    kv_scales=w.kv_scales)
    rows = oracle.q4h_dequantize(w.kv, w.kv_scales)
    o4, l4 = oracle.decode_absorbed(w.q, rows, w.block_table, w.seqlens, w.softmax_scale)
    assert np.array_equal(o3, o4) and np.array_equal(l3, l4)
