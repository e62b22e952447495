"""CPU oracle for MLA latent-cache decode -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package. The GPU library
(``mla_latent_kv_10_amd``) never imports it and shares no code with it.

Thin ctypes wrapper over ``mla_oracle.c`` (plain fp64 C, see that file for the
definitions and the passages of the pages each one follows). Arrays are numpy;
bf16 / fp16 values travel as their uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmlaoracle.so")
_lib = None

D_LATENT, D_ROPE, D_K, BLOCK_TOKENS = 512, 64, 576, 64
D_HEAD = 128


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB_PATH):
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
               os.path.join(_HERE, "mla_oracle.c"), "-o", _LIB_PATH + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        i32, i64, dbl, vp, u16 = (ctypes.c_int32, ctypes.c_int64, ctypes.c_double,
                                  ctypes.c_void_p, ctypes.c_uint16)
        lib.oracle_bf16_value.argtypes = [u16]
        lib.oracle_bf16_value.restype = dbl
        lib.oracle_fp16_value.argtypes = [u16]
        lib.oracle_fp16_value.restype = dbl
        lib.oracle_q8_value.argtypes = [ctypes.c_int8, u16]
        lib.oracle_q8_value.restype = dbl
        lib.oracle_decode_absorbed.argtypes = [i32, i32, i32, vp, i32, vp, vp, i64, vp, i32, vp,
                                               dbl, vp, i64, vp, vp]
        lib.oracle_decode_absorbed.restype = ctypes.c_int
        lib.oracle_decode_absorbed_abs.argtypes = [i32, i32, i32, vp, i32, vp, vp, i64, vp, i32,
                                                   vp, dbl, vp, i64, vp, vp, vp]
        lib.oracle_decode_absorbed_abs.restype = ctypes.c_int
        lib.oracle_decode_absorbed_f64q.argtypes = [i32, i32, i32, vp, i32, vp, vp, i64, vp, i32,
                                                    vp, dbl, vp, vp]
        lib.oracle_decode_absorbed_f64q.restype = ctypes.c_int
        lib.oracle_decode_decompressed.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, i64, vp,
                                                   i32, vp, dbl, vp, vp]
        lib.oracle_decode_decompressed.restype = ctypes.c_int
        lib.oracle_absorb_query.argtypes = [i64, i32, vp, vp, vp, vp]
        lib.oracle_absorb_query.restype = None
        lib.oracle_project_output.argtypes = [i64, i32, vp, vp, vp]
        lib.oracle_project_output.restype = None
        lib.oracle_combine.argtypes = [i32, i64, vp, vp, vp, vp]
        lib.oracle_combine.restype = None
        lib.oracle_plan.argtypes = [i32, vp, i32, i32, vp, vp, vp, vp]
        lib.oracle_plan.restype = ctypes.c_int
        lib.oracle_fp8_value.argtypes = [ctypes.c_uint8]
        lib.oracle_fp8_value.restype = dbl
        lib.oracle_fp8_bits.argtypes = [ctypes.c_float]
        lib.oracle_fp8_bits.restype = ctypes.c_uint8
        lib.oracle_quantize_fp8_row.argtypes = [vp, vp, vp]
        lib.oracle_quantize_fp8_row.restype = None
        lib.oracle_fp16_bits.argtypes = [ctypes.c_float]
        lib.oracle_fp16_bits.restype = u16
        lib.oracle_quantize_q8_0_row.argtypes = [vp, vp, vp]
        lib.oracle_quantize_q8_0_row.restype = None
        lib.oracle_cache_append.argtypes = [i32, i32, i32, vp, vp, i32, vp, i64, vp, vp]
        lib.oracle_hadamard32.argtypes = [vp, vp]
        lib.oracle_hadamard32.restype = None
        lib.oracle_q4_value.argtypes = [ctypes.c_int, u16]
        lib.oracle_q4_value.restype = dbl
        lib.oracle_quantize_q4h_row.argtypes = [vp, vp, vp]
        lib.oracle_quantize_q4h_row.restype = None
        lib.oracle_q4h_dequantize.argtypes = [i64, vp, vp, vp]
        lib.oracle_q4h_dequantize.restype = None
        lib.oracle_cache_append.restype = i64
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_threads.restype = None
        _lib = lib
    return _lib


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


Q4_ROW_BYTES = D_K // 2


def _kind(kv) -> int:
    """Cache type from the array: bf16 bits (uint16), q8_0 (int8), fp8 (uint8
    rows of 576), q4_0 in Hadamard rotation (uint8 rows of 288 code bytes) or
    the rows themselves (float64)."""
    if kv.dtype == np.uint8 and kv.shape[-1] == Q4_ROW_BYTES:
        return 3
    return {np.dtype(np.uint16): 0, np.dtype(np.int8): 1, np.dtype(np.uint8): 2,
            np.dtype(np.float64): 4}[kv.dtype]


def _p(a):
    return None if a is None else a.ctypes.data


def max_threads() -> int:
    """Host threads the oracle's parallel loops use."""
    return int(_load().oracle_max_threads())


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def bf16_value(bits: int) -> float:
    return _load().oracle_bf16_value(bits)


def fp16_value(bits: int) -> float:
    return _load().oracle_fp16_value(bits)


def q8_value(q: int, scale_bits: int) -> float:
    return _load().oracle_q8_value(q, scale_bits)


def fp8_value(bits: int) -> float:
    """OCP E4M3 byte -> its value (exact)."""
    return _load().oracle_fp8_value(bits)


def fp8_bits(x: float) -> int:
    """float32 -> OCP E4M3 byte, nearest even, saturated to +-448."""
    return int(_load().oracle_fp8_bits(float(np.float32(x))))


def quantize_fp8(x):
    """fp8 cache writer on float32 rows of 576 -> (uint8 codes, float32 scale per row)."""
    x = _c(x, np.float32)
    rows = x.size // D_K
    flat = x.reshape(rows, D_K)
    q = np.empty((rows, D_K), np.uint8)
    sc = np.empty(rows, np.float32)
    for r in range(rows):
        _load().oracle_quantize_fp8_row(_p(flat[r]), _p(q[r]), sc[r:].ctypes.data)
    return q.reshape(x.shape), sc.reshape(x.shape[:-1])


def decode_absorbed(q, kv, block_table, seqlens, softmax_scale, *, kv_scales=None, rows=None,
                    with_abs=False):
    """Absorbed-form decode (fp64). q: uint16 [B, s_q, H, 576] bf16 bits.

    kv: uint16 bf16 bits, int8 (with kv_scales uint16 fp16 bits [nb, 64, 18]),
    uint8 fp8 E4M3 (with kv_scales float32 [nb, 64]), uint8 q4_0 codes
    [nb, 64, 288] in Hadamard rotation (with kv_scales uint16 fp16 bits [nb, 64, 18])
    or float64 rows [nb, 64, 576] (no scales).
    rows: optional int64 row ids r = (b * s_q + i) * H + h.
    Returns (out float64 [n, 512], lse float64 [n]); all rows -> shaped [B, s_q, H, ...].
    with_abs: also return out_abs = sum_t p_t |row_t| (same shape as out).
    """
    q = _c(q, np.uint16)
    B, s_q, H, dk = q.shape
    assert dk == D_K
    kind = _kind(kv)
    kv = _c(kv, kv.dtype)
    sc = None if kind in (0, 4) else _c(kv_scales, np.float32 if kind == 2 else np.uint16)
    bt = _c(block_table, np.int32)
    sl = _c(seqlens, np.int32)
    rr = None if rows is None else _c(rows, np.int64)
    n = B * s_q * H if rr is None else rr.size
    out = np.empty((n, D_LATENT), np.float64)
    lse = np.empty(n, np.float64)
    if with_abs:
        oabs = np.empty((n, D_LATENT), np.float64)
        rc = _load().oracle_decode_absorbed_abs(B, s_q, H, _p(q), kind, _p(kv), _p(sc),
                                                kv.shape[0], _p(bt), bt.shape[1], _p(sl),
                                                float(softmax_scale), _p(rr), n, _p(out),
                                                _p(lse), _p(oabs))
    else:
        rc = _load().oracle_decode_absorbed(B, s_q, H, _p(q), kind, _p(kv), _p(sc), kv.shape[0],
                                            _p(bt), bt.shape[1], _p(sl), float(softmax_scale),
                                            _p(rr), n, _p(out), _p(lse))
    if rc != 0:
        raise ValueError("row id out of range")
    if rr is None:
        res = (out.reshape(B, s_q, H, D_LATENT), lse.reshape(B, s_q, H))
        if with_abs:
            res = res + (oabs.reshape(B, s_q, H, D_LATENT),)
        return res
    return (out, lse, oabs) if with_abs else (out, lse)


def decode_absorbed_f64q(q, kv, block_table, seqlens, softmax_scale):
    q = _c(q, np.float64)
    B, s_q, H, dk = q.shape
    kv = _c(kv, np.uint16)
    bt = _c(block_table, np.int32)
    sl = _c(seqlens, np.int32)
    out = np.empty((B, s_q, H, D_LATENT), np.float64)
    lse = np.empty((B, s_q, H), np.float64)
    _load().oracle_decode_absorbed_f64q(B, s_q, H, _p(q), 0, _p(kv), None, kv.shape[0], _p(bt),
                                        bt.shape[1], _p(sl), float(softmax_scale), _p(out),
                                        _p(lse))
    return out, lse


def decode_decompressed(q_nope, q_rope, w_uk, w_uv, kv, block_table, seqlens, softmax_scale):
    q_nope = _c(q_nope, np.float64)
    q_rope = _c(q_rope, np.float64)
    B, s_q, H, _ = q_nope.shape
    w_uk = _c(w_uk, np.float64)
    w_uv = _c(w_uv, np.float64)
    assert w_uk.shape == (H, D_HEAD, D_LATENT) and w_uv.shape == (H, D_HEAD, D_LATENT)
    kv = _c(kv, np.uint16)
    bt = _c(block_table, np.int32)
    sl = _c(seqlens, np.int32)
    out = np.empty((B, s_q, H, D_HEAD), np.float64)
    lse = np.empty((B, s_q, H), np.float64)
    _load().oracle_decode_decompressed(B, s_q, H, _p(q_nope), _p(q_rope), _p(w_uk), _p(w_uv),
                                       _p(kv), kv.shape[0], _p(bt), bt.shape[1], _p(sl),
                                       float(softmax_scale), _p(out), _p(lse))
    return out, lse


def absorb_query(q_nope, q_rope, w_uk):
    q_nope = _c(q_nope, np.float64)
    q_rope = _c(q_rope, np.float64)
    H = q_nope.shape[-2]
    rows = q_nope.size // D_HEAD
    out = np.empty(q_nope.shape[:-1] + (D_K,), np.float64)
    _load().oracle_absorb_query(rows, H, _p(q_nope), _p(q_rope), _p(_c(w_uk, np.float64)),
                                _p(out))
    return out


def project_output(o_lat, w_uv):
    o_lat = _c(o_lat, np.float64)
    H = o_lat.shape[-2]
    rows = o_lat.size // D_LATENT
    out = np.empty(o_lat.shape[:-1] + (D_HEAD,), np.float64)
    _load().oracle_project_output(rows, H, _p(o_lat), _p(_c(w_uv, np.float64)), _p(out))
    return out


def fp16_bits(x: float) -> int:
    """IEEE binary16 bits of float32 x, round to nearest even."""
    return int(_load().oracle_fp16_bits(float(np.float32(x))))


def quantize_q8_0(x):
    """q8_0 cache writer on float32 rows of 576 -> (int8 codes, fp16 scale bits [.., 18])."""
    x = _c(x, np.float32)
    rows = x.size // D_K
    flat = x.reshape(rows, D_K)
    q = np.empty((rows, D_K), np.int8)
    sc = np.empty((rows, D_K // 32), np.uint16)
    for r in range(rows):
        _load().oracle_quantize_q8_0_row(_p(flat[r]), _p(q[r]), _p(sc[r]))
    return q.reshape(x.shape), sc.reshape(x.shape[:-1] + (D_K // 32,))


def cache_append(rows, block_table, seqlens, kv, kv_scales=None):
    """Write the new rows (bf16 bits [B, s_q, 576]) into the paged cache kv
    (bf16 bits or int8 with kv_scales), in place. Returns rows written."""
    rows = _c(rows, np.uint16)
    B, s_q, dk = rows.shape
    assert dk == D_K and kv.flags["C_CONTIGUOUS"]
    kind = _kind(kv)
    if kind:
        assert kv_scales is not None and kv_scales.flags["C_CONTIGUOUS"]
    bt = _c(block_table, np.int32)
    sl = _c(seqlens, np.int32)
    return int(_load().oracle_cache_append(B, s_q, kind, _p(rows), _p(bt), bt.shape[1], _p(sl),
                                           kv.shape[0], _p(kv), _p(kv_scales)))


def hadamard32(x):
    """y = R x per 32-value block (R = H / sqrt(32), H the Sylvester-Hadamard
    matrix), in double, from the matrix entries. x: float64 [..., 32k]."""
    x = _c(x, np.float64)
    flat = x.reshape(-1, 32)
    y = np.empty_like(flat)
    for i in range(flat.shape[0]):
        _load().oracle_hadamard32(_p(flat[i]), y[i:].ctypes.data)
    return y.reshape(x.shape)


def q4_value(code: int, scale_bits: int) -> float:
    return float(_load().oracle_q4_value(int(code), int(scale_bits)))


def quantize_q4h(x):
    """Rotating q4_0 cache writer on float32 rows of 576 -> (uint8 codes [.., 288],
    fp16 scale bits [.., 18])."""
    x = _c(x, np.float32)
    rows = x.size // D_K
    flat = x.reshape(rows, D_K)
    q = np.empty((rows, Q4_ROW_BYTES), np.uint8)
    sc = np.empty((rows, D_K // 32), np.uint16)
    for r in range(rows):
        _load().oracle_quantize_q4h_row(_p(flat[r]), _p(q[r]), _p(sc[r]))
    return q.reshape(x.shape[:-1] + (Q4_ROW_BYTES,)), sc.reshape(x.shape[:-1] + (D_K // 32,))


def q4h_dequantize(codes, scales):
    """The whole q4_0-in-rotation cache read back once, in C (parallel over
    rows): codes uint8 [..., 288], scales uint16 fp16 bits [..., 18] ->
    float64 [..., 576], for decode_absorbed over large workloads."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint16)
    rows = codes.size // Q4_ROW_BYTES
    out = np.empty(codes.shape[:-1] + (D_K,), np.float64)
    _load().oracle_q4h_dequantize(rows, _p(codes), _p(scales), _p(out))
    return out


def q4h_rows(codes, scales):
    """The cached rows a q4_0-in-rotation cache stands for, in double: per block
    the stored values scale * (code - 8), rotated back by R. codes uint8
    [..., 288], scales uint16 fp16 bits [..., 18] -> float64 [..., 576]."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint16)
    lo = (codes & 0xF).astype(np.int64)
    hi = (codes >> 4).astype(np.int64)
    c = np.stack([lo, hi], axis=-1).reshape(codes.shape[:-1] + (D_K,))
    d = np.vectorize(fp16_value)(scales.astype(np.int64))
    y = d.repeat(32, axis=-1) * (c - 8)
    return hadamard32(y)


def combine(part_out, part_lse):
    """part_out float32 [S, R, 512], part_lse float32 [S, R] -> (out f64 [R,512], lse f64 [R])."""
    po = _c(part_out, np.float32)
    pl = _c(part_lse, np.float32)
    S, R = pl.shape
    assert po.shape == (S, R, D_LATENT)
    out = np.empty((R, D_LATENT), np.float64)
    lse = np.empty(R, np.float64)
    _load().oracle_combine(S, R, _p(po), _p(pl), _p(out), _p(lse))
    return out, lse


def plan(seqlens, max_blocks: int, P: int):
    """The library's split partition -> dict of int32 arrays."""
    sl = _c(seqlens, np.int32)
    B = sl.size
    pre = np.empty(B + 1, np.int32)
    ps = np.empty(P + 1, np.int32)
    fp = np.empty(B, np.int32)
    lp = np.empty(B, np.int32)
    rc = _load().oracle_plan(B, _p(sl), int(max_blocks), int(P), _p(pre), _p(ps), _p(fp), _p(lp))
    if rc != 0:
        raise ValueError("bad plan arguments")
    return dict(seq_prefix=pre, part_start=ps, seq_first_part=fp, seq_last_part=lp)
