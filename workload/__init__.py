"""Seeded synthetic workloads for MLA latent-cache decode.

Shared by the CPU oracle's tests, the GPU parity tests and the benchmark.
Holds no attention arithmetic: it draws random numbers (counter-based
splitmix64 + Box-Muller, in ``gen.c``), rounds them to the storage formats,
lays out a paged cache and its block table, and for the quantized cache runs
the q8_0 cache writer.

Shapes follow the decode step of a DeepSeek-style MLA layer: each cached
token row holds the 512-wide latent c_KV followed by the 64-wide decoupled
RoPE key (576 values), the cache is paged in 64-token blocks, and the query
row per head is already absorbed (576 wide).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

D_LATENT = 512
D_ROPE = 64
D_K = D_LATENT + D_ROPE
BLOCK_TOKENS = 64
Q8_GROUP = 32
Q8_GROUPS = D_K // Q8_GROUP
SOFTMAX_SCALE = 1.0 / math.sqrt(192.0)  # 128 no-RoPE + 64 RoPE dims per head

# stream ids of the generator
S_Q, S_KV, S_SEQLENS, S_PERM, S_OUTLIER, S_WUK, S_WUV, S_QNOPE, S_QROPE = range(1, 10)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmlagen.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile gen.c into libmlagen.so next to it."""
    if force or not os.path.exists(_LIB_PATH):
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
               os.path.join(_HERE, "gen.c"), "-o", _LIB_PATH + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        u64, i64, i32, dbl, vp = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32,
                                  ctypes.c_double, ctypes.c_void_p)
        lib.gen_key.argtypes = [u64, u64]
        lib.gen_key.restype = u64
        lib.gen_raw_at.argtypes = [u64, u64, u64]
        lib.gen_raw_at.restype = u64
        lib.gen_normal_value.argtypes = [u64, u64, u64]
        lib.gen_normal_value.restype = dbl
        lib.gen_f32_to_bf16.argtypes = [ctypes.c_float]
        lib.gen_f32_to_bf16.restype = ctypes.c_uint16
        lib.gen_f32_to_fp16.argtypes = [ctypes.c_float]
        lib.gen_f32_to_fp16.restype = ctypes.c_uint16
        for name in ("gen_normal_bf16", "gen_normal_f32", "gen_normal_f64"):
            getattr(lib, name).argtypes = [vp, i64, u64, u64, i64, dbl]
            getattr(lib, name).restype = None
        lib.gen_uniform_int.argtypes = [vp, i64, u64, u64, i32, i32]
        lib.gen_permutation.argtypes = [vp, i64, u64, u64]
        lib.gen_bernoulli.argtypes = [vp, i64, u64, u64, dbl]
        lib.gen_scale_rows_bf16.argtypes = [vp, i64, i64, vp, ctypes.c_float]
        lib.gen_quantize_q8_0.argtypes = [vp, i64, i32, vp, vp]
        lib.gen_quantize_fp8.argtypes = [vp, i64, i32, vp, vp]
        lib.gen_quantize_q4_0.argtypes = [vp, i64, i32, vp, vp]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


# ---------------------------------------------------------------- primitives
def normal_bf16(n: int, seed: int, stream: int, offset: int = 0, stddev: float = 1.0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    _load().gen_normal_bf16(_ptr(out), n, seed, stream, offset, stddev)
    return out


def normal_f32(n: int, seed: int, stream: int, offset: int = 0, stddev: float = 1.0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    _load().gen_normal_f32(_ptr(out), n, seed, stream, offset, stddev)
    return out


def normal_f64(n: int, seed: int, stream: int, offset: int = 0, stddev: float = 1.0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    _load().gen_normal_f64(_ptr(out), n, seed, stream, offset, stddev)
    return out


def uniform_int(n: int, seed: int, stream: int, lo: int, hi: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    _load().gen_uniform_int(_ptr(out), n, seed, stream, lo, hi)
    return out


def permutation(n: int, seed: int, stream: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    _load().gen_permutation(_ptr(out), n, seed, stream)
    return out


def bernoulli(n: int, seed: int, stream: int, p: float) -> np.ndarray:
    out = np.empty(n, dtype=np.uint8)
    _load().gen_bernoulli(_ptr(out), n, seed, stream, p)
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def quantize_q8_0(x: np.ndarray):
    """q8_0 cache writer on float32 rows of 576 values -> (int8 rows, fp16-bit scales)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows = x.size // D_K
    q = np.empty(x.shape, dtype=np.int8)
    d = np.empty(x.shape[:-1] + (Q8_GROUPS,), dtype=np.uint16)
    _load().gen_quantize_q8_0(_ptr(x), rows, D_K, _ptr(q), _ptr(d))
    return q, d


def quantize_q4_0(x: np.ndarray):
    """q4_0 block writer on float32 rows of 576 -> (uint8 codes [.., 288], fp16-bit
    scales [.., 18]); the values stand for the rotated blocks of a q4_0 cache in
    Hadamard rotation."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows = x.size // D_K
    q = np.empty(x.shape[:-1] + (D_K // 2,), np.uint8)
    d = np.empty(x.shape[:-1] + (Q8_GROUPS,), np.uint16)
    _load().gen_quantize_q4_0(_ptr(x), rows, D_K, _ptr(q), _ptr(d))
    return q, d


def quantize_fp8(x: np.ndarray):
    """fp8 (E4M3) cache writer on float32 rows of 576 -> (uint8 rows, float32 scale per row)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows = x.size // D_K
    q = np.empty(x.shape, dtype=np.uint8)
    d = np.empty(x.shape[:-1], dtype=np.float32)
    _load().gen_quantize_fp8(_ptr(x), rows, D_K, _ptr(q), _ptr(d))
    return q, d


# ------------------------------------------------------------------ workloads
@dataclass
class Workload:
    name: str
    B: int
    s_q: int
    H: int
    seqlens: np.ndarray            # int32 [B]
    block_table: np.ndarray        # int32 [B, max_blocks], -1 = unused slot
    q: np.ndarray                  # uint16 bf16 bits [B, s_q, H, 576]
    kv: np.ndarray                 # uint16 bf16 bits, int8 or uint8 fp8, [num_blocks, 64, 576],
    #                                or uint8 q4_0 codes [num_blocks, 64, 288] (q4_0h)
    kv_scales: Optional[np.ndarray]  # uint16 fp16 bits [num_blocks, 64, 18] (q8_0, q4_0h),
    #                                  float32 [num_blocks, 64] (fp8) or None
    kv_dtype: str                  # "bf16" | "q8_0" | "fp8" | "q4_0h"
    softmax_scale: float = SOFTMAX_SCALE
    seed: int = 0
    recipe: dict = field(default_factory=dict)

    @property
    def num_blocks(self) -> int:
        return int(self.kv.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def rows(self) -> int:
        return self.B * self.s_q * self.H

    @property
    def max_seqlen(self) -> int:
        return int(self.seqlens.max()) if self.B else 0


def make_workload(name: str, B: int, s_q: int, H: int, seqlens, *, seed: int,
                  table: str = "sequential", kv_dtype: str = "bf16",
                  outlier_frac: float = 0.0, outlier_scale: float = 8.0,
                  max_blocks: Optional[int] = None) -> Workload:
    """Build a paged-cache decode workload.

    seqlens: int, sequence of ints, or ("uniform", lo, hi) drawn from the seed.
    table: "sequential" (sequence b owns a contiguous run of physical blocks)
           or "permuted" (a seeded random permutation of the physical pool).
    Rows past a sequence's length in its last block hold random data too;
    they must never reach the result.
    """
    if isinstance(seqlens, tuple) and seqlens and seqlens[0] == "uniform":
        sl = uniform_int(B, seed, S_SEQLENS, int(seqlens[1]), int(seqlens[2]))
    elif np.isscalar(seqlens):
        sl = np.full(B, int(seqlens), dtype=np.int32)
    else:
        sl = np.asarray(seqlens, dtype=np.int32).copy()
        assert sl.shape == (B,)
    nblk = (np.maximum(sl, 0).astype(np.int64) + BLOCK_TOKENS - 1) // BLOCK_TOKENS
    mb = int(max_blocks) if max_blocks is not None else max(1, int(nblk.max()) if B else 1)
    total = int(nblk.sum())
    pool = max(total, 1)
    if table == "sequential":
        phys = np.arange(pool, dtype=np.int32)
    elif table == "permuted":
        phys = permutation(pool, seed, S_PERM)
    else:
        raise ValueError(table)
    bt = np.full((B, mb), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        n = int(nblk[b])
        bt[b, :n] = phys[off:off + n]
        off += n
    q = normal_bf16(B * s_q * H * D_K, seed, S_Q).reshape(B, s_q, H, D_K)
    n_el = pool * BLOCK_TOKENS * D_K
    scales = None
    if kv_dtype == "bf16":
        kv = normal_bf16(n_el, seed, S_KV).reshape(pool, BLOCK_TOKENS, D_K)
        if outlier_frac > 0:
            mask = bernoulli(pool * BLOCK_TOKENS, seed, S_OUTLIER, outlier_frac)
            _load().gen_scale_rows_bf16(_ptr(kv), pool * BLOCK_TOKENS, D_K, _ptr(mask),
                                        float(outlier_scale))
    elif kv_dtype == "q8_0":
        x = normal_f32(n_el, seed, S_KV).reshape(pool, BLOCK_TOKENS, D_K)
        kv, scales = quantize_q8_0(x)
        del x
    elif kv_dtype == "fp8":
        x = normal_f32(n_el, seed, S_KV).reshape(pool, BLOCK_TOKENS, D_K)
        kv, scales = quantize_fp8(x)
        del x
    elif kv_dtype == "q4_0h":
        # the rotated blocks of N(0,1) rows are N(0,1) values (see gen.c)
        x = normal_f32(n_el, seed, S_KV).reshape(pool, BLOCK_TOKENS, D_K)
        kv, scales = quantize_q4_0(x)
        del x
    else:
        raise ValueError(kv_dtype)
    recipe = dict(seed=seed, table=table, kv_dtype=kv_dtype, outlier_frac=outlier_frac,
                  outlier_scale=outlier_scale, distribution="N(0,1)")
    return Workload(name=name, B=B, s_q=s_q, H=H, seqlens=sl, block_table=bt, q=q, kv=kv,
                    kv_scales=scales, kv_dtype=kv_dtype, seed=seed, recipe=recipe)


# The five decode workloads: tiny; DeepSeek-V3 shaped 128 heads x 4K; ragged
# paged 16 heads; 128K long context with a causal pair of query tokens; q8_0
# latent cache at 8K. Seed = 1000 + index.
CONFIGS = {
    1: dict(name="tiny_b1_h16_l256", B=1, s_q=1, H=16, seqlens=256, table="sequential"),
    2: dict(name="dsv3_b64_h128_l4096", B=64, s_q=1, H=128, seqlens=4096, table="sequential"),
    3: dict(name="ragged_b128_h16_l1-8192", B=128, s_q=1, H=16, seqlens=("uniform", 1, 8192),
            table="permuted", max_blocks=128),
    4: dict(name="long_b4_sq2_h128_l131072", B=4, s_q=2, H=128, seqlens=131072,
            table="sequential", outlier_frac=0.01, outlier_scale=8.0),
    5: dict(name="q8_b64_h128_l8192", B=64, s_q=1, H=128, seqlens=8192, table="sequential",
            kv_dtype="q8_0"),
    # the DeepSeek-V3 shape over an fp8 (E4M3, per-token fp32 scale) cache
    6: dict(name="fp8_b64_h128_l4096", B=64, s_q=1, H=128, seqlens=4096, table="sequential",
            kv_dtype="fp8"),
    # the q8_0 workload's shape over a q4_0 cache stored in Hadamard rotation
    7: dict(name="q4h_b64_h128_l8192", B=64, s_q=1, H=128, seqlens=8192, table="sequential",
            kv_dtype="q4_0h"),
}


def config_workload(idx: int, **overrides) -> Workload:
    spec = dict(CONFIGS[idx])
    spec.update(overrides)
    name = spec.pop("name")
    return make_workload(name, seed=1000 + idx, **spec)


def config_flops_bytes(w: Workload):
    """Algorithmic work of one decode call: (bytes, flops, visible_token_rows).

    Bytes: every cached token row that some query can see, read once per
    sequence (1152 B bf16, 576 + 36 B q8_0, 576 + 4 B fp8 or 288 + 36 B q4_0h), plus q,
    out (bf16) and lse
    (fp32) per query row, plus the block-table entries and seqlens read.
    Flops: 2*576 (scores) + 2*512 (value product) per visible (token, row).
    """
    per_tok = {"bf16": D_K * 2, "q8_0": D_K + Q8_GROUPS * 2, "fp8": D_K + 4,
               "q4_0h": D_K // 2 + Q8_GROUPS * 2}[w.kv_dtype]
    L = np.clip(w.seqlens.astype(np.int64), 0, w.max_blocks * BLOCK_TOKENS)
    kv_bytes = int(L.sum()) * per_tok
    nblk = (L + BLOCK_TOKENS - 1) // BLOCK_TOKENS
    rows = w.rows
    qob = rows * (D_K * 2 + D_LATENT * 2 + 4)
    meta = int(nblk.sum()) * 4 + w.B * 4
    vis = 0
    for i in range(w.s_q):
        vis += int(np.maximum(L - w.s_q + 1 + i, 0).sum()) * w.H
    flops = vis * (2 * D_K + 2 * D_LATENT)
    return kv_bytes + qob + meta, flops, vis
