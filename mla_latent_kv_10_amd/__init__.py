"""Python binding of libmla (MLA latent-cache decode on MI355X / gfx950).

Argument marshalling only: every step of the decode runs in the HIP kernels
of ``libmla.so`` (built from ``csrc/libmla.hip``; the C ABI is
``include/mla.h``). PyTorch provides device memory and the current stream.
If the shared library is missing the import of this module still works, but
every call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

from ._build import LIB_PATH, build  # noqa: F401

D_LATENT, D_ROPE, D_K, BLOCK_TOKENS = 512, 64, 576, 64
KV_BF16, KV_Q8_0, KV_FP8, KV_Q4_0H = 0, 1, 2, 3
MAX_BATCH, MAX_ROWS = 2048, 4096

STATUS = {0: "MLA_OK", 1: "MLA_ERR_INVALID_ARG", 2: "MLA_ERR_UNSUPPORTED",
          3: "MLA_ERR_WORKSPACE_TOO_SMALL", 4: "MLA_ERR_HIP"}

# Entry points declared in include/mla.h
EXPORTS = ("mla_workspace_size", "mla_num_parts", "mla_decode", "mla_decode_noalloc",
           "mla_combine", "mla_plan", "mla_absorb_query", "mla_project_output",
           "mla_cache_append", "mla_status_str", "mla_last_error")
D_HEAD = 128
NOALLOC_SCRATCH_BYTES = 72 << 20


class MlaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seqlen_q", ctypes.c_int32),
                ("num_heads", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("num_blocks", ctypes.c_int64), ("max_seqlen", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("num_parts", ctypes.c_int32),
                ("m_tile", ctypes.c_int32)]


_lib = None


def lib():
    """Load libmla.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libmla is not built ({LIB_PATH} missing): run "
                               "mla_latent_kv_10_amd.build() or __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        pp = ctypes.POINTER(Problem)
        L.mla_workspace_size.argtypes = [pp, ctypes.POINTER(ctypes.c_size_t)]
        L.mla_num_parts.argtypes = [pp, ctypes.POINTER(i32)]
        L.mla_decode.argtypes = [pp, vp, vp, vp, vp, vp, f32, vp, vp, vp, ctypes.c_size_t, vp]
        L.mla_decode_noalloc.argtypes = [pp, vp, vp, vp, vp, vp, f32, vp, vp, vp]
        L.mla_combine.argtypes = [i32, i64, vp, vp, vp, vp, vp]
        L.mla_plan.argtypes = [pp, vp, vp, i64, vp]
        L.mla_absorb_query.argtypes = [i64, i32, vp, vp, vp, vp, vp]
        L.mla_project_output.argtypes = [i64, i32, vp, vp, vp, vp]
        L.mla_cache_append.argtypes = [i32, i32, vp, vp, i32, vp, i64, i32, vp, vp, vp]
        for name in ("mla_workspace_size", "mla_num_parts", "mla_decode", "mla_decode_noalloc",
                     "mla_combine", "mla_plan", "mla_absorb_query", "mla_project_output",
                     "mla_cache_append"):
            getattr(L, name).restype = ctypes.c_int
        L.mla_status_str.argtypes = [ctypes.c_int]
        L.mla_status_str.restype = ctypes.c_char_p
        L.mla_last_error.argtypes = []
        L.mla_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise MlaError(status, lib().mla_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def make_problem(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor, *,
                 kv_dtype: int, max_seqlen: int = 0, num_parts: int = 0,
                 m_tile: int = 0) -> Problem:
    B, s_q, H, dk = q.shape
    return Problem(batch=B, seqlen_q=s_q, num_heads=H, max_blocks_per_seq=block_table.shape[1],
                   num_blocks=kv_cache.shape[0], max_seqlen=int(max_seqlen), kv_dtype=kv_dtype,
                   num_parts=int(num_parts), m_tile=int(m_tile))


def workspace_size(problem: Problem) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().mla_workspace_size(ctypes.byref(problem), ctypes.byref(n)))
    return n.value


def problem_num_parts(problem: Problem) -> int:
    n = ctypes.c_int32(0)
    _check(lib().mla_num_parts(ctypes.byref(problem), ctypes.byref(n)))
    return n.value


def _require(t: torch.Tensor, name: str, dtype, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _cache_kind(kv_cache: torch.Tensor) -> int:
    """bf16 -> KV_BF16, int8 -> KV_Q8_0, uint8 rows of 576 -> KV_FP8 (E4M3 bytes),
    uint8 rows of 288 -> KV_Q4_0H (q4_0 codes in Hadamard rotation)."""
    kinds = {torch.bfloat16: KV_BF16, torch.int8: KV_Q8_0, torch.uint8: KV_FP8}
    if not isinstance(kv_cache, torch.Tensor) or kv_cache.dtype not in kinds:
        raise TypeError("kv_cache must be a bfloat16, int8 (q8_0) or uint8 (fp8 E4M3 or "
                        "q4_0 codes) tensor")
    _require(kv_cache, "kv_cache", kv_cache.dtype, 3)
    if kv_cache.dtype == torch.uint8 and kv_cache.shape[-1] == D_K // 2:
        return KV_Q4_0H
    return kinds[kv_cache.dtype]


def _check_cache_shape(kind: int, kv_cache: torch.Tensor):
    width = D_K // 2 if kind == KV_Q4_0H else D_K
    if tuple(kv_cache.shape[1:]) != (BLOCK_TOKENS, width):
        raise ValueError(f"kv_cache must be [num_blocks, 64, {width}]")


def _check_scales(kind: int, kv_cache: torch.Tensor, kv_scales):
    if kind == KV_BF16:
        return
    if kv_scales is None:
        raise ValueError("kv_scales is required for a quantised (q8_0, fp8 or q4_0) cache")
    if kind in (KV_Q8_0, KV_Q4_0H):
        _require(kv_scales, "kv_scales", torch.float16, 3)
        if tuple(kv_scales.shape) != (kv_cache.shape[0], BLOCK_TOKENS, D_K // 32):
            raise ValueError("kv_scales must be [num_blocks, 64, 18]")
    else:
        _require(kv_scales, "kv_scales", torch.float32, 2)
        if tuple(kv_scales.shape) != (kv_cache.shape[0], BLOCK_TOKENS):
            raise ValueError("kv_scales must be [num_blocks, 64] (fp32, one per token)")


def _decode_args(q, kv_cache, block_table, seqlens, out, lse, kv_scales, workspace,
                 max_seqlen, num_parts, m_tile):
    """Check the decode arguments -> (problem, out, lse, device)."""
    _require(q, "q", torch.bfloat16, 4)
    if q.shape[-1] != D_K:
        raise ValueError("q rows must be 576 wide")
    kind = _cache_kind(kv_cache)
    _check_cache_shape(kind, kv_cache)
    _check_scales(kind, kv_cache, kv_scales)
    _require(block_table, "block_table", torch.int32, 2)
    _require(seqlens, "seqlens", torch.int32, 1)
    B, s_q, H, _ = q.shape
    if block_table.shape[0] != B or seqlens.shape[0] != B:
        raise ValueError("block_table and seqlens must have B rows")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("libmla runs on the GPU only: q must be a device tensor")
    for name, t in (("kv_cache", kv_cache), ("block_table", block_table), ("seqlens", seqlens),
                    ("kv_scales", kv_scales), ("out", out), ("lse", lse),
                    ("workspace", workspace)):
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, q on {dev}")
    if out is None:
        out = torch.empty((B, s_q, H, D_LATENT), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, s_q, H), dtype=torch.float32, device=dev)
    _require(out, "out", torch.bfloat16, 4)
    _require(lse, "lse", torch.float32, 3)
    if tuple(out.shape) != (B, s_q, H, D_LATENT) or tuple(lse.shape) != (B, s_q, H):
        raise ValueError("out must be [B, s_q, H, 512] and lse [B, s_q, H]")
    prob = make_problem(q, kv_cache, block_table, kv_dtype=kind,
                        max_seqlen=max_seqlen, num_parts=num_parts, m_tile=m_tile)
    return prob, out, lse, dev


def mla_decode(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
               seqlens: torch.Tensor, softmax_scale: float,
               out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, *,
               kv_scales: Optional[torch.Tensor] = None, max_seqlen: int = 0,
               num_parts: int = 0, m_tile: int = 0,
               workspace: Optional[torch.Tensor] = None):
    """Decode step over a paged latent cache (see include/mla.h).

    q bf16 [B, s_q, H, 576]; kv_cache bf16 [nb, 64, 576], int8 (q8_0, with
    kv_scales float16 [nb, 64, 18]), uint8 (fp8 E4M3, with kv_scales
    float32 [nb, 64]) or uint8 [nb, 64, 288] (q4_0 codes in Hadamard rotation,
    with kv_scales float16 [nb, 64, 18]); block_table int32 [B, max_blocks];
    seqlens int32 [B] (device). Returns (out bf16 [B, s_q, H, 512],
    lse float32 [B, s_q, H]). Runs on the current stream; never synchronises.
    """
    prob, out, lse, dev = _decode_args(q, kv_cache, block_table, seqlens, out, lse, kv_scales,
                                       workspace, max_seqlen, num_parts, m_tile)
    with torch.cuda.device(dev):
        ws_bytes = workspace_size(prob)
        if workspace is None:
            workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
        _check(lib().mla_decode(ctypes.byref(prob), _ptr(q), _ptr(kv_cache), _ptr(kv_scales),
                                _ptr(block_table), _ptr(seqlens), float(softmax_scale),
                                _ptr(out), _ptr(lse), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(dev)))
    return out, lse


def mla_decode_noalloc(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
                       seqlens: torch.Tensor, softmax_scale: float,
                       out: torch.Tensor, lse: torch.Tensor, *,
                       kv_scales: Optional[torch.Tensor] = None, max_seqlen: int = 0,
                       num_parts: int = 0, m_tile: int = 0):
    """mla_decode on the library's own per-device workspace (no workspace
    argument, no allocation by the library): the caller passes out and lse.
    Calls that overlap on one device race (include/mla.h)."""
    prob, out, lse, dev = _decode_args(q, kv_cache, block_table, seqlens, out, lse, kv_scales,
                                       None, max_seqlen, num_parts, m_tile)
    with torch.cuda.device(dev):
        _check(lib().mla_decode_noalloc(ctypes.byref(prob), _ptr(q), _ptr(kv_cache),
                                        _ptr(kv_scales), _ptr(block_table), _ptr(seqlens),
                                        float(softmax_scale), _ptr(out), _ptr(lse),
                                        _stream(dev)))
    return out, lse


def mla_combine(partial_out: torch.Tensor, partial_lse: torch.Tensor,
                out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """LSE merge of partial results: partial_out float32 [S, R, 512],
    partial_lse float32 [S, R] -> (out bf16 [R, 512], lse float32 [R])."""
    _require(partial_out, "partial_out", torch.float32, 3)
    _require(partial_lse, "partial_lse", torch.float32, 2)
    S, R, dl = partial_out.shape
    if dl != D_LATENT or tuple(partial_lse.shape) != (S, R):
        raise ValueError("partial_out must be [S, R, 512] and partial_lse [S, R]")
    dev = partial_out.device
    if dev.type != "cuda":
        raise ValueError("libmla runs on the GPU only: partials must be device tensors")
    for name, t in (("partial_lse", partial_lse), ("out", out), ("lse", lse)):
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, partial_out on {dev}")
    if out is None:
        out = torch.empty((R, D_LATENT), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((R,), dtype=torch.float32, device=dev)
    _require(out, "out", torch.bfloat16, 2)
    _require(lse, "lse", torch.float32, 1)
    with torch.cuda.device(dev):
        _check(lib().mla_combine(S, R, _ptr(partial_out), _ptr(partial_lse), _ptr(out),
                                 _ptr(lse), _stream(dev)))
    return out, lse


def mla_plan(seqlens: torch.Tensor, *, batch: int, seqlen_q: int, num_heads: int,
             max_blocks_per_seq: int, num_blocks: int, kv_dtype: int = KV_BF16,
             max_seqlen: int = 0, num_parts: int = 0, m_tile: int = 0):
    """The split partition mla_decode would use -> dict of int32 device tensors."""
    _require(seqlens, "seqlens", torch.int32, 1)
    if seqlens.device.type != "cuda":
        raise ValueError("libmla runs on the GPU only: seqlens must be a device tensor")
    prob = Problem(batch=batch, seqlen_q=seqlen_q, num_heads=num_heads,
                   max_blocks_per_seq=max_blocks_per_seq, num_blocks=num_blocks,
                   max_seqlen=max_seqlen, kv_dtype=kv_dtype, num_parts=num_parts,
                   m_tile=m_tile)
    dev = seqlens.device
    with torch.cuda.device(dev):
        P = problem_num_parts(prob)
        cap = 3 * batch + P + 2
        buf = torch.empty(cap, dtype=torch.int32, device=dev)
        _check(lib().mla_plan(ctypes.byref(prob), _ptr(seqlens), _ptr(buf), cap, _stream(dev)))
    B = batch
    return dict(P=P, seq_prefix=buf[:B + 1], part_start=buf[B + 1:B + P + 2],
                seq_first_part=buf[B + P + 2:2 * B + P + 2],
                seq_last_part=buf[2 * B + P + 2:3 * B + P + 2])


def _on_device(name: str, t: torch.Tensor, dev):
    if t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")


def mla_absorb_query(q_nope: torch.Tensor, q_rope: torch.Tensor, w_uk_t: torch.Tensor,
                     q_abs: Optional[torch.Tensor] = None) -> torch.Tensor:
    """q_abs = [W_UK[h]^T q_nope ; q_rope] per query row (include/mla.h).

    q_nope bf16 [..., H, 128], q_rope bf16 [..., H, 64], w_uk_t bf16 [H, 512, 128]
    (W_UK transposed per head) -> q_abs bf16 [..., H, 576]."""
    _require(w_uk_t, "w_uk_t", torch.bfloat16, 3)
    H = w_uk_t.shape[0]
    if tuple(w_uk_t.shape[1:]) != (D_LATENT, D_HEAD):
        raise ValueError("w_uk_t must be [H, 512, 128]")
    if q_nope.dtype != torch.bfloat16 or q_rope.dtype != torch.bfloat16:
        raise TypeError("q_nope and q_rope must be bfloat16")
    if not (q_nope.is_contiguous() and q_rope.is_contiguous()):
        raise ValueError("q_nope and q_rope must be contiguous")
    if q_nope.shape[-2:] != (H, D_HEAD) or q_rope.shape[-2:] != (H, D_ROPE) \
            or q_nope.shape[:-1] != q_rope.shape[:-1]:
        raise ValueError("q_nope must be [..., H, 128] and q_rope [..., H, 64]")
    dev = q_nope.device
    if dev.type != "cuda":
        raise ValueError("libmla runs on the GPU only")
    for name, t in (("q_rope", q_rope), ("w_uk_t", w_uk_t)):
        _on_device(name, t, dev)
    rows = q_nope.numel() // D_HEAD
    if q_abs is None:
        q_abs = torch.empty(q_nope.shape[:-1] + (D_K,), dtype=torch.bfloat16, device=dev)
    if q_abs.dtype != torch.bfloat16 or not q_abs.is_contiguous() or q_abs.numel() != rows * D_K:
        raise ValueError("q_abs must be contiguous bf16 [..., H, 576]")
    _on_device("q_abs", q_abs, dev)
    with torch.cuda.device(dev):
        _check(lib().mla_absorb_query(rows, H, _ptr(q_nope), _ptr(q_rope), _ptr(w_uk_t),
                                      _ptr(q_abs), _stream(dev)))
    return q_abs


def mla_project_output(o_lat: torch.Tensor, w_uv: torch.Tensor,
                       o: Optional[torch.Tensor] = None) -> torch.Tensor:
    """o = W_UV[h] o_lat per query row: o_lat bf16 [..., H, 512], w_uv bf16
    [H, 128, 512] -> o bf16 [..., H, 128]."""
    _require(w_uv, "w_uv", torch.bfloat16, 3)
    H = w_uv.shape[0]
    if tuple(w_uv.shape[1:]) != (D_HEAD, D_LATENT):
        raise ValueError("w_uv must be [H, 128, 512]")
    if o_lat.dtype != torch.bfloat16 or not o_lat.is_contiguous() or o_lat.shape[-2:] != (H, D_LATENT):
        raise ValueError("o_lat must be contiguous bf16 [..., H, 512]")
    dev = o_lat.device
    if dev.type != "cuda":
        raise ValueError("libmla runs on the GPU only")
    _on_device("w_uv", w_uv, dev)
    rows = o_lat.numel() // D_LATENT
    if o is None:
        o = torch.empty(o_lat.shape[:-1] + (D_HEAD,), dtype=torch.bfloat16, device=dev)
    if o.dtype != torch.bfloat16 or not o.is_contiguous() or o.numel() != rows * D_HEAD:
        raise ValueError("o must be contiguous bf16 [..., H, 128]")
    _on_device("o", o, dev)
    with torch.cuda.device(dev):
        _check(lib().mla_project_output(rows, H, _ptr(o_lat), _ptr(w_uv), _ptr(o),
                                        _stream(dev)))
    return o


def mla_cache_append(rows: torch.Tensor, block_table: torch.Tensor, seqlens: torch.Tensor,
                     kv_cache: torch.Tensor, kv_scales: Optional[torch.Tensor] = None) -> None:
    """Write the new rows (bf16 [B, s_q, 576]) of a decode step into the paged
    cache in place: bf16 [nb, 64, 576], int8 q8_0 with kv_scales float16
    [nb, 64, 18], uint8 fp8 with kv_scales float32 [nb, 64], or uint8 q4_0 codes
    [nb, 64, 288] in Hadamard rotation with kv_scales float16 [nb, 64, 18]
    (include/mla.h)."""
    _require(rows, "rows", torch.bfloat16, 3)
    if rows.shape[-1] != D_K:
        raise ValueError("rows must be [B, s_q, 576]")
    B, s_q, _ = rows.shape
    _require(block_table, "block_table", torch.int32, 2)
    _require(seqlens, "seqlens", torch.int32, 1)
    kind = _cache_kind(kv_cache)
    _check_cache_shape(kind, kv_cache)
    _check_scales(kind, kv_cache, kv_scales)
    if block_table.shape[0] != B or seqlens.shape[0] != B:
        raise ValueError("block_table and seqlens must have B rows")
    dev = rows.device
    if dev.type != "cuda":
        raise ValueError("libmla runs on the GPU only")
    for name, t in (("block_table", block_table), ("seqlens", seqlens), ("kv_cache", kv_cache),
                    ("kv_scales", kv_scales)):
        if t is not None:
            _on_device(name, t, dev)
    with torch.cuda.device(dev):
        _check(lib().mla_cache_append(B, s_q, _ptr(rows), _ptr(block_table),
                                      block_table.shape[1], _ptr(seqlens), kv_cache.shape[0],
                                      kind, _ptr(kv_cache), _ptr(kv_scales),
                                      _stream(dev)))
