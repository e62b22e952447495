"""The C-ABI library loads, exports what include/mla.h declares, and rejects
bad arguments on the host before any HIP call (CPU only: no kernel runs)."""
import ctypes
import math
import os
import re

import pytest

import mla_latent_kv_10_amd as mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mla.LIB_PATH):
        mla.build(force=False)
    return mla.lib()


def _declared():
    text = open(os.path.join(ROOT, "include", "mla.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", text)))


def test_header_declares_the_documented_entry_points():
    assert _declared() == sorted(mla.EXPORTS)


def test_every_declared_symbol_is_exported(L):
    for name in _declared():
        assert hasattr(L, name), name


def test_status_strings(L):
    for code, name in mla.STATUS.items():
        assert L.mla_status_str(code).decode() == name
    assert L.mla_status_str(99).decode() == "unknown mla_status"


def _prob(**kw):
    d = dict(batch=2, seqlen_q=1, num_heads=16, max_blocks_per_seq=4, num_blocks=8,
             max_seqlen=0, kv_dtype=0, num_parts=1, m_tile=0)
    d.update(kw)
    return mla.Problem(**d)


def _decode(L, prob, *, q=0x1000, kv=0x2000, sc=None, bt=0x3000, sl=0x4000, scale=0.1,
            out=0x5000, lse=0x6000, ws=0x7000, ws_bytes=1 << 30):
    vp = ctypes.c_void_p
    return L.mla_decode(None if prob is None else ctypes.byref(prob), vp(q), vp(kv),
                        vp(sc) if sc else None, vp(bt), vp(sl), ctypes.c_float(scale), vp(out),
                        vp(lse), vp(ws) if ws else None, ws_bytes, None)


@pytest.mark.parametrize("field,value,status", [
    ("batch", -1, 1), ("batch", 4097, 2), ("seqlen_q", 0, 1), ("num_heads", 0, 1),
    ("num_heads", 5000, 2), ("max_blocks_per_seq", 0, 1), ("num_blocks", -1, 1),
    ("max_seqlen", -5, 1), ("kv_dtype", 7, 1), ("num_parts", -1, 1), ("m_tile", 48, 1),
])
def test_descriptor_validation(L, field, value, status):
    assert _decode(L, _prob(**{field: value})) == status
    assert L.mla_last_error().decode() != ""


def test_null_descriptor_and_arrays(L):
    assert _decode(L, None) == 1
    assert _decode(L, _prob(), q=0) == 1
    assert _decode(L, _prob(), lse=0) == 1
    assert _decode(L, _prob(kv_dtype=1)) == 1           # q8_0 needs kv_scales
    assert _decode(L, _prob(), ws=0) == 1


def test_alignment_and_scale(L):
    assert _decode(L, _prob(), q=0x1008) == 1
    assert _decode(L, _prob(), out=0x5004) == 1
    assert _decode(L, _prob(), lse=0x6002) == 1
    assert _decode(L, _prob(kv_dtype=1), sc=0x8004) == 1
    assert _decode(L, _prob(), scale=math.nan) == 1
    assert _decode(L, _prob(), scale=math.inf) == 1


def test_empty_batch_is_a_no_op(L):
    assert _decode(L, _prob(batch=0), q=0, kv=0) == 0


def _ws(L, prob):
    n = ctypes.c_size_t(0)
    assert L.mla_workspace_size(ctypes.byref(prob), ctypes.byref(n)) == 0
    return n.value


def test_workspace_size_formula(L):
    # one part: only the block prefix; P parts: + 2P slots of lse and bf16 rows
    assert _ws(L, _prob(num_parts=1)) == 256
    B, M, P = 2, 16, 5
    pre = 256
    lse = (2 * P * M * 4 + 255) // 256 * 256
    assert _ws(L, _prob(num_parts=P)) == pre + lse + 2 * P * M * 512 * 2
    assert _ws(L, _prob(num_parts=3, seqlen_q=2, num_heads=128)) == 256 + 2 * 3 * 256 * 4 + 2 * 3 * 256 * 512 * 2


def test_row_tile_choices(L):
    n = ctypes.c_size_t(0)
    # the 16-row tile exists for the bf16 cache only
    for mt in (16, 32, 64, 128):
        assert L.mla_workspace_size(ctypes.byref(_prob(m_tile=mt)), ctypes.byref(n)) == 0
    assert L.mla_workspace_size(ctypes.byref(_prob(m_tile=16, kv_dtype=1)),
                                ctypes.byref(n)) == 2
    assert "m_tile" in L.mla_last_error().decode()
    for mt in (32, 64, 128):
        assert L.mla_workspace_size(ctypes.byref(_prob(m_tile=mt, kv_dtype=1)),
                                    ctypes.byref(n)) == 0
    # the q4_0 cache in Hadamard rotation: as q8_0
    assert L.mla_workspace_size(ctypes.byref(_prob(m_tile=16, kv_dtype=3)),
                                ctypes.byref(n)) == 2
    assert "q4_0" in L.mla_last_error().decode()
    for mt in (0, 32, 64, 128):
        assert L.mla_workspace_size(ctypes.byref(_prob(m_tile=mt, kv_dtype=3)),
                                    ctypes.byref(n)) == 0
    assert _decode(L, _prob(kv_dtype=3)) == 1           # q4_0 needs kv_scales too


def test_workspace_too_small(L):
    need = _ws(L, _prob(num_parts=4))
    assert _decode(L, _prob(num_parts=4), ws_bytes=need - 1) == 3
    assert "workspace" in L.mla_last_error().decode()


def test_num_parts_override(L):
    n = ctypes.c_int32(0)
    assert L.mla_num_parts(ctypes.byref(_prob(num_parts=7)), ctypes.byref(n)) == 0
    assert n.value == 7


def test_combine_and_plan_validation(L):
    vp = ctypes.c_void_p
    assert L.mla_combine(0, 4, vp(0x1000), vp(0x2000), vp(0x3000), vp(0x4000), None) == 1
    assert L.mla_combine(2, -1, vp(0x1000), vp(0x2000), vp(0x3000), vp(0x4000), None) == 1
    assert L.mla_combine(2, 0, None, None, None, None, None) == 0
    assert L.mla_combine(2, 3, vp(0x1008), vp(0x2000), vp(0x3000), vp(0x4000), None) == 1
    prob = _prob(num_parts=3)
    assert L.mla_plan(ctypes.byref(prob), vp(0x1000), vp(0x2000), 3 * 2 + 3 + 1, None) == 1
    assert L.mla_plan(ctypes.byref(prob), vp(0x1000), None, 100, None) == 1


def test_binding_refuses_host_tensors():
    import torch
    q = torch.zeros(1, 1, 16, 576, dtype=torch.bfloat16)
    kv = torch.zeros(4, 64, 576, dtype=torch.bfloat16)
    bt = torch.zeros(1, 4, dtype=torch.int32)
    sl = torch.full((1,), 256, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU only"):
        mla.mla_decode(q, kv, bt, sl, 0.1)
    with pytest.raises(ValueError, match="GPU only"):
        mla.mla_combine(torch.zeros(2, 3, 512), torch.zeros(2, 3))
