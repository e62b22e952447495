"""Host-side checks of the LDS tile layouts used by the bf16 decode kernels
(128-, 32/64- and 16-row tiles; no GPU). The index formulas below restate the kernels' own
(lane offsets of the LDS-DMA copies, score and value operand reads, tail
clearing); the checks are that the copies fill every 16-byte unit of the
36 KiB tile exactly once from whole 128-byte lines, that every read fetches
the token and chunk its MFMA operand needs, and that the reads of one LDS
cycle hit distinct 16-byte bank groups (16 lanes per cycle for 16-byte reads,
32 for the 8-byte transposing reads, 256-byte bank window)."""
import itertools

ROW = 1152          # bytes per cached token (576 bf16)
TOKENS, CHUNKS = 32, 72


def _copies(doff):
    """unit -> (token, chunk) for the 36 copies of a tile: copy j of wave w
    writes units 64 (4 j + w) .. +63, lane l reading doff(w, l) + 128 j."""
    m = {}
    for w, j, l in itertools.product(range(4), range(9), range(64)):
        off = doff(w, l) + 128 * j
        assert off % 16 == 0
        u = (1024 * w + 4096 * j) // 16 + l
        assert u not in m
        m[u] = (off // ROW, (off % ROW) // 16)
    assert len(m) == TOKENS * CHUNKS and len(set(m.values())) == TOKENS * CHUNKS
    return m


def _whole_lines(doff):
    for w, j in itertools.product(range(4), range(9)):
        lines = {}
        for l in range(64):
            off = doff(w, l) + 128 * j
            lines.setdefault(off // 128, set()).add(off % 128)
        assert len(lines) == 8 and all(len(v) == 8 for v in lines.values())


# ---- 128-row and 32/64-row kernels (32x32x16 MFMA operands)
def pipe_doff(w, l):
    dc0 = (l >> 4) & 1
    dr = (l & 3) | ((((l >> 2) & 1) ^ dc0) << 2)
    dcc = dc0 | ((((l >> 3) ^ w) & 1) << 1) | (((l >> 5) & 1) << 2)
    return (8 * w + dr) * ROW + 16 * dcc


def test_pipe_layout():
    m = _copies(pipe_doff)
    _whole_lines(pipe_doff)
    for u, (t, c) in m.items():          # tail clearing
        c0 = (u >> 4) & 1
        assert 8 * ((u >> 6) & 3) + ((u & 3) | ((((u >> 2) & 1) ^ c0) << 2)) == t
    for k in range(36):                  # score operand: token l32, chunk 2k + hi
        groups = {}
        for lane in range(64):
            hi, l32 = lane >> 5, lane & 31
            R, r = l32 >> 3, l32 & 7
            kpart = 1024 * R + 16 * ((r & 3) | ((((r >> 2) ^ hi) & 1) << 2) | (hi << 4))
            kofs = kpart + 128 * ((R & 1) ^ (k & 1))
            byte = 4096 * (k >> 2) + 512 * ((k >> 1) & 1) + kofs
            assert m[byte // 16] == (l32, 2 * k + hi)
            groups.setdefault(lane >> 4, []).append((byte // 16) % 16)
        assert all(len(set(v)) == 16 for v in groups.values())
    # value operand, transposing 8-byte reads, for the column bases of the
    # 128-row kernel (128 w, 4 blocks of 32 columns) and of the 32/64-row
    # kernel with two waves per row group (256 cg, 8 blocks)
    cases = [(128 * w, cb) for w in range(4) for cb in range(4)]
    cases += [(256 * cg, ct) for cg in range(2) for ct in range(8)]
    for (cbase, cb), kk, p in itertools.product(cases, range(2), range(2)):
        groups = {}
        for lane in range(64):
            g16, i16 = lane >> 4, lane & 15
            vh, vq, vs = g16 >> 1, i16 & 3, i16 >> 2
            vlane = 64 * cbase + 16 * vs + 64 * (vh ^ (vq >> 1)) + 256 * (vq >> 1) + 8 * (vq & 1)
            vofs = vlane + 1024 * p + 128 * ((g16 & 1) ^ p)
            byte = vofs + 4096 * (cb >> 1) + 512 * (cb & 1) + 2048 * kk
            assert m[byte // 16] == (4 * vh + vs + 8 * p + 16 * kk,
                                     cbase // 8 + 4 * cb + 2 * (g16 & 1) + (vq >> 1))
            assert (byte % 16) // 8 == vq & 1
            groups.setdefault(lane >> 5, []).append(((byte // 16) % 16, (byte % 16) // 8))
        assert all(len(set(v)) == 32 for v in groups.values())


# ---- 16-row kernel (16x16x32 MFMA operands)
def narrow_doff(w, l):
    return (8 * w + (l & 7)) * ROW + 16 * (2 * (l >> 4) + (((l >> 3) ^ w) & 1))


def test_narrow_layout():
    m = _copies(narrow_doff)
    _whole_lines(narrow_doff)
    for u, (t, c) in m.items():
        assert 8 * ((u >> 6) & 3) + (u & 7) == t
    for ks, h, g in itertools.product(range(18), range(2), range(4)):
        banks = []                       # score operand: token i16 + 16 h, chunk 4 ks + g
        for i16 in range(16):
            kofs = 1024 * (i16 >> 3) + 16 * (i16 & 7) + 128 * ((i16 >> 3) ^ (g & 1)) + 256 * (g >> 1)
            byte = 4096 * (ks >> 1) + 512 * (ks & 1) + 2048 * h + kofs
            assert m[byte // 16] == (16 * h + i16, 4 * ks + g)
            banks.append((byte // 16) % 16)
        assert len(set(banks)) == 16
    for w, ct, h, half in itertools.product(range(4), range(8), range(2), range(2)):
        slots = []                       # value operand, 32 lanes per LDS cycle
        for gl, vs, vq in itertools.product(range(2), range(4), range(4)):
            g = 2 * half + gl
            vb = (8192 * w + 2048 * h + 1024 * (g >> 1) + 16 * (4 * (g & 1) + vs) +
                  128 * ((g >> 1) ^ (vq >> 1)) + 8 * (vq & 1))
            byte = vb + 4096 * (ct >> 2) + 256 * (ct & 3)
            assert m[byte // 16] == (16 * h + 4 * g + vs, 16 * w + 2 * ct + (vq >> 1))
            assert (byte % 16) // 8 == vq & 1
            slots.append(((byte // 16) % 16, (byte % 16) // 8))
        assert len(set(slots)) == 32
