"""Host-side checks of the LDS tile layouts used by the bf16 decode kernels
(128-, 32/64- and 16-row tiles), of the 128-row kernel's query-row load, and
of the index arithmetic of the q4_0 (Hadamard) path (no GPU). The index formulas below restate the kernels' own
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


# ---- query rows of the 128-row kernel: load 4C + R of a wave reads block
# (C, R) of the K-tile layout with the copies' lane placement (rows past M
# read row M - 1); pass p writes blocks C = 4p .. 4p + 3 at 1024 (4 (C - 4p) + R)
# of the wave's 18 KiB region and reads k-steps 16p .. 16p + 15 back at
# kstep_ofs(k) - 16384 p + kofs.
def test_query_rows_load_and_read_back():
    for M in (128, 40, 16, 256):
        for row0 in range(0, 128, 32):
            region = {}
            for C, R, l in itertools.product(range(9), range(4), range(64)):
                dc0 = (l >> 4) & 1
                dr = (l & 3) | ((((l >> 2) & 1) ^ dc0) << 2)
                dcq = dc0 | ((((l >> 3) ^ R) & 1) << 1) | (((l >> 5) & 1) << 2)
                src_row = min(row0 + 8 * R + dr, M - 1)
                assert 0 <= src_row < M
                p = C // 4
                byte = 1024 * (4 * (C - 4 * p) + R) + 16 * l
                assert byte + 16 <= 18432          # inside the wave's region
                region[(p, byte // 16)] = (8 * R + dr, 8 * C + dcq)
            # each load reads eight whole 128-byte lines when no row is clamped
            if row0 + 32 <= M:
                for C, R in itertools.product(range(9), range(4)):
                    lines = {}
                    for l in range(64):
                        dc0 = (l >> 4) & 1
                        dr = (l & 3) | ((((l >> 2) & 1) ^ dc0) << 2)
                        dcq = dc0 | ((((l >> 3) ^ R) & 1) << 1) | (((l >> 5) & 1) << 2)
                        off = (8 * R + dr) * ROW + 16 * (8 * C + dcq)
                        lines.setdefault(off // 128, set()).add(off % 128)
                    assert len(lines) == 8 and all(len(v) == 8 for v in lines.values())
            for k, lane in itertools.product(range(36), range(64)):
                hi, l32 = lane >> 5, lane & 31
                R, r = l32 >> 3, l32 & 7
                kpart = 1024 * R + 16 * ((r & 3) | ((((r >> 2) ^ hi) & 1) << 2) | (hi << 4))
                kofs = kpart + 128 * ((R & 1) ^ (k & 1))
                p = k // 16
                byte = 4096 * (k >> 2) + 512 * ((k >> 1) & 1) - 16384 * p + kofs
                assert region[(p, byte // 16)] == (l32, 2 * k + hi)


# ---- q4_0 cache in Hadamard rotation: the matrix-core form of n = H (c - 8)
def _hadamard(m, k):
    return -1 if bin(m & k).count("1") & 1 else 1


def test_q4_hadamard_product_and_tile_writes():
    import numpy as np
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 16, size=(32, 32))          # [token, code index] of one block
    packed = np.zeros((32, 16), np.int64)               # 16 bytes per token, low nibble first
    for j in range(32):
        packed[:, j // 2] |= codes[:, j] << (4 * (j & 1))
    # B operand: lane (t, hi) of MFMA 1 holds codes 8 hi + e from the dword at
    # byte 4 hi, of MFMA 2 codes 16 + 8 hi + e from byte 8 + 4 hi, each as
    # bf16 bits 0x4300 | c, i.e. the value 128 + c
    def dword(t, byte):
        return sum(int(packed[t, byte + i]) << (8 * i) for i in range(4))

    def nib8(w):
        vals = []
        for k in range(4):
            lo, hi_ = (w >> (8 * k)) & 0xF, (w >> (8 * k + 4)) & 0xF
            for bits in ((0x4300 | lo), (0x4300 | hi_)):
                assert bits >> 7 == 0x86                 # exponent of 128, mantissa = c
                vals.append(128 + (bits & 0x7F))
        return vals
    D = np.zeros((32, 32), np.int64)                    # D[m][t]
    for t, hi in itertools.product(range(32), range(2)):
        b0 = nib8(dword(t, 4 * hi))
        b1 = nib8(dword(t, 8 + 4 * hi))
        assert b0 == [128 + c for c in codes[t, 8 * hi:8 * hi + 8]]
        assert b1 == [128 + c for c in codes[t, 16 + 8 * hi:16 + 8 * hi + 8]]
        for m in range(32):
            D[m, t] += sum(_hadamard(m, 8 * hi + e) * b0[e] for e in range(8))
            D[m, t] += sum(_hadamard(m, 16 + 8 * hi + e) * b1[e] for e in range(8))
    D[0, :] -= 4352
    H = np.array([[_hadamard(m, j) for j in range(32)] for m in range(32)])
    assert np.array_equal(D, H @ (codes.T - 8))
    assert np.abs(D).max() <= 256                       # exact in bf16 (8 significant bits)
    # accumulator element i of lane (t, hi) is row m = 8 (i >> 2) + 4 hi + (i & 3);
    # the lane writes rows 8 q + 4 hi .. + 3 as 8 bytes at offset 8 hi of
    # chunk 4 g + q of token t: every (token, column) once, in column order
    for g in (0, 5, 17):
        seen = {}
        for t, hi, q in itertools.product(range(32), range(2), range(4)):
            chunk = 4 * g + q
            for e in range(4):
                col = 8 * chunk + 4 * hi + e
                i = 4 * q + e
                assert 8 * (i >> 2) + 4 * hi + (i & 3) == col - 32 * g
                assert (t, col) not in seen
                seen[(t, col)] = True
        assert len(seen) == 32 * 32


def _rg_unit(t, c):
    R, r, C, cc = t >> 3, t & 7, c >> 3, c & 7
    return 64 * (4 * C + R) + ((r & 3) | ((((r >> 2) ^ cc) & 1) << 2) | (((R ^ (cc >> 1)) & 1) << 3)
                               | ((cc & 1) << 4) | (((cc >> 2) & 1) << 5))


def test_q4_half_blocks_of_the_128_row_kernel():
    """Blocks 16 and 17 of a tile are converted by token halves on 16x16x32
    MFMAs: the H operands built from the sign table equal H[m][k]; the
    product of lane (l & 15, l >> 4) gives n[m][th] for m = 4 (l >> 4) + i
    (and + 16); together with the full blocks 0..15 (four per wave) every
    8-byte half-unit of both tiles is written exactly once, with the rows
    it holds."""
    import numpy as np
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 16, size=(32, 32))          # one block: [token, code index]
    packed = np.zeros((32, 16), np.int64)
    for j in range(32):
        packed[:, j // 2] |= codes[:, j] << (4 * (j & 1))
    H = np.array([[_hadamard(m, j) for j in range(32)] for m in range(32)])
    want = H @ (codes.T - 8)                             # n[m][t]
    writes = {}
    for w in range(4):
        for g in range(w, 16, 4):                        # full blocks: lane (t, hi), 4 q
            for t, hi, q in itertools.product(range(32), range(2), range(4)):
                key = (_rg_unit(t, 4 * g + q), hi)
                assert key not in writes
                writes[key] = (g, t, [8 * q + 4 * hi + i for i in range(4)])
        g = 16 + (w >> 1)
        for lane in range(64):
            l16, qd = lane & 15, lane >> 4
            th = 16 * (w & 1) + l16
            rmask = (0x963C5AF066CCAA00 >> (8 * (l16 & 7))) & 0xFFFFFFFF
            s0 = 0x80008000 if ((l16 >> 3) & qd & 1) else 0
            s1 = 0x80008000 if (qd & 2) else 0
            a0, a1 = [], []
            for j in range(4):
                ha = 0x3F803F80 | (((rmask >> (2 * j)) & 1) << 15) | (((rmask >> (2 * j + 1)) & 1) << 31)
                ha ^= s0
                for h in range(2):
                    a0.append(-1 if (ha >> (16 * h + 15)) & 1 else 1)
                    a1.append(-1 if ((ha ^ s1) >> (16 * h + 15)) & 1 else 1)
            assert a0 == [_hadamard(l16, 8 * qd + e) for e in range(8)]
            assert a1 == [_hadamard(l16 + 16, 8 * qd + e) for e in range(8)]
            # word qd of the token's 16 bytes holds codes 8 qd .. 8 qd + 7
            wd = sum(int(packed[th, 4 * qd + i]) << (8 * i) for i in range(4))
            assert [(wd >> (4 * e)) & 0xF for e in range(8)] == list(codes[th, 8 * qd:8 * qd + 8])
            for base, off in ((0, 0), (16, 2)):
                key = (_rg_unit(th, 4 * g + off + (qd >> 1)), qd & 1)
                assert key not in writes
                writes[key] = (g, th, [base + 4 * qd + i for i in range(4)])
    assert len(writes) == 32 * 72 * 2
    for (u, half), (g, t, rows) in writes.items():
        # the half-unit belongs to token t, chunk c with rows 8 (c % 4) + 4 half ..
        c = [c for c in range(72) if _rg_unit(t, c) == u]
        assert len(c) == 1 and c[0] // 4 == g
        assert rows == [8 * (c[0] % 4) + 4 * half + i for i in range(4)]
    # the product over 16x16x32 (rows m, 16 tokens, k = 32 codes) is n
    for h in range(2):
        for m in range(32):
            for n in range(16):
                t = 16 * h + n
                acc = sum(_hadamard(m, k) * (128 + codes[t, k]) for k in range(32))
                assert acc - (4352 if m == 0 else 0) == want[m, t]


def test_q4_code_copies_of_the_64_row_kernel():
    # load k < 9: lane (l32, hi) reads 16 bytes at l32 * 288 + (2k + hi) * 16
    # into unit 64 k + l, which must be unit 32 g + t of block g = 2k + hi,
    # token t = l32; the two scale loads cover the 1152 scale bytes
    seen = set()
    for k, l in itertools.product(range(9), range(64)):
        hi, l32 = l >> 5, l & 31
        src = l32 * 288 + (2 * k + hi) * 16
        assert src + 16 <= 32 * 288
        unit = 64 * k + l
        assert unit == 32 * (2 * k + hi) + l32
        assert src == 288 * (unit % 32) + 16 * (unit // 32)
        seen.add(unit)
    assert seen == set(range(18 * 32))
