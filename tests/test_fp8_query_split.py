"""Host checks of the fp8 score chain of the 128-row kernel (no GPU).

The kernel scores an E4M3 cache on the fp8 matrix core against the query
carried as two E4M3 parts per value (hi + lo, one power-of-two scale per row).
Checked here, in plain Python:
  * the split itself: with 2^e chosen from the row's largest bf16 exponent so
    that the largest |x 2^e| lies in [128, 256), hi = E4M3(x 2^e) to nearest
    even and lo = E4M3(x 2^e - hi) add up to x 2^e exactly for every value
    with |x 2^e| >= 1/4, and to within one E4M3 subnormal step (2^-9 after
    scaling) below that;
  * the operand layouts: for every k-step and lane, the 32 code bytes the
    lane reads from the fp8 stage (chunk c of token t at byte 512 c +
    16 (t ^ 4 (c & 1))) and the 32 query bytes it holds after the lane swap
    cover the same 64-column k-step slice, column for column in the same byte
    order, and the 64 lanes of a k-step cover each (token or row, column)
    exactly once.
"""
import numpy as np


def e4m3_rne(x: float) -> float:
    """OCP E4M3 value nearest to x (ties to even); |x| stays below 448 here."""
    if x == 0.0:
        return 0.0
    a = abs(x)
    e = max(int(np.floor(np.log2(a))), -6)   # subnormals share the 2^-6 exponent
    ulp = 2.0 ** (e - 3)
    q = a / ulp
    r = np.floor(q)
    if q - r > 0.5 or (q - r == 0.5 and int(r) % 2 == 1):
        r += 1
    v = r * ulp
    assert v <= 448.0
    return float(np.copysign(v, x))


def bf16_round(x: np.ndarray) -> np.ndarray:
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32)


def row_exponent(row: np.ndarray) -> int:
    """e of the kernel: 134 - (biased bf16 exponent of the row's largest |x|), clamped."""
    bits = (row.astype(np.float32).view(np.uint32) >> 16) & 0x7FFF
    return int(min(100, max(-100, 134 - ((int(bits.max()) >> 7) & 0xFF))))


def test_split_is_exact_down_to_a_quarter():
    rng = np.random.default_rng(11)
    for trial in range(40):
        scale = 2.0 ** rng.integers(-20, 20)
        row = bf16_round(rng.standard_normal(576) * scale)
        row[rng.integers(0, 576, 8)] = 0.0
        e = row_exponent(row)
        big = np.abs(row).max() * 2.0 ** e
        assert 128.0 <= big < 256.0
        for x in row.astype(np.float64):
            q = x * 2.0 ** e
            hi = e4m3_rne(q)
            lo = e4m3_rne(q - hi)
            if abs(q) >= 0.25:
                assert hi + lo == q, (x, e, hi, lo)
            else:
                assert abs(hi + lo - q) <= 2.0 ** -10, (x, e, hi, lo)


def test_zero_row_keeps_zero_parts():
    row = np.zeros(576, np.float32)
    e = row_exponent(row)
    assert e == 100
    assert all(e4m3_rne(float(x) * 2.0 ** e) == 0.0 for x in row)


def stage_byte(t: int, col: int) -> int:
    """Byte of token t, column col in an fp8 stage: chunk c = col // 16."""
    c = col // 16
    return 512 * c + 16 * (t ^ (4 * (c & 1))) + col % 16


def test_score_operands_cover_the_same_columns():
    inverse = {stage_byte(t, col): (t, col) for t in range(32) for col in range(576)}
    assert len(inverse) == 32 * 576
    for k in range(9):
        seen_k, seen_q = set(), set()
        for lane in range(64):
            l32, hi = lane & 31, lane >> 5
            ofs0 = 1024 * hi + 16 * l32            # kofs8_0
            ofs1 = 1024 * hi + 512 + 16 * (l32 ^ 4)  # kofs8_1
            kbytes = [2048 * k + ofs0 + i for i in range(16)] + [2048 * k + ofs1 + i for i in range(16)]
            kcols = []
            for b in kbytes:
                t, col = inverse[b]
                assert t == l32
                kcols.append(col)
            # query: before the swap lane (row, h) holds bf16 chunks 2 s + h
            # (8 columns each) of k-steps s; the swap with the partner lane
            # leaves chunks 8 k + 4 hi + j (j = 0..3) in this lane, in order
            qcols = [8 * (8 * k + 4 * hi + j) + i for j in range(4) for i in range(8)]
            assert kcols == qcols == list(range(64 * k + 32 * hi, 64 * k + 32 * hi + 32))
            seen_k.update((l32, c) for c in kcols)
            seen_q.update((l32, c) for c in qcols)
        assert seen_k == seen_q == {(t, c) for t in range(32) for c in range(64 * k, 64 * k + 64)}


def test_lane_swap_delivers_the_needed_chunks():
    # permlane32 swap of A and B: lanes 0-31 get (A_lo, A_hi), lanes 32-63 (B_lo, B_hi)
    for k in range(9):
        owner = {}   # chunk -> (register, lane half) before the swap
        for s in range(4 * k, 4 * k + 4):
            for h in range(2):
                owner[2 * s + h] = (s - 4 * k, h)
        for hi in range(2):
            # the kernel swaps (qf[4k], qf[4k+2]) and (qf[4k+1], qf[4k+3])
            got = []
            for a, b in ((0, 2), (1, 3)):
                first = (a, 0) if hi == 0 else (b, 0)     # new vdst
                second = (a, 1) if hi == 0 else (b, 1)    # new vsrc
                got += [first, second]
            want = [owner[8 * k + 4 * hi + j] for j in range(4)]
            assert got == want
