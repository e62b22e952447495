"""Host restatement of the plan steps every decode kernel runs in its
prologue, checked against the oracle's plan (no GPU): the wave's block-count
scan (shifts by 1, 2, 4, 8 lanes within rows of 16, then the totals of the
lower rows added) and the part membership of a sequence by interval tests on
the block prefix, which replaces part indices computed by division."""
import numpy as np
import pytest

import oracle
import workload as wl


def _wave_scan(v):
    """Inclusive scan of 64 lane values as the kernel forms it."""
    x = np.array(v, dtype=np.int64)
    for n in (1, 2, 4, 8):
        y = np.zeros_like(x)
        for lane in range(64):
            if lane % 16 >= n:
                y[lane] = x[lane - n]
        x = x + y
    r = [x[15], x[31], x[47]]
    for lane in range(64):
        row = lane // 16
        x[lane] += sum(r[:row])
    return x


def test_wave_scan_is_the_inclusive_prefix():
    rng = np.random.default_rng(5)
    for _ in range(20):
        v = rng.integers(0, 200, 64)
        assert np.array_equal(_wave_scan(v), np.cumsum(v))


def _members(pre, T, P, part):
    """The sequences a part works on, by the kernels' interval tests."""
    p_lo, p_hi = part * T // P, (part + 1) * T // P
    out = []
    for b in range(len(pre) - 1):
        lo, hi = int(pre[b]), int(pre[b + 1])
        if hi > lo:
            mine = lo < p_hi and hi > p_lo
        else:
            mine = (p_lo <= lo < p_hi) if lo < T else part == P - 1
        if mine:
            out.append(b)
    return out


@pytest.mark.parametrize("B,P,seed", [(1, 1, 1), (5, 3, 2), (64, 256, 4), (7, 40, 5),
                                      (300, 17, 6), (12, 500, 7), (40, 64, 8)])
def test_part_membership_matches_the_oracle_plan(B, P, seed):
    sl = wl.uniform_int(B, seed, 7, 0, 3000)
    sl[::5] = 0
    sl[-1] = 0                    # an empty sequence at the end of the pool
    max_blocks = 40
    pl = oracle.plan(sl, max_blocks, P)
    pre = pl["seq_prefix"]
    T = int(pre[-1])
    fp, lp = pl["seq_first_part"], pl["seq_last_part"]
    for part in range(P):
        got = _members(pre, T, P, part)
        want = [b for b in range(B) if fp[b] <= part <= lp[b]]
        assert got == want
        # contiguous: the kernels walk [b_first, b_last]
        assert got == list(range(got[0], got[-1] + 1)) if got else True
