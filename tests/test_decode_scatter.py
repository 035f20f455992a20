"""CPU check of the decode kernel's reduce-scatter of per-lane dot products (no GPU).

A token row's LPT lanes each hold GW partial sums, one per query head.  Exchange
step s pairs lanes at distance LPT >> (s+1): 16 by a swizzle (lane ^ 16), 8 by
row_ror:8 (lane ^ 8), 4 by row_half_mirror (lane l <-> l ^ 7 inside 8 lanes), 2 and
1 by quad_perm (lane ^ 2, lane ^ 1).  While more than one value is live, a step
keeps the lower half of the live register slots and adds the partner's upper
half; once one is left it only adds.  Register slot j of a lane holds head
j ^ head_off(lane), with head_off's bit for step s the lane's distance bit, taken
relative to bit 2 for the steps after a splitting distance-4 step.  These are
the formulas of decode.hip, restated here: every lane must end with the full
sums of heads head_off .. head_off + VPL, and owner(g) / slot(g) must name where
head g is (the broadcast of the weights reads it there).
"""

import numpy as np
import pytest


def ilog2(x):
    return 0 if x <= 1 else 1 + ilog2(x // 2)


def partner(lane, d):
    return lane ^ 7 if d == 4 else lane ^ d


def params(lpt, gw):
    ns = min(ilog2(gw), ilog2(lpt))
    return ns, gw >> ns, lpt >= 8 and ilog2(lpt) - 3 < ns


def head_off(lane, lpt, gw):
    ns, _, mirror = params(lpt, gw)
    off = 0
    for s in range(ns):
        d = lpt >> (s + 1)
        bit = 1 if lane & d else 0
        if mirror and d < 4:
            bit ^= (lane >> 2) & 1
        if bit:
            off += gw >> (s + 1)
    return off


def owner(g, lpt, gw):
    ns, _, mirror = params(lpt, gw)
    lane = 0
    for s in range(ns):
        d = lpt >> (s + 1)
        bit = 1 if g & (gw >> (s + 1)) else 0
        if mirror and d < 4:
            bit ^= (lane >> 2) & 1
        if bit:
            lane |= d
    return lane


def reduce_scatter(part, lpt, gw):
    """part[lane][head] -> registers after every exchange step."""
    v = np.array([[part[l][j ^ head_off(l, lpt, gw)] for j in range(gw)] for l in range(lpt)])
    n, d = gw, lpt // 2
    while d >= 1:
        new = v.copy()
        for l in range(lpt):
            p = partner(l, d)
            if n > 1:
                for k in range(n // 2):
                    new[l][k] = v[l][k] + v[p][n // 2 + k]
            else:
                new[l][0] = v[l][0] + v[p][0]
        n = max(1, n // 2)
        v, d = new, d // 2
    return v


@pytest.mark.parametrize("lpt", [2, 4, 8, 16, 32])
@pytest.mark.parametrize("gw", [1, 2, 4, 8, 16, 32])
def test_every_lane_ends_with_its_heads(lpt, gw):
    rng = np.random.default_rng(lpt * 100 + gw)
    part = rng.integers(-1000, 1000, (lpt, gw)).astype(np.int64)   # exact sums
    v = reduce_scatter(part, lpt, gw)
    _, vpl, _ = params(lpt, gw)
    total = part.sum(0)
    for l in range(lpt):
        for k in range(vpl):
            assert v[l][k] == total[head_off(l, lpt, gw) + k], (l, k)
    for g in range(gw):
        assert head_off(owner(g, lpt, gw), lpt, gw) + (g & (vpl - 1)) == g


def test_mirror_correction_is_needed():
    """Without the relative bits, lanes paired by row_half_mirror disagree on the
    head order (8 lanes per token, 4 heads: two splitting steps after distance 4)."""
    lpt, gw = 8, 4
    part = np.arange(lpt * gw).reshape(lpt, gw)
    ns, _, _ = params(lpt, gw)

    def plain_off(lane):
        return sum(gw >> (s + 1) for s in range(ns) if lane & (lpt >> (s + 1)))

    v = np.array([[part[l][j ^ plain_off(l)] for j in range(gw)] for l in range(lpt)])
    n, d = gw, lpt // 2
    while d >= 1:
        new = v.copy()
        for l in range(lpt):
            p = partner(l, d)
            if n > 1:
                for k in range(n // 2):
                    new[l][k] = v[l][k] + v[p][n // 2 + k]
            else:
                new[l][0] = v[l][0] + v[p][0]
        n = max(1, n // 2)
        v, d = new, d // 2
    total = part.sum(0)
    assert any(v[l][0] != total[plain_off(l)] for l in range(lpt))
