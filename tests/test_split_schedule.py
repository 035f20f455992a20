"""CPU check of the split-KV schedule the decode kernels use (no GPU).

The split kernel lays the tiles of every (sequence, KV head) segment end to end
and gives share w of nw = min(num_splits, total) the tiles
[w*total//nw, (w+1)*total//nw); a piece (share w, segment s) writes its partial
to slot w + s.  The merge kernel finds the shares of segment s as
share_of(first tile) .. share_of(last tile) with
share_of(X) = ((X+1)*nw - 1) // total.  These are the formulas of decode.hip,
restated here to check their invariants over many shapes.
"""

import numpy as np
import pytest


def schedule(tiles_per_seq, hkv, num_splits):
    seg_tiles = np.repeat(np.asarray(tiles_per_seq, dtype=np.int64), hkv)
    starts = np.concatenate([[0], np.cumsum(seg_tiles)])
    total = int(starts[-1])
    nw = min(num_splits, total)
    pieces = []                      # (share, segment, first tile, n tiles)
    for w in range(nw):
        x, x1 = w * total // nw, (w + 1) * total // nw
        assert x < x1, "empty share"
        while x < x1:
            s = int(np.searchsorted(starts, x, side="right") - 1)
            n = min(int(starts[s + 1]) - x, x1 - x)
            pieces.append((w, s, x - int(starts[s]), n))
            x += n
    return seg_tiles, starts, total, nw, pieces


def share_of(x, total, nw):
    return ((x + 1) * nw - 1) // total


@pytest.mark.parametrize("seed", range(40))
def test_schedule_invariants(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 40))
    hkv = int(rng.choice([1, 2, 8]))
    tiles = rng.integers(0, 50, size=B) * (rng.random(B) > 0.2)
    splits = int(rng.choice([1, 2, 3, 7, 64, 997, 4096]))
    seg_tiles, starts, total, nw, pieces = schedule(tiles, hkv, splits)
    if total == 0:
        assert not pieces
        return
    # every tile covered exactly once
    cover = np.zeros(total, dtype=int)
    for w, s, t0, n in pieces:
        cover[starts[s] + t0: starts[s] + t0 + n] += 1
    assert np.all(cover == 1)
    # partial slots are unique and inside the workspace
    slots = [w + s for w, s, t0, n in pieces if not (t0 == 0 and n == seg_tiles[s])]
    assert len(slots) == len(set(slots))
    assert all(0 <= x < splits + len(seg_tiles) for x in slots)
    # the merge finds exactly the shares that wrote pieces of each segment
    for s in range(len(seg_tiles)):
        if seg_tiles[s] == 0:
            continue
        writers = sorted(w for w, ps, t0, n in pieces if ps == s)
        w0 = share_of(int(starts[s]), total, nw)
        w1 = share_of(int(starts[s + 1]) - 1, total, nw)
        assert writers == list(range(w0, w1 + 1))
