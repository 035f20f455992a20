"""CPU check of the stream-K schedule of the packed-rows kernel (no GPU).

A (sequence, KV head) pair with q_len > 0 counts C start-up units plus one unit
per 64-key block of its window (at least one unit in all); the pairs' units, in
pair order, are cut into nw shares [w*T//nw, (w+1)*T//nw).  Share w runs a piece
per pair it touches: the piece's blocks are its units past the C start-up ones;
a piece that covers its whole pair writes the output, any other writes partials
to slot 2w (it starts at the share's start) or 2w + 1; each share records the
pair that begins in it and is cut at its end.  The merge finds that pair's
pieces in shares w .. share_of(last unit), slot 2w + 1 (2w if the pair begins at
the share's start) and 2v for the later shares v.  These are the formulas of
prefill.hip, restated here to check their invariants over many shapes.
"""

import numpy as np
import pytest

BN = 64


def units(lq, lk, window, c):
    nkb = (lk + BN - 1) // BN
    kbw = max(0, lk - lq - window + 1) // BN if (window > 0 and nkb > 0) else 0
    return (max(1, c + nkb - kbw) if lq > 0 else 0), kbw, nkb


def share_of(x, total, nw):
    return ((x + 1) * nw - 1) // total


def schedule(lqs, lks, window, c, nw):
    U = [units(lq, lk, window, c) for lq, lk in zip(lqs, lks)]
    pref = np.concatenate([[0], np.cumsum([u for u, _, _ in U])]).astype(np.int64)
    total = int(pref[-1])
    pieces, cuts = [], []
    for w in range(nw):
        lo, hi = w * total // nw, (w + 1) * total // nw
        cut = None
        if lo < hi:
            p = int(np.searchsorted(pref, lo, side="right") - 1)   # the pair holding unit lo
            while p < len(U) and pref[p] < hi:
                u, kbw, nkb = U[p]
                if u > 0:
                    start = int(pref[p])
                    plo, phi = max(lo, start) - start, min(hi, start + u) - start
                    whole = plo == 0 and phi == u
                    slot = None if whole else 2 * w + (0 if start <= lo else 1)
                    if start >= lo and start + u > hi:
                        cut = (p, start, start + u)
                    kb0, kb1 = kbw + max(0, plo - c), min(nkb, kbw + max(0, phi - c))
                    pieces.append(dict(w=w, p=p, plo=plo, phi=phi, slot=slot, blocks=range(kb0, max(kb0, kb1))))
                p += 1
        cuts.append(cut)
    return U, pref, total, pieces, cuts


def merge_slots(cut, w, total, nw):
    p, u0, u1 = cut
    lo = w * total // nw
    out = []
    for v in range(w, share_of(u1 - 1, total, nw) + 1):
        if v * total // nw < (v + 1) * total // nw:
            out.append(2 * v + (1 if (v == w and u0 > lo) else 0))
    return out


@pytest.mark.parametrize("seed", range(60))
def test_streamk_schedule_invariants(seed):
    rng = np.random.default_rng(seed)
    P = int(rng.choice([1, 2, 3, 7, 64, 256, 513]))
    nw = int(rng.choice([1, 2, 5, 64, 512]))
    c = int(rng.integers(0, 5))
    window = int(rng.choice([0, 0, 1, 100, 4096]))
    lqs = rng.choice([0, 1, 1, 4, 32], P)
    lks = np.maximum(rng.choice([0, 1, 16, 63, 64, 65, 1000, 30000], P), 0)
    U, pref, total, pieces, cuts = schedule(lqs, lks, window, c, nw)
    # Every key block of every pair is computed by exactly one piece.
    seen = {}
    for pc in pieces:
        for kb in pc["blocks"]:
            seen[(pc["p"], kb)] = seen.get((pc["p"], kb), 0) + 1
    for p, (u, kbw, nkb) in enumerate(U):
        for kb in range(kbw, nkb if u else kbw):
            assert seen.get((p, kb)) == 1, (p, kb)
    assert all(kbw <= kb < nkb for (p, kb) in seen for (_, kbw, nkb) in [U[p]])
    # Partial slots are unique and inside the workspace.
    slots = [pc["slot"] for pc in pieces if pc["slot"] is not None]
    assert len(slots) == len(set(slots)) and all(0 <= s < 2 * nw for s in slots)
    by_slot = {pc["slot"]: pc for pc in pieces if pc["slot"] is not None}
    # Every cut pair is merged once, from pieces that tile its units in order.
    merged = set()
    for w, cut in enumerate(cuts):
        if cut is None:
            continue
        got = [by_slot[s] for s in merge_slots(cut, w, total, nw)]
        assert all(g["p"] == cut[0] for g in got)
        spans = sorted((g["plo"], g["phi"]) for g in got)
        assert spans[0][0] == 0 and spans[-1][1] == U[cut[0]][0]
        assert all(a[1] == b[0] for a, b in zip(spans, spans[1:]))
        assert cut[0] not in merged
        merged.add(cut[0])
    assert merged == {pc["p"] for pc in pieces if pc["slot"] is not None}
    # A pair that no share cuts is written whole, by one piece.
    for p, (u, _, _) in enumerate(U):
        if u > 0 and p not in merged:
            assert sum(1 for pc in pieces if pc["p"] == p) == 1


def test_startup_units_balance_pieces():
    """With start-up units, a share that holds more pieces holds fewer key blocks."""
    lqs, lks = [1] * 8, [64 * 20] * 8
    _, _, _, pieces, _ = schedule(lqs, lks, 0, 3, 12)
    per = {}
    for pc in pieces:
        n, b = per.get(pc["w"], (0, 0))
        per[pc["w"]] = (n + 1, b + len(pc["blocks"]))
    by_pieces = {}
    for n, b in per.values():
        by_pieces.setdefault(n, []).append(b)
    assert max(by_pieces[2]) <= min(by_pieces[1])
