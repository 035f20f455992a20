"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each ``pin_*`` takes a loaded :class:`oracle.Oracle` and raises (AssertionError or
the oracle's own error) when the oracle disagrees with what the pages and the
mathematics fix:

* a library routine: ``torch.nn.functional.scaled_dot_product_attention`` in
  float64 on dense K/V rebuilt from the packed inputs (never from the pages),
  with its ``enable_gqa`` head expansion;
* brute force on tiny inputs: one dense block-diagonal masked softmax over the
  whole packed batch, in numpy;
* closed forms: one key -> its value; zero query -> mean of values; constant
  values; two keys with a hand-derived sigmoid weight; one dominant key;
* invariants: weights sum to one, GQA equals MHA on repeated KV heads, placement
  of pages does not change the output, decode equals the last prefill row,
  batch independence, and the packing example printed on the pages.

The same battery runs against copies of the oracle with a planted mistake
(see test_oracle_mutants.py); every mistake there must fail at least one pin.
"""

from __future__ import annotations

import json
import math
from pathlib import Path

import numpy as np
import torch
import torch.nn.functional as F

import workload as W
from oracle import ERANGE, EINVAL, OracleError

GOLDEN = Path(__file__).resolve().parent / "golden"

REL = 1e-12   # fp64 agreement between two exact-in-real-arithmetic evaluations


def f64(a: np.ndarray) -> np.ndarray:
    """Exact widening of generator arrays (float32 or bf16 bits) to float64."""
    if a.dtype == np.uint16:
        return W.bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def close(a, b, rel=REL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.isfinite(a).all(), f"{what}: non-finite values"
    scale = max(1.0, float(np.abs(b).max()) if b.size else 1.0)
    err = float(np.abs(a - b).max()) if a.size else 0.0
    assert err <= rel * scale, f"{what}: max err {err:.3e} > {rel * scale:.3e}"


def fill_pages(orc, case: W.DecodeCase, table=None, num_blocks=None):
    """Oracle-written page pools for a decode case (NaN sentinel elsewhere)."""
    table = case.block_table if table is None else table
    nb = case.num_blocks if num_blocks is None else num_blocks
    kc = W.nan_pool(nb, case.num_kv_heads, case.block_size, case.head_dim, case.dtype)
    vc = W.nan_pool(nb, case.num_kv_heads, case.block_size, case.head_dim, case.dtype)
    orc.paged_kv_write(case.k, case.v, case.cu_ctx, case.start_pos, table, kc, vc)
    return kc, vc


def decode(orc, case: W.DecodeCase, **kw):
    kc, vc = fill_pages(orc, case)
    return orc.gqa_paged_decode(case.q, kc, vc, case.block_table, case.context_lens, case.scale, **kw)


def sdpa_decode(case: W.DecodeCase) -> np.ndarray:
    """Library attention of each sequence's single query over its packed K/V."""
    out = np.zeros((case.batch, case.num_q_heads, case.head_dim))
    q, k, v = f64(case.q), f64(case.k), f64(case.v)
    for b in range(case.batch):
        a, e = int(case.cu_ctx[b]), int(case.cu_ctx[b + 1])
        if e == a:
            continue
        qt = torch.from_numpy(q[b]).unsqueeze(0).unsqueeze(2)             # [1, Hq, 1, d]
        kt = torch.from_numpy(k[a:e]).permute(1, 0, 2).unsqueeze(0)      # [1, Hkv, n, d]
        vt = torch.from_numpy(v[a:e]).permute(1, 0, 2).unsqueeze(0)
        r = F.scaled_dot_product_attention(qt, kt.contiguous(), vt.contiguous(),
                                           scale=float(case.scale), enable_gqa=True)
        out[b] = r[0, :, 0].numpy()
    return out


def sdpa_prefill(case: W.PrefillCase, causal: bool) -> np.ndarray:
    """Library attention run separately on every sequence of a packed batch."""
    q, k, v = f64(case.q), f64(case.k), f64(case.v)
    out = np.zeros_like(q)
    for s in range(case.batch):
        a, e = int(case.cu_seqlens[s]), int(case.cu_seqlens[s + 1])
        if e == a:
            continue
        qt = torch.from_numpy(q[a:e]).permute(1, 0, 2).unsqueeze(0)
        kt = torch.from_numpy(k[a:e]).permute(1, 0, 2).unsqueeze(0)
        vt = torch.from_numpy(v[a:e]).permute(1, 0, 2).unsqueeze(0)
        r = F.scaled_dot_product_attention(qt.contiguous(), kt.contiguous(), vt.contiguous(),
                                           is_causal=causal, scale=float(case.scale), enable_gqa=True)
        out[a:e] = r[0].permute(1, 0, 2).numpy()
    return out


def blockdiag_bruteforce(case: W.PrefillCase, causal: bool) -> np.ndarray:
    """One dense T x T masked softmax over the whole packed batch (numpy)."""
    q, k, v = f64(case.q), f64(case.k), f64(case.v)
    T = case.total_tokens
    G = case.num_q_heads // case.num_kv_heads
    seq_of = np.repeat(np.arange(case.batch), case.lengths)
    allowed = seq_of[:, None] == seq_of[None, :]
    if causal:
        allowed &= np.arange(T)[:, None] >= np.arange(T)[None, :]
    kk = np.repeat(k, G, axis=1)   # [T, Hq, d]: query head qh reads KV head qh // G
    vv = np.repeat(v, G, axis=1)
    s = np.einsum("ihd,jhd->hij", q, kk) * float(case.scale)
    s = np.where(allowed[None], s, -np.inf)
    s = s - s.max(axis=2, keepdims=True)
    w = np.exp(s)
    w = w / w.sum(axis=2, keepdims=True)
    return np.einsum("hij,jhd->ihd", w, vv)


# A small sweep of decode shapes: (lengths, Hq, Hkv, d, bs, dtype, seed)
DECODE_SWEEP = [
    ([5, 11], 4, 2, 16, 4, W.F32, 11),
    ([1, 2, 3, 40], 4, 4, 8, 1, W.F32, 12),
    ([17, 9], 8, 1, 16, 8, W.BF16, 13),
    ([6, 33, 12], 6, 3, 8, 2, W.BF16, 14),
    ([40], 4, 2, 16, 8, W.BF16, 15),
    ([3, 24, 7, 1], 8, 2, 8, 4, W.F32, 16),
]

PREFILL_SWEEP = [
    ([3, 9, 5], 4, 2, 16, W.F32, 21),
    ([1, 7, 12], 6, 3, 8, W.BF16, 22),
    ([20], 8, 1, 8, W.BF16, 23),
    ([4, 4, 10, 2], 4, 4, 16, W.F32, 24),
]


# ---------------------------------------------------------------------------
# library routine and brute force
# ---------------------------------------------------------------------------

def pin_decode_matches_library(orc):
    for lens, hq, hkv, d, bs, dt, seed in DECODE_SWEEP:
        c = W.make_decode_case(lens, hq, hkv, d, bs, dt, seed)
        close(decode(orc, c), sdpa_decode(c), what=f"decode {lens} {hq}/{hkv} d{d} bs{bs} {dt}")


def pin_prefill_matches_library(orc):
    for lens, hq, hkv, d, dt, seed in PREFILL_SWEEP:
        c = W.make_prefill_case(lens, hq, hkv, d, 4, dt, seed)
        for causal in (True, False):
            got = orc.gqa_varlen_prefill(c.q, c.k, c.v, c.cu_seqlens, c.scale, causal=causal)
            close(got, sdpa_prefill(c, causal), what=f"prefill {lens} causal={causal}")


def pin_prefill_matches_bruteforce(orc):
    for lens, hq, hkv, d, dt, seed in PREFILL_SWEEP[:3]:
        c = W.make_prefill_case(lens, hq, hkv, d, 4, dt, seed)
        for causal in (True, False):
            got = orc.gqa_varlen_prefill(c.q, c.k, c.v, c.cu_seqlens, c.scale, causal=causal)
            close(got, blockdiag_bruteforce(c, causal), what=f"brute force {lens} causal={causal}")


def pin_prefill_row_sampling(orc):
    c = W.make_prefill_case([5, 14, 3], 4, 2, 8, 4, W.BF16, 25)
    full = orc.gqa_varlen_prefill(c.q, c.k, c.v, c.cu_seqlens, c.scale)
    rows = np.array([0, 4, 5, 18, 21, 7], dtype=np.int32)
    part = orc.gqa_varlen_prefill(c.q, c.k, c.v, c.cu_seqlens, c.scale, rows=rows)
    assert np.array_equal(part, full[rows]), "sampled rows differ from the full evaluation"


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def pin_single_key_returns_its_value(orc):
    """With one cached token the only weight is 1, so the output is that value exactly."""
    c = W.make_decode_case([1, 1, 1], 4, 2, 16, 4, W.F32, 31)
    out = decode(orc, c)
    G = c.num_q_heads // c.num_kv_heads
    expect = np.repeat(f64(c.v), G, axis=1)     # [B, Hq, d] since every context is one token
    assert np.array_equal(out, expect), "one-token context must return the value row exactly"


def pin_prefill_first_row_is_value(orc):
    """Causal row 0 of each sequence sees only its own key, so it equals its value row."""
    c = W.make_prefill_case([3, 9, 5], 4, 2, 16, 4, W.F32, 32)
    out = orc.gqa_varlen_prefill(c.q, c.k, c.v, c.cu_seqlens, c.scale, causal=True)
    G = c.num_q_heads // c.num_kv_heads
    for a in c.cu_seqlens[:-1]:
        assert np.array_equal(out[a], np.repeat(f64(c.v[a]), G, axis=0)), f"row {a}"


def pin_zero_query_gives_mean(orc):
    """q = 0 makes every score 0 and every weight 1/n: the output is the mean value."""
    c = W.make_decode_case([7, 19], 4, 2, 8, 4, W.F32, 33)
    c.q[...] = 0.0
    out = decode(orc, c)
    G = c.num_q_heads // c.num_kv_heads
    v = f64(c.v)
    for b in range(c.batch):
        a, e = c.cu_ctx[b], c.cu_ctx[b + 1]
        close(out[b], np.repeat(v[a:e].mean(axis=0), G, axis=0), rel=1e-14, what="mean")


def pin_constant_values(orc):
    """If every value row is the same vector, any weighting returns it."""
    c = W.make_decode_case([9, 4], 8, 2, 8, 4, W.F32, 34)
    row = np.arange(1, 9, dtype=np.float32) * np.float32(0.5)
    c.v[...] = row
    out = decode(orc, c)
    close(out, np.broadcast_to(row.astype(np.float64), out.shape), rel=1e-14, what="constant")


def pin_two_keys_sigmoid(orc):
    """Two keys: weight of key 0 is 1 / (1 + exp(-(s0 - s1))), worked by hand.

    d = 4, q = (2, 0, 0, 0), k0 = (3, 0, 0, 0), k1 = (0, 1, 0, 0), scale = 1/sqrt(4) = 0.5,
    so s0 = 0.5 * 6 = 3, s1 = 0, and out = sig(3) v0 + (1 - sig(3)) v1.
    """
    c = W.make_decode_case([2], 1, 1, 4, 2, W.F32, 35, scale=0.5)
    c.q[...] = 0.0
    c.q[0, 0, 0] = 2.0
    c.k[...] = 0.0
    c.k[0, 0, 0] = 3.0
    c.k[1, 0, 1] = 1.0
    c.v[0, 0, :] = [1.0, 2.0, 3.0, 4.0]
    c.v[1, 0, :] = [-1.0, 0.5, 0.0, 8.0]
    w0 = 1.0 / (1.0 + math.exp(-3.0))
    expect = w0 * np.array([1.0, 2.0, 3.0, 4.0]) + (1.0 - w0) * np.array([-1.0, 0.5, 0.0, 8.0])
    out, probs = decode(orc, c, want_probs=True)
    close(out[0, 0], expect, rel=1e-15, what="two-key output")
    close(probs[0, 0, :2], [w0, 1.0 - w0], rel=1e-15, what="two-key weights")


def pin_dominant_key_large_logits(orc):
    """One key aligned with a huge query dominates; softmax stays exact for logits ~ 1e3."""
    c = W.make_decode_case([6], 2, 1, 4, 4, W.F32, 36, scale=0.5)
    c.q[...] = 0.0
    c.q[0, :, 0] = 40.0
    c.k[...] = 0.0
    c.k[3, 0, 0] = 50.0          # s = 0.5 * 40 * 50 = 1000 for key 3, 0 for the rest
    out = decode(orc, c)
    expect = np.repeat(f64(c.v[3]), 2, axis=0)
    close(out[0], expect, rel=1e-15, what="dominant key")


def pin_weights_sum_to_one(orc):
    for lens, hq, hkv, d, bs, dt, seed in DECODE_SWEEP[:4]:
        c = W.make_decode_case(lens, hq, hkv, d, bs, dt, seed)
        _, p = decode(orc, c, want_probs=True)
        for b, n in enumerate(c.context_lens):
            s = p[b, :, :n].sum(axis=1)
            assert np.all(np.abs(s - 1.0) < 1e-12), f"weights sum {s}"
            assert np.all(p[b, :, :n] >= 0.0)


def pin_identical_keys_uniform(orc):
    """All keys equal -> all scores equal -> uniform weights 1/n."""
    c = W.make_decode_case([5, 12], 4, 2, 8, 4, W.F32, 37)
    c.k[...] = c.k[0]
    _, p = decode(orc, c, want_probs=True)
    for b, n in enumerate(c.context_lens):
        close(p[b, :, :n], np.full((4, n), 1.0 / n), rel=1e-14, what="uniform weights")


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

def pin_gqa_equals_repeated_mha(orc):
    """GQA(Hq, Hkv) equals MHA(Hq) when each KV head is repeated for its G query heads."""
    c = W.make_decode_case([13, 6, 21], 6, 3, 8, 4, W.BF16, 41)
    G = 2
    m = W.make_decode_case([13, 6, 21], 6, 6, 8, 4, W.BF16, 41)
    m.q = c.q
    m.k = np.repeat(c.k, G, axis=1)
    m.v = np.repeat(c.v, G, axis=1)
    m.block_table, m.num_blocks = c.block_table, c.num_blocks
    assert np.array_equal(decode(orc, c), decode(orc, m)), "GQA differs from repeated-head MHA"
    p = W.make_prefill_case([5, 8], 6, 3, 8, 4, W.BF16, 42)
    got = orc.gqa_varlen_prefill(p.q, p.k, p.v, p.cu_seqlens, p.scale)
    mha = orc.gqa_varlen_prefill(p.q, np.repeat(p.k, G, axis=1), np.repeat(p.v, G, axis=1),
                                 p.cu_seqlens, p.scale)
    assert np.array_equal(got, mha), "prefill GQA differs from repeated-head MHA"


def pin_placement_invariance(orc):
    """Another page permutation, a larger pool and extra table columns leave the output bit-identical."""
    c = W.make_decode_case([9, 30, 4], 4, 2, 8, 4, W.BF16, 43)
    base = decode(orc, c)
    rng = np.random.default_rng(99)
    table, nb = W.place_pages(rng, c.context_lens, c.block_size, pool_factor=3.0, extra_cols=5)
    kc, vc = fill_pages(orc, c, table=table, num_blocks=nb)
    moved = orc.gqa_paged_decode(c.q, kc, vc, table, c.context_lens, c.scale)
    assert np.array_equal(base, moved), "output depends on physical placement"


def pin_batch_independence(orc):
    c = W.make_decode_case([9, 30, 4], 4, 2, 8, 4, W.F32, 44)
    full = decode(orc, c)
    for b in range(c.batch):
        a, e = c.cu_ctx[b], c.cu_ctx[b + 1]
        one = W.make_decode_case([int(c.context_lens[b])], 4, 2, 8, 4, W.F32, 45)
        one.q, one.k, one.v = c.q[b:b + 1].copy(), c.k[a:e].copy(), c.v[a:e].copy()
        assert np.array_equal(decode(orc, one)[0], full[b]), f"sequence {b} depends on its batch"


def pin_decode_equals_last_prefill_row(orc):
    """Decode over pages written from a prefill batch equals each sequence's last causal row."""
    p = W.make_prefill_case([6, 13, 1], 4, 2, 16, 4, W.BF16, 46)
    pre = orc.gqa_varlen_prefill(p.q, p.k, p.v, p.cu_seqlens, p.scale, causal=True)
    kc = W.nan_pool(p.num_blocks, p.num_kv_heads, p.block_size, p.head_dim, p.dtype)
    vc = W.nan_pool(p.num_blocks, p.num_kv_heads, p.block_size, p.head_dim, p.dtype)
    orc.paged_kv_write(p.k, p.v, p.cu_seqlens, np.zeros(p.batch, np.int32), p.block_table, kc, vc)
    last = p.cu_seqlens[1:] - 1
    dec = orc.gqa_paged_decode(p.q[last], kc, vc, p.block_table, p.lengths, p.scale)
    close(dec, pre[last], what="decode vs last prefill row")


def pin_packing_example(orc):
    """The pages' packing example: lengths 3, 9, 5 -> 17 packed tokens, no cross-sequence mixing."""
    g = json.loads((GOLDEN / "packing_3_9_5.json").read_text())
    p = W.make_prefill_case(g["lengths"], 4, 2, 8, 4, W.F32, 47)
    assert p.total_tokens == g["total_tokens"]
    assert p.cu_seqlens.tolist() == g["cu_seqlens"]
    out = orc.gqa_varlen_prefill(p.q, p.k, p.v, p.cu_seqlens, p.scale, causal=True)
    assert out.shape[0] == g["total_tokens"]
    for s in range(p.batch):
        a, e = g["cu_seqlens"][s], g["cu_seqlens"][s + 1]
        alone = orc.gqa_varlen_prefill(p.q[a:e], p.k[a:e], p.v[a:e], np.array([0, e - a], np.int32),
                                       p.scale, causal=True)
        assert np.array_equal(alone, out[a:e]), f"segment {s} is affected by its neighbours"


def pin_noncausal_last_row_equals_causal(orc):
    """The last row of a sequence sees every key of it under both masks."""
    p = W.make_prefill_case([4, 11], 4, 2, 8, 4, W.BF16, 48)
    last = p.cu_seqlens[1:] - 1
    a = orc.gqa_varlen_prefill(p.q, p.k, p.v, p.cu_seqlens, p.scale, causal=True, rows=last)
    b = orc.gqa_varlen_prefill(p.q, p.k, p.v, p.cu_seqlens, p.scale, causal=False, rows=last)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# paged write and gather
# ---------------------------------------------------------------------------

def pin_write_gather_roundtrip(orc):
    for lens, hq, hkv, d, bs, dt, seed in DECODE_SWEEP:
        c = W.make_decode_case(lens, hq, hkv, d, bs, dt, seed)
        kc, vc = fill_pages(orc, c)
        k2, v2 = orc.paged_kv_gather(kc, vc, c.block_table, c.context_lens)
        assert k2.tobytes() == c.k.tobytes() and v2.tobytes() == c.v.tobytes(), "gather(write(K)) != K"
        # every slot not covered by a valid position keeps the sentinel
        used = np.zeros((c.num_blocks, c.block_size), dtype=bool)
        for b, n in enumerate(c.context_lens):
            for pos in range(int(n)):
                used[c.block_table[b, pos // bs], pos % bs] = True
        sentinel = W.nan_pool(1, 1, 1, 1, dt).reshape(-1)[0]
        kbits = kc.view(np.uint16 if dt == W.BF16 else np.uint32)
        sbits = np.asarray(sentinel).view(kbits.dtype)
        assert np.all(kbits.transpose(0, 2, 1, 3)[~used] == sbits), "an unused slot was written"
        assert not np.any(np.isnan(f64(k2)))


def pin_write_chunks_equal_one_write(orc):
    """Writing tokens in two chunks (second chunk at start_pos = first chunk's length) equals one write."""
    c = W.make_decode_case([10, 23, 5], 4, 2, 8, 4, W.BF16, 51)
    kc1, vc1 = fill_pages(orc, c)
    kc2 = W.nan_pool(c.num_blocks, 2, 4, 8, c.dtype)
    vc2 = W.nan_pool(c.num_blocks, 2, 4, 8, c.dtype)
    first = np.array([3, 11, 5], dtype=np.int32)
    second = c.context_lens - first
    k1, v1, k2, v2 = [], [], [], []
    for b in range(c.batch):
        a = int(c.cu_ctx[b])
        k1.append(c.k[a:a + first[b]]); v1.append(c.v[a:a + first[b]])
        k2.append(c.k[a + first[b]:c.cu_ctx[b + 1]]); v2.append(c.v[a + first[b]:c.cu_ctx[b + 1]])
    orc.paged_kv_write(np.concatenate(k1), np.concatenate(v1), W.cu_from_lengths(first),
                       np.zeros(3, np.int32), c.block_table, kc2, vc2)
    orc.paged_kv_write(np.concatenate(k2), np.concatenate(v2), W.cu_from_lengths(second),
                       first, c.block_table, kc2, vc2)
    assert kc1.tobytes() == kc2.tobytes() and vc1.tobytes() == vc2.tobytes()


def pin_copy_blocks_moves_pages(orc):
    """A block copy makes the destination pages read back (by the independent
    gather) exactly as the source pages did, and leaves every other block alone."""
    c = W.make_decode_case([13, 9, 20], 4, 2, 8, 4, W.BF16, 61)
    kc, vc = fill_pages(orc, c)
    used = set(int(x) for x in c.block_table.reshape(-1) if x >= 0)
    spare = [b for b in range(c.num_blocks) if b not in used]
    src = np.array([c.block_table[0, 1], c.block_table[2, 4]], dtype=np.int32)   # a full page and a partial one
    dst = np.array(spare[:2], dtype=np.int32)
    k0, v0 = kc.copy(), vc.copy()
    orc.paged_kv_copy_blocks(kc, vc, src, dst)
    moved = c.block_table.copy()
    moved[0, 1], moved[2, 4] = dst
    ka, va = orc.paged_kv_gather(k0, v0, c.block_table, c.context_lens)
    kb, vb = orc.paged_kv_gather(kc, vc, moved, c.context_lens)
    assert ka.tobytes() == kb.tobytes() and va.tobytes() == vb.tobytes(), "copied pages read back differently"
    other = np.ones(c.num_blocks, dtype=bool)
    other[dst] = False
    assert kc[other].tobytes() == k0[other].tobytes() and vc[other].tobytes() == v0[other].tobytes()
    # whole blocks move, tail slots (past the context) included
    assert kc[dst].tobytes() == k0[src].tobytes() and vc[dst].tobytes() == v0[src].tobytes()


def pin_copy_blocks_in_order(orc):
    """Pairs apply in order: a -> b then b -> c leaves a's contents in c."""
    kc = W.f32_to_bf16_bits(np.random.default_rng(62).standard_normal((5, 2, 4, 8)).astype(np.float32))
    vc = W.f32_to_bf16_bits(np.random.default_rng(63).standard_normal((5, 2, 4, 8)).astype(np.float32))
    k0, v0 = kc.copy(), vc.copy()
    orc.paged_kv_copy_blocks(kc, vc, np.array([0, 1], np.int32), np.array([1, 2], np.int32))
    assert kc[2].tobytes() == k0[0].tobytes() and kc[1].tobytes() == k0[0].tobytes()
    assert vc[2].tobytes() == v0[0].tobytes() and kc[3:].tobytes() == k0[3:].tobytes()


def _model_check(m, content, expect):
    """Invariants of refcounted paging after any operation, against a token-level
    simulation of the pool: counters equal references, free blocks are unreferenced,
    no table holds a block twice, and every sequence reads back its own tokens."""
    refs = np.zeros(m.num_blocks, dtype=np.int64)
    for sid, table in m.tables.items():
        assert len(set(table)) == len(table), "a table holds a block twice"
        assert len(table) == -(-m.lengths[sid] // m.block_size), "table length != pages of the sequence"
        for b in table:
            refs[b] += 1
        got = [content[table[p // m.block_size]][p % m.block_size] for p in range(m.lengths[sid])]
        assert got == expect[sid], f"sequence {sid} reads back other tokens"
    assert list(refs) == list(m.ref), "reference counters != references"


def pin_block_model_invariants(orc):
    """Random fork / append / free sequences against a token-level simulation in
    which the reported copies and every written slot are applied to a pool of labels."""
    import random
    from oracle.block_model import BlockModel, OutOfBlocks
    for trial in range(40):
        rnd = random.Random(trial)
        bs = rnd.choice([1, 2, 4, 16])
        m = BlockModel(rnd.randint(8, 40), bs)
        content = [[None] * bs for _ in range(m.num_blocks)]
        expect = {}
        label = 0
        for _ in range(120):
            op = rnd.random()
            live = sorted(m.tables)
            if op < 0.15 or not live:
                sid = m.new_sequence()
                expect[sid] = []
            elif op < 0.35:
                parent = rnd.choice(live)
                sid = m.fork(parent)
                expect[sid] = list(expect[parent])
            elif op < 0.85:
                sid = rnd.choice(live)
                n = rnd.randint(0, 2 * bs + 1)
                try:
                    cp = m.append(sid, n)
                except OutOfBlocks:
                    _model_check(m, content, expect)
                    continue
                if cp is not None:
                    content[cp[1]] = list(content[cp[0]])
                start = m.lengths[sid] - n
                for pos in range(start, start + n):
                    content[m.tables[sid][pos // bs]][pos % bs] = label
                    expect[sid].append(label)
                    label += 1
            else:
                sid = rnd.choice(live)
                m.free(sid)
                del expect[sid]
            _model_check(m, content, expect)


def pin_block_model_shared_prompt(orc):
    """The pages' scenario: a system prompt shared by 50 requests is stored once; each
    request that diverges copies only the block it modifies (the prompt's partly
    filled last block), and the full prompt blocks stay shared by all."""
    from oracle.block_model import BlockModel
    bs, prompt = 16, 100                  # 6 full blocks + 4 tokens in a 7th
    m = BlockModel(200, bs)
    root = m.new_sequence()
    assert m.append(root, prompt) is None
    kids = [m.fork(root) for _ in range(50)]
    assert len(m.free_blocks()) == 200 - 7, "the prompt is stored once"
    assert all(m.ref[b] == 51 for b in m.tables[root])
    copies = [m.append(k, 3) for k in kids]            # 3 new tokens each, inside the 7th block
    assert all(cp is not None and cp[0] == m.tables[root][6] for cp in copies)
    assert len({cp[1] for cp in copies}) == 50
    assert all(m.ref[b] == 51 for b in m.tables[root][:6]), "full prompt blocks stay shared"
    assert m.ref[m.tables[root][6]] == 1
    assert m.append(root, 1) is None, "the last holder writes in place"
    assert len(m.free_blocks()) == 200 - 7 - 50
    for k in kids:
        m.free(k)
    m.free(root)
    assert len(m.free_blocks()) == 200 and all(r == 0 for r in m.ref)


def pin_window_decode_is_truncated_context(orc):
    """Local attention in decode equals plain decode over a context that holds only
    the newest `window` tokens (rebuilt from the packed rows, fresh placement)."""
    c = W.make_decode_case([9, 1, 30, 17], 4, 2, 16, 4, W.F32, 71)
    kc, vc = fill_pages(orc, c)
    for win in (1, 3, 8, 17, 40):
        got = orc.gqa_paged_decode(c.q, kc, vc, c.block_table, c.context_lens, c.scale, window=win)
        keep = np.minimum(c.context_lens, win).astype(np.int32)
        rows = np.concatenate([np.arange(c.cu_ctx[b + 1] - keep[b], c.cu_ctx[b + 1]) for b in range(c.batch)])
        t = W.DecodeCase(name="t", dtype=c.dtype, num_q_heads=4, num_kv_heads=2, head_dim=16, block_size=4,
                         context_lens=keep, cu_ctx=W.cu_from_lengths(keep), q=c.q, k=c.k[rows], v=c.v[rows],
                         block_table=W.place_pages(np.random.default_rng(win), keep, 4)[0],
                         num_blocks=W.place_pages(np.random.default_rng(win), keep, 4)[1], scale=c.scale)
        close(got, decode(orc, t), rel=1e-12, what=f"window {win}")


def pin_window_one_returns_own_value(orc):
    """window = 1: every query sees only its own position, so the output is that value row."""
    c = W.make_decode_case([5, 12], 4, 2, 16, 4, W.BF16, 72)
    kc, vc = fill_pages(orc, c)
    got = orc.gqa_paged_decode(c.q, kc, vc, c.block_table, c.context_lens, c.scale, window=1)
    v = f64(c.v)
    for b in range(c.batch):
        last = int(c.cu_ctx[b + 1]) - 1
        for qh in range(4):
            assert np.array_equal(got[b, qh], v[last, qh // 2])
    p = W.make_prefill_case([6, 3], 4, 2, 8, 4, W.BF16, 73)
    out = orc.gqa_varlen_prefill(p.q, p.k, p.v, p.cu_seqlens, p.scale, window=1)
    pv = f64(p.v)
    for i in range(p.total_tokens):
        for qh in range(4):
            assert np.array_equal(out[i, qh], pv[i, qh // 2])


def _band_sdpa(q, k, v, scale, rows_pos, nkeys, win):
    """Library attention of query rows at positions rows_pos over keys 0..nkeys-1 with
    an explicit mask keeping key j iff pos - win < j <= pos."""
    mask = (np.arange(nkeys)[None, :] <= rows_pos[:, None]) & (np.arange(nkeys)[None, :] > rows_pos[:, None] - win)
    qt = torch.from_numpy(q).permute(1, 0, 2).unsqueeze(0).contiguous()
    kt = torch.from_numpy(k).permute(1, 0, 2).unsqueeze(0).contiguous()
    vt = torch.from_numpy(v).permute(1, 0, 2).unsqueeze(0).contiguous()
    r = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask), scale=float(scale),
                                       enable_gqa=True)
    return r[0].permute(1, 0, 2).numpy()


def pin_window_matches_library(orc):
    """Prefill and multi-token queries with a window against torch SDPA with an explicit band mask."""
    p = W.make_prefill_case([20, 7, 33], 8, 2, 16, 4, W.F32, 74)
    for win in (1, 5, 16, 100):
        got = orc.gqa_varlen_prefill(p.q, p.k, p.v, p.cu_seqlens, p.scale, window=win)
        want = np.zeros_like(got)
        for b in range(p.batch):
            a, e = int(p.cu_seqlens[b]), int(p.cu_seqlens[b + 1])
            want[a:e] = _band_sdpa(f64(p.q[a:e]), f64(p.k[a:e]), f64(p.v[a:e]), p.scale, np.arange(e - a), e - a, win)
        close(got, want, rel=1e-12, what=f"prefill window {win}")
    c = W.make_extend_case([9, 0, 25], [4, 6, 11], 8, 2, 16, 4, W.BF16, 75)
    kc, vc = extend_pages(orc, c)
    for win in (1, 4, 13, 64):
        got = orc.gqa_paged_extend(c.q, c.cu_q, kc, vc, c.block_table, c.context_lens, c.scale, window=win)
        want = np.zeros_like(got)
        for b in range(c.batch):
            qa, qe = int(c.cu_q[b]), int(c.cu_q[b + 1])
            ka, ke = int(c.cu_ctx[b]), int(c.cu_ctx[b + 1])
            pos = (ke - ka) - (qe - qa) + np.arange(qe - qa)
            want[qa:qe] = _band_sdpa(f64(c.q[qa:qe]), f64(c.k[ka:ke]), f64(c.v[ka:ke]), c.scale, pos, ke - ka, win)
        close(got, want, rel=1e-12, what=f"extend window {win}")


def pin_window_weights_outside_are_zero(orc):
    c = W.make_decode_case([30, 4], 4, 2, 16, 4, W.BF16, 76)
    kc, vc = fill_pages(orc, c)
    _, probs = orc.gqa_paged_decode(c.q, kc, vc, c.block_table, c.context_lens, c.scale, want_probs=True,
                                    window=10)
    assert np.all(probs[0, :, :20] == 0) and np.all(probs[0, :, 20:30] > 0)
    assert np.allclose(probs[0].sum(-1), 1.0, rtol=1e-12) and np.allclose(probs[1, :, :4].sum(-1), 1.0, rtol=1e-12)


def _torch_fp8_values(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def pin_fp8_codes(orc):
    """Every E4M3 code against torch's float8_e4m3fn and the format's closed form."""
    codes = np.arange(256, dtype=np.uint8)
    got, ref = orc.fp8_decode(codes), _torch_fp8_values(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2 and np.array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6 and got[0x38] == 1.0
    assert got[0xB8] == -1.0 and got[0x80] == 0.0


def pin_fp8_rounding(orc):
    """Nearest-even encoding against torch's conversion, on random values, every code
    value and every midpoint between neighbouring codes (the ties)."""
    vals = orc.fp8_decode(np.arange(256, dtype=np.uint8))
    fin = np.sort(vals[~np.isnan(vals)])
    x = np.concatenate([np.random.default_rng(77).uniform(-448, 448, 20000), fin, (fin[1:] + fin[:-1]) / 2,
                        np.random.default_rng(78).normal(0, 0.01, 5000)]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(orc.fp8_encode(x), want)


def _fp8_pools(orc, c):
    kc = np.full((c.num_blocks, c.num_kv_heads, c.block_size, c.head_dim), 0x7F, dtype=np.uint8)
    vc = kc.copy()
    ks = np.full((c.num_blocks, c.num_kv_heads, c.block_size), np.nan, dtype=np.float32)
    vs = ks.copy()
    orc.paged_kv_write_fp8(c.k, c.v, c.cu_ctx, c.start_pos, c.block_table, kc, vc, ks, vs)
    return kc, vc, ks, vs


def pin_fp8_write(orc):
    """The quantising write: each row's scale is its largest magnitude over 448 (fp32),
    its codes are torch's nearest-even conversion of x / scale, the values are within
    half a code step of the inputs, and slots no token reaches keep the sentinel."""
    c = W.make_decode_case([9, 30, 4], 4, 2, 16, 4, W.BF16, 79)
    c.k[3, 1] = 0                                   # an all-zero row: scale 1, codes 0
    kc, vc, ks, vs = _fp8_pools(orc, c)
    x = {"k": f64(c.k).astype(np.float32), "v": f64(c.v).astype(np.float32)}
    used = np.zeros((c.num_blocks, c.block_size), dtype=bool)
    for b in range(c.batch):
        for pos in range(int(c.context_lens[b])):
            t = int(c.cu_ctx[b]) + pos
            blk, slot = c.block_table[b, pos // 4], pos % 4
            used[blk, slot] = True
            for h in range(2):
                for name, codes, scales in (("k", kc, ks), ("v", vc, vs)):
                    row = x[name][t, h]
                    amax = np.float32(np.abs(row).max())
                    sc = amax / np.float32(448.0) if amax > 0 else np.float32(1.0)
                    assert scales[blk, h, slot] == sc
                    y = np.clip(row / sc, np.float32(-448), np.float32(448)).astype(np.float32)
                    want = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
                    assert np.array_equal(codes[blk, h, slot], want)
                    deq = _torch_fp8_values(codes[blk, h, slot]) * float(sc)
                    bound = np.maximum(2.0 ** -4 * np.abs(row), 2.0 ** -10 * float(sc)) * (1 + 1e-6)
                    assert np.all(np.abs(deq - row) <= bound)
    assert np.all(kc.transpose(0, 2, 1, 3)[~used] == 0x7F) and np.all(np.isnan(ks.transpose(0, 2, 1)[~used]))
    assert ks[c.block_table[0, 0], 1, 3] == 1.0 and not kc[c.block_table[0, 0], 1, 3].any()


def pin_fp8_decode_is_attention_over_dequantized(orc):
    """Decode over fp8 pages = attention over the values code * scale, here rebuilt
    with torch's fp8 conversion and checked against SDPA on dense K/V."""
    c = W.make_decode_case([13, 1, 40], 8, 2, 16, 4, W.BF16, 80)
    kc, vc, ks, vs = _fp8_pools(orc, c)
    got = orc.gqa_paged_decode(f64(c.q), orc.dequantize_fp8(kc, ks), orc.dequantize_fp8(vc, vs), c.block_table,
                               c.context_lens, c.scale)
    q = f64(c.q)
    for b in range(c.batch):
        n = int(c.context_lens[b])
        kk = np.zeros((n, 2, 16))
        vv = np.zeros((n, 2, 16))
        for pos in range(n):
            blk, slot = c.block_table[b, pos // 4], pos % 4
            kk[pos] = _torch_fp8_values(kc[blk, :, slot]) * ks[blk, :, slot, None].astype(np.float64)
            vv[pos] = _torch_fp8_values(vc[blk, :, slot]) * vs[blk, :, slot, None].astype(np.float64)
        r = F.scaled_dot_product_attention(torch.from_numpy(q[b][:, None]), torch.from_numpy(kk.transpose(1, 0, 2).copy()),
                                           torch.from_numpy(vv.transpose(1, 0, 2).copy()), scale=float(c.scale),
                                           enable_gqa=True)
        close(got[b], r[:, 0].numpy(), rel=1e-12, what=f"fp8 decode seq {b}")


def extend_pages(orc, case: W.ExtendCase):
    kc = W.nan_pool(case.num_blocks, case.num_kv_heads, case.block_size, case.head_dim, case.dtype)
    vc = W.nan_pool(case.num_blocks, case.num_kv_heads, case.block_size, case.head_dim, case.dtype)
    orc.paged_kv_write(case.k, case.v, case.cu_ctx, case.start_pos, case.block_table, kc, vc)
    return kc, vc


def extend(orc, case: W.ExtendCase):
    kc, vc = extend_pages(orc, case)
    return orc.gqa_paged_extend(case.q, case.cu_q, kc, vc, case.block_table, case.context_lens, case.scale)


def sdpa_extend(case: W.ExtendCase) -> np.ndarray:
    """Library attention per sequence: its query rows against its packed K/V with
    an explicit boolean mask keeping key j for row i iff j <= ctx - q_len + i."""
    q, k, v = f64(case.q), f64(case.k), f64(case.v)
    out = np.zeros_like(q)
    for b in range(case.batch):
        qa, qe = int(case.cu_q[b]), int(case.cu_q[b + 1])
        ka, ke = int(case.cu_ctx[b]), int(case.cu_ctx[b + 1])
        if qe == qa:
            continue
        n, ctx = qe - qa, ke - ka
        mask = np.arange(ctx)[None, :] <= (ctx - n + np.arange(n))[:, None]
        qt = torch.from_numpy(q[qa:qe]).permute(1, 0, 2).unsqueeze(0).contiguous()
        kt = torch.from_numpy(k[ka:ke]).permute(1, 0, 2).unsqueeze(0).contiguous()
        vt = torch.from_numpy(v[ka:ke]).permute(1, 0, 2).unsqueeze(0).contiguous()
        r = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask), scale=float(case.scale),
                                           enable_gqa=True)
        out[qa:qe] = r[0].permute(1, 0, 2).numpy()
    return out


def pin_fp8_extend_is_attention_over_dequantized(orc):
    """Multi-token queries over fp8 pages = attention over the values code * scale:
    the oracle over its dequantised pools against SDPA with a bottom-right mask on
    dense K/V rebuilt with torch's fp8 conversion."""
    c = W.make_extend_case([0, 7, 40, 3], [5, 1, 9, 16], 8, 2, 16, 4, W.BF16, 89)
    kc, vc, ks, vs = _fp8_pools(orc, c)
    got = orc.gqa_paged_extend(f64(c.q), c.cu_q, orc.dequantize_fp8(kc, ks), orc.dequantize_fp8(vc, vs),
                               c.block_table, c.context_lens, c.scale)
    q = f64(c.q)
    for b in range(c.batch):
        qa, qe = int(c.cu_q[b]), int(c.cu_q[b + 1])
        n, ctx = qe - qa, int(c.context_lens[b])
        kk = np.zeros((ctx, 2, 16))
        vv = np.zeros((ctx, 2, 16))
        for pos in range(ctx):
            blk, slot = c.block_table[b, pos // 4], pos % 4
            kk[pos] = _torch_fp8_values(kc[blk, :, slot]) * ks[blk, :, slot, None].astype(np.float64)
            vv[pos] = _torch_fp8_values(vc[blk, :, slot]) * vs[blk, :, slot, None].astype(np.float64)
        mask = np.arange(ctx)[None, :] <= (ctx - n + np.arange(n))[:, None]
        r = F.scaled_dot_product_attention(torch.from_numpy(q[qa:qe]).permute(1, 0, 2).unsqueeze(0).contiguous(),
                                           torch.from_numpy(kk.transpose(1, 0, 2).copy()).unsqueeze(0),
                                           torch.from_numpy(vv.transpose(1, 0, 2).copy()).unsqueeze(0),
                                           attn_mask=torch.from_numpy(mask), scale=float(c.scale), enable_gqa=True)
        close(got[qa:qe], r[0].permute(1, 0, 2).numpy(), rel=1e-12, what=f"fp8 extend seq {b}")


def pin_extend_matches_library(orc):
    for dt, seed in ((W.F32, 81), (W.BF16, 82)):
        c = W.make_extend_case([0, 7, 40, 3, 100], [5, 1, 9, 16, 2], 8, 2, 16, 4, dt, seed)
        close(extend(orc, c), sdpa_extend(c), what=f"extend vs SDPA {dt}")


def pin_extend_single_token_is_decode(orc):
    """One query token per sequence is a decode step (same keys, same order)."""
    c = W.make_extend_case([4, 0, 37, 12], [1, 1, 1, 1], 8, 4, 16, 4, W.F32, 83)
    d = W.make_decode_case(c.context_lens, 8, 4, 16, 4, W.F32, 84)
    d.q, d.k, d.v, d.block_table, d.num_blocks = c.q, c.k, c.v, c.block_table, c.num_blocks
    close(extend(orc, c), decode(orc, d), rel=0.0, what="extend q_len=1 vs decode")


def pin_extend_without_prefix_is_causal_prefill(orc):
    """No cached prefix: the rows are exactly a causal varlen prefill of the new tokens."""
    c = W.make_extend_case([0, 0, 0], [6, 1, 13], 8, 2, 16, 4, W.F32, 85)
    p = W.make_prefill_case(c.q_lens, 8, 2, 16, 4, W.F32, 86)
    p.q, p.k, p.v = c.q, c.k, c.v
    close(extend(orc, c), orc.gqa_varlen_prefill(p.q, p.k, p.v, p.cu_seqlens, c.scale, causal=True),
          what="extend without prefix vs causal prefill")


def pin_extend_rows_shift_with_prefix(orc):
    """Bottom-right alignment: the last row of every sequence sees its whole
    context, and the first row sees exactly the prefix plus itself (brute force)."""
    c = W.make_extend_case([9, 2, 30], [4, 7, 3], 4, 2, 16, 4, W.F32, 87)
    got = extend(orc, c)
    q, k, v = f64(c.q), f64(c.k), f64(c.v)
    G = c.num_q_heads // c.num_kv_heads
    for b in range(c.batch):
        ka = int(c.cu_ctx[b])
        ctx, n = int(c.context_lens[b]), int(c.q_lens[b])
        for i in (0, n - 1):
            r = int(c.cu_q[b]) + i
            keys = ctx - n + i + 1
            for qh in range(c.num_q_heads):
                h = qh // G
                s = (k[ka:ka + keys, h] @ q[r, qh]) * float(c.scale)
                w = np.exp(s - s.max())
                close(got[r, qh], (w / w.sum()) @ v[ka:ka + keys, h], rel=1e-12, what=f"extend b{b} row{i}")


def pin_extend_row_sampling(orc):
    """Sampled rows (any order, repeats) equal the same rows of the full evaluation,
    and each equals the library attention of its sequence."""
    c = W.make_extend_case([11, 0, 6], [5, 3, 9], 4, 2, 16, 4, W.BF16, 88)
    kc, vc = extend_pages(orc, c)
    full = orc.gqa_paged_extend(c.q, c.cu_q, kc, vc, c.block_table, c.context_lens, c.scale)
    rows = np.array([16, 0, 4, 5, 8, 7, 0], dtype=np.int32)
    part = orc.gqa_paged_extend(c.q, c.cu_q, kc, vc, c.block_table, c.context_lens, c.scale, rows=rows)
    assert np.array_equal(part, full[rows]), "sampled rows differ from the full evaluation"
    close(part, sdpa_extend(c)[rows], rel=1e-12, what="sampled extend rows vs library")


def pin_contract_errors(orc):
    c = W.make_decode_case([5, 11], 4, 2, 16, 4, W.F32, 52)
    kc, vc = fill_pages(orc, c)
    bad = c.block_table.copy()
    bad[1, 2] = c.num_blocks          # outside the pool
    try:
        orc.gqa_paged_decode(c.q, kc, vc, bad, c.context_lens, c.scale)
        raise AssertionError("out-of-pool block id not reported")
    except OracleError as e:
        assert str(ERANGE) in str(e)
    try:
        orc.gqa_paged_decode(c.q[:, :3], kc, vc, c.block_table, c.context_lens, c.scale)
        raise AssertionError("Hq % Hkv != 0 not reported")
    except OracleError as e:
        assert str(EINVAL) in str(e)
    p = W.make_prefill_case([4], 4, 2, 8, 4, W.F32, 53)
    try:
        orc.gqa_varlen_prefill(p.q, p.k, p.v, p.cu_seqlens, p.scale, causal=False, window=2)
        raise AssertionError("a window without the causal mask not reported")
    except OracleError as e:
        assert str(EINVAL) in str(e)


def pin_zero_scale_gives_mean(orc):
    """scale = 0 makes every score 0: each output is the plain mean of the values its
    row sees (decode: the whole context; causal prefill: the prefix up to the row)."""
    c = W.make_decode_case([7, 19, 1], 8, 2, 16, 4, W.F32, 37, scale=0.0)
    out = decode(orc, c)
    G = c.num_q_heads // c.num_kv_heads
    v = f64(c.v)
    for b in range(c.batch):
        a, e = c.cu_ctx[b], c.cu_ctx[b + 1]
        close(out[b], np.repeat(v[a:e].mean(axis=0), G, axis=0), rel=1e-14, what="zero-scale decode")
    p = W.make_prefill_case([5, 12], 4, 2, 8, 4, W.F32, 38, scale=0.0)
    pre = orc.gqa_varlen_prefill(p.q, p.k, p.v, p.cu_seqlens, 0.0, causal=True)
    vv = f64(p.v)
    for s_ in range(p.batch):
        a, e = int(p.cu_seqlens[s_]), int(p.cu_seqlens[s_ + 1])
        for i in range(a, e):
            close(pre[i], np.repeat(vv[a:i + 1].mean(axis=0), 2, axis=0), rel=1e-14, what="zero-scale prefill")


def pin_negative_scale_matches_library(orc):
    """A negative scale is an ordinary softmax of scale * q.k.  The library routine
    takes the square root of its scale, so it is asked for the same scores written
    as |scale| * (-q).k (negating a bf16 query flips its sign bit: exact)."""
    def flipped(case):
        import copy
        g = copy.copy(case)
        g.q = case.q ^ np.uint16(0x8000)
        g.scale = -case.scale
        return g
    for lens, hq, hkv, d, seed in [([9, 33], 8, 2, 16, 39), ([1, 70], 4, 4, 32, 40)]:
        c = W.make_decode_case(lens, hq, hkv, d, 4, W.BF16, seed, scale=-0.75)
        close(decode(orc, c), sdpa_decode(flipped(c)), what="negative-scale decode")
    p = W.make_prefill_case([6, 31], 8, 2, 16, 4, W.BF16, 41, scale=-0.4)
    for causal in (True, False):
        close(orc.gqa_varlen_prefill(p.q, p.k, p.v, p.cu_seqlens, p.scale, causal=causal),
              sdpa_prefill(flipped(p), causal), what="negative-scale prefill")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
