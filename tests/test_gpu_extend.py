"""Multi-token queries over the paged cache (chunked prefill on a cached prefix,
draft verification) on the GPU against the fp64 oracle."""

import numpy as np
import pytest
import torch

import workload as W
import paged_gqa_kv_02_amd as pg
from gpu_helpers import DevDecode, DevExtend, assert_close, oracle_extend, say, to_dev, to_f64

pytestmark = pytest.mark.gpu

PREFIX = [0, 1, 31, 64, 100, 7, 250]
QLENS = [1, 33, 64, 5, 129, 40, 16]


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 4), (8, 2), (32, 8), (16, 1), (64, 1)])
@pytest.mark.parametrize("d", [64, 128])
def test_shapes(orc, hq, hkv, d):
    c = W.make_extend_case(PREFIX, QLENS, hq, hkv, d, 16, W.BF16, seed=700 + hq * 10 + hkv + d)
    say(f"extend shape {hq}/{hkv} d{d}")
    out = to_f64(DevExtend(c).extend())
    assert_close(out, oracle_extend(orc, c), W.BF16, f"extend {hq}/{hkv} d{d}")


@pytest.mark.parametrize("d,bs", [(128, 4), (128, 8), (128, 16), (128, 32), (128, 64), (128, 128), (128, 256),
                                  (64, 8), (64, 16), (64, 256)])
def test_block_sizes(orc, d, bs):
    c = W.make_extend_case([0, bs - 1, bs, 3 * bs + 1, 70], [bs + 1, 1, 2 * bs, 64, 97], 8, 2, d, bs, W.BF16,
                           seed=800 + bs + d)
    say(f"extend bs{bs} d{d}")
    out = to_f64(DevExtend(c).extend())
    assert_close(out, oracle_extend(orc, c), W.BF16, f"extend bs{bs} d{d}")


def test_single_token_equals_decode(orc):
    """q_len = 1 everywhere: the decode phase (same cache, same queries)."""
    c = W.make_extend_case([0, 15, 16, 300, 1000, 2047], [1] * 6, 32, 8, 128, 16, W.BF16, seed=810)
    say("extend q_len=1 vs decode")
    dev = DevExtend(c)
    ext = to_f64(dev.extend())
    dc = W.DecodeCase(name="x", dtype=W.BF16, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                      context_lens=c.context_lens, cu_ctx=c.cu_ctx, q=c.q, k=c.k, v=c.v,
                      block_table=c.block_table, num_blocks=c.num_blocks, scale=c.scale)
    dec = to_f64(DevDecode(dc).decode())
    ref = oracle_extend(orc, c)
    assert_close(ext, ref, W.BF16, "extend q_len=1")
    assert_close(dec, ref, W.BF16, "decode")


def test_no_prefix_equals_causal_prefill(orc):
    """ctx = q_len: a causal prefill; the paged kernel reads the same keys in the same
    tiles as the packed one, so the two agree bit for bit."""
    lens = [1, 31, 32, 33, 100, 257, 64]
    c = W.make_extend_case([0] * len(lens), lens, 32, 8, 128, 16, W.BF16, seed=811)
    say("extend without prefix vs prefill")
    ext = DevExtend(c).extend()
    pre = pg.gqa_varlen_prefill(to_dev(c.q), to_dev(c.k), to_dev(c.v), to_dev(c.cu_q), c.max_q_len,
                                scale=float(c.scale))
    torch.cuda.synchronize()
    assert torch.equal(ext.view(torch.int16), pre.view(torch.int16))
    assert_close(to_f64(ext), oracle_extend(orc, c), W.BF16, "extend without prefix")


def test_chunked_prompt_equals_one_prefill(orc):
    """A prompt processed in chunks (write the chunk's K/V at its position, then
    attend over prefix + chunk) gives the rows a single causal prefill gives."""
    rng = np.random.default_rng(812)
    hq, hkv, d, bs = 32, 8, 128, 16
    lens = np.array([700, 129, 1030], dtype=np.int32)
    p = W.make_prefill_case(lens, hq, hkv, d, bs, W.BF16, seed=812)
    table = to_dev(p.block_table)
    kc = torch.zeros((p.num_blocks, hkv, bs, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    q, k, v = to_dev(p.q), to_dev(p.k), to_dev(p.v)
    out = torch.empty_like(q)
    done = np.zeros(len(lens), dtype=np.int32)
    chunk = 256
    say("extend chunked prompt")
    while (done < lens).any():
        n = np.minimum(lens - done, chunk).astype(np.int32)
        n = np.where(rng.random(len(lens)) < 0.3, np.minimum(n, 1 + rng.integers(0, 64, len(lens))), n)
        n = n.astype(np.int32)
        rows = np.concatenate([np.arange(p.cu_seqlens[b] + done[b], p.cu_seqlens[b] + done[b] + n[b])
                               for b in range(len(lens))]).astype(np.int64)
        ridx = torch.from_numpy(rows).cuda()
        cu = to_dev(W.cu_from_lengths(n))
        pg.paged_kv_write(k[ridx].contiguous(), v[ridx].contiguous(), cu, to_dev(done.copy()), table, kc, vc)
        ctx = (done + n).astype(np.int32)
        o = pg.gqa_paged_extend(q[ridx].contiguous(), cu, kc, vc, table, to_dev(ctx), int(n.max()),
                                int(ctx.max()), scale=float(p.scale))
        out[ridx] = o
        done = ctx
    torch.cuda.synchronize()
    pre = pg.gqa_varlen_prefill(q, k, v, to_dev(p.cu_seqlens), p.max_seqlen, scale=float(p.scale))
    ref = orc.gqa_varlen_prefill(p.q, p.k, p.v, p.cu_seqlens, p.scale)
    assert_close(to_f64(out), ref, W.BF16, "chunked prompt")
    assert_close(to_f64(pre), ref, W.BF16, "one prefill")


def test_edges(orc):
    """Empty sequences (q_len 0), a sequence whose context is shorter than its
    query count (rows with no key give 0), and one with no context at all."""
    c = W.make_extend_case([5, 0, 40, 3, 0, 16], [0, 0, 70, 9, 4, 33], 8, 2, 128, 16, W.BF16, seed=813)
    ctx = c.context_lens.copy()
    ctx[3] = 4        # 9 query rows, 4 cached positions: rows 0..4 see nothing
    ctx[4] = 0        # 4 query rows, no cache
    say("extend edges")
    out = to_f64(DevExtend(c, context_lens=ctx).extend())
    ref = oracle_extend(orc, c, context_lens=ctx)
    qa = int(c.cu_q[3])
    assert (ref[qa:qa + 5] == 0).all() and (ref[int(c.cu_q[4]):int(c.cu_q[5])] == 0).all()
    assert (out[qa:qa + 5] == 0).all() and (out[int(c.cu_q[4]):int(c.cu_q[5])] == 0).all()
    assert_close(out, ref, W.BF16, "extend edges")


def test_sharpened_queries(orc):
    """q x 4 (exact in bf16): peaked softmax, O(1) outputs, so a misplaced mask shows."""
    c = W.make_extend_case([10, 200, 63], [100, 17, 65], 32, 8, 128, 16, W.BF16, seed=814)
    c.q = W.f32_to_bf16_bits(W.bf16_bits_to_f32(c.q) * np.float32(4.0))
    say("extend sharpened")
    out = to_f64(DevExtend(c).extend())
    ref = oracle_extend(orc, c)
    assert np.abs(ref).max() > 0.5
    assert_close(out, ref, W.BF16, "extend sharpened")


@pytest.mark.parametrize("key", ["chunked_prefill", "spec_verify"])
def test_workload_every_output(orc, key):
    """The full multi-token workloads in the benchmark's launch configuration,
    every output element against the oracle."""
    c = W.make_workload(key)
    say(f"extend workload {key} B={c.batch} total_q={c.total_q}")
    out = to_f64(DevExtend(c).extend())
    torch.cuda.synchronize()
    e = assert_close(out, oracle_extend(orc, c), W.BF16, key)
    say(f"extend {key}: {e}")


@pytest.mark.parametrize("q_len,window,hq,hkv", [(4, 0, 32, 8), (1, 0, 32, 8), (40, 0, 32, 8), (7, 300, 8, 2),
                                                 (4, 0, 64, 1), (33, 1000, 16, 4)])
def test_key_split(orc, q_len, window, hq, hkv):
    """Few query tokens over long contexts: the library splits key ranges into
    chunks (fp32 partials + merge).  Checked against the oracle, and against the
    same call with no workspace (no split)."""
    prefix = [3000, 17, 1024 - q_len, 1025 - q_len, 2048, 4000, 64, 2500]
    hkv_pairs = hkv if hkv <= 2 else 2           # few (sequence, KV head) pairs, so the call splits
    hq = hq // hkv * hkv_pairs
    hkv = hkv_pairs
    c = W.make_extend_case(prefix, [q_len] * len(prefix), hq, hkv, 128, 16, W.BF16, seed=900 + q_len + window + hq)
    n = pg.gqa_paged_extend_workspace_size(c.batch, c.total_q, c.max_q_len, hq, hkv, 128, c.max_context_len)
    assert n > 0, "this shape is meant to split"
    say(f"extend key split q_len={q_len} window={window} {hq}/{hkv}")
    dev = DevExtend(c)
    args = (dev.q, dev.cu_q, dev.kc, dev.vc, dev.table, dev.ctx, c.max_q_len, c.max_context_len)
    split = pg.gqa_paged_extend(*args, scale=float(c.scale), window=window)
    plain = pg.gqa_paged_extend(*args, scale=float(c.scale), window=window,
                                workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    kc = W.nan_pool(c.num_blocks, c.num_kv_heads, c.block_size, c.head_dim, c.dtype)
    vc = W.nan_pool(c.num_blocks, c.num_kv_heads, c.block_size, c.head_dim, c.dtype)
    orc.paged_kv_write(c.k, c.v, c.cu_ctx, c.start_pos, c.block_table, kc, vc)
    ref = orc.gqa_paged_extend(c.q, c.cu_q, kc, vc, c.block_table, c.context_lens, c.scale, window=window)
    assert_close(to_f64(split), ref, W.BF16, "split")
    assert_close(to_f64(plain), ref, W.BF16, "no split")


@pytest.mark.parametrize("q_len", [3, 37])
@pytest.mark.parametrize("hq,hkv,d", [(1, 1, 128), (1, 1, 64), (2, 1, 64), (2, 2, 64)])
def test_key_split_short_rows(orc, q_len, hq, hkv, d):
    """Key split where a query row has 64 or 128 outputs (Hq x d), so one merge
    workgroup takes 2 or 4 rows; odd query lengths make those rows belong to
    different sequences."""
    prefix = [3000, 17, 1024 - q_len, 1025 - q_len, 2048, 4000, 64, 2500, 0, 7000]
    c = W.make_extend_case(prefix, [q_len] * len(prefix), hq, hkv, d, 16, W.BF16, seed=970 + q_len + hq + d)
    n = pg.gqa_paged_extend_workspace_size(c.batch, c.total_q, c.max_q_len, hq, hkv, d, c.max_context_len)
    assert n > 0, "this shape is meant to split"
    say(f"extend key split, short rows: q_len={q_len} {hq}/{hkv} d={d}")
    dev = DevExtend(c)
    out = to_f64(dev.extend())
    assert_close(out, oracle_extend(orc, c), W.BF16, f"short rows {hq}/{hkv} d{d}")


def test_key_split_is_deterministic():
    c = W.make_extend_case([32000, 9000, 20000, 100], [4] * 4, 64, 8, 128, 16, W.BF16, seed=950)
    assert pg.gqa_paged_extend_workspace_size(c.batch, c.total_q, c.max_q_len, 64, 8, 128, c.max_context_len) > 0
    dev = DevExtend(c)
    say("extend key split twice")
    a = dev.extend()
    b = dev.extend()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("hq,hkv,qlens,window", [
    (32, 8, [4, 1, 3, 4, 2, 4], 0),      # 4 tokens x 4 heads: 16 packed rows
    (64, 8, [4, 4, 1, 3, 4, 2], 0),      # 4 x 8 = 32 rows, a full tile
    (32, 2, [2, 1, 2, 2, 2, 1], 37),     # 2 x 16 rows, window inside the first block
    (32, 1, [1, 1, 1, 1, 1, 1], 0),      # 32 heads of one token
    (2, 1, [16, 9, 16, 1, 5, 16], 300),  # 16 x 2 rows, causal across many tokens
    (8, 8, [32, 17, 32, 32, 1, 8], 0),   # one head per KV head: 32 tokens
    (8, 8, [33, 17, 32, 32, 1, 8], 0),   # 33 tokens: not packed
    (24, 2, [2, 1, 2, 2, 1, 2], 0),      # G = 12: 24 rows, heads not a power of two
    (24, 1, [1, 1, 1, 1, 1, 1], 100),    # G = 24, one token
    (40, 2, [1, 1, 1, 1, 1, 1], 0),      # G = 20
])
def test_packed_rows(orc, hq, hkv, qlens, window):
    """Calls whose query tokens times the group fit one 32-row tile run on the
    packed-rows kernel (rows = (token, head) pairs; up to 16 rows two waves split
    each key block, past 16 all four waves compute, 16 rows by a key half each):
    ragged token counts, causal masks between the packed tokens, windows, and
    long contexts that split into key chunks."""
    prefix = [3000, 0, 61, 64, 1500, 127 - qlens[5]]
    c = W.make_extend_case(prefix, qlens, hq, hkv, 128, 16, W.BF16, seed=990 + hq + hkv + sum(qlens) + window)
    say(f"extend packed rows {hq}/{hkv} q_lens {qlens} window {window}")
    dev = DevExtend(c)
    out = to_f64(pg.gqa_paged_extend(dev.q, dev.cu_q, dev.kc, dev.vc, dev.table, dev.ctx, c.max_q_len,
                                     c.max_context_len, scale=float(c.scale), window=window))
    assert_close(out, oracle_extend(orc, c, window=window), W.BF16, f"packed {hq}/{hkv}")
    plain = to_f64(pg.gqa_paged_extend(dev.q, dev.cu_q, dev.kc, dev.vc, dev.table, dev.ctx, c.max_q_len,
                                       c.max_context_len, scale=float(c.scale), window=window,
                                       workspace=torch.empty(16, dtype=torch.uint8, device="cuda")))
    assert_close(plain, oracle_extend(orc, c, window=window), W.BF16, f"packed {hq}/{hkv}, no split")
