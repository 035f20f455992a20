"""Local attention (sliding window) on the GPU against the fp64 oracle: decode,
packed prefill and multi-token queries with a window, including block tables
whose pages before the window have been released."""

import numpy as np
import pytest
import torch

import workload as W
import paged_gqa_kv_02_amd as pg
from gpu_helpers import DevDecode, DevExtend, assert_close, oracle_extend, oracle_pools, say, to_dev, to_f64

pytestmark = pytest.mark.gpu

LENS = [1, 17, 96, 203, 3, 1000, 2100]


def _oracle_decode(orc, case, window):
    kc, vc = oracle_pools(orc, case)
    return orc.gqa_paged_decode(case.q, kc, vc, case.block_table, case.context_lens, case.scale, window=window)


@pytest.mark.parametrize("window", [1, 7, 32, 100, 256, 5000])
def test_decode_windows(orc, window):
    case = W.make_decode_case(LENS, 32, 8, 128, 16, W.BF16, seed=1000 + window)
    say(f"decode window {window}")
    dev = DevDecode(case)
    out = to_f64(pg.gqa_paged_decode(dev.q, dev.kc, dev.vc, dev.table, dev.ctx, case.max_context_len,
                                     scale=float(case.scale), window=window))
    assert_close(out, _oracle_decode(orc, case, window), W.BF16, f"decode window {window}")


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
@pytest.mark.parametrize("d,bs,hq,hkv", [(128, 1, 8, 2), (64, 16, 16, 1), (32, 256, 4, 4), (128, 8, 64, 1)])
def test_decode_window_shapes(orc, dtype, d, bs, hq, hkv):
    case = W.make_decode_case([5, 40, 333, 64, 65], hq, hkv, d, bs, dtype, seed=1100 + d + bs + hq)
    for window in (3, 64, 100):
        say(f"decode window {window} {dtype} d{d} bs{bs} {hq}/{hkv}")
        dev = DevDecode(case)
        out = to_f64(pg.gqa_paged_decode(dev.q, dev.kc, dev.vc, dev.table, dev.ctx, case.max_context_len,
                                         scale=float(case.scale), window=window))
        assert_close(out, _oracle_decode(orc, case, window), dtype, f"window {window} {dtype} d{d} bs{bs}")


@pytest.mark.parametrize("num_splits", [1, 3, 37, 1000])
def test_decode_window_split_counts(orc, num_splits):
    case = W.make_decode_case(LENS, 32, 8, 128, 16, W.BF16, seed=1200)
    say(f"decode window 300 splits {num_splits}")
    dev = DevDecode(case)
    out = to_f64(pg.gqa_paged_decode(dev.q, dev.kc, dev.vc, dev.table, dev.ctx, case.max_context_len,
                                     scale=float(case.scale), window=300, num_splits=num_splits))
    assert_close(out, _oracle_decode(orc, case, 300), W.BF16, f"splits {num_splits}")


def test_decode_released_pages_are_not_read(orc):
    """Pages wholly before the window released: their table entries point outside
    the pool and the pool blocks hold NaN; the result is unchanged."""
    bs, window = 16, 200
    case = W.make_decode_case([900, 201, 1500, 40], 32, 8, 128, bs, W.BF16, seed=1300)
    dev = DevDecode(case)
    ref = _oracle_decode(orc, case, window)
    table = case.block_table.copy()
    nan_blocks = []
    for b, ctx in enumerate(case.context_lens):
        first_kept_page = max(0, int(ctx) - window) // bs
        nan_blocks += table[b, :first_kept_page].tolist()
        table[b, :first_kept_page] = -1
    say("decode window with released pages")
    kc, vc = dev.kc.clone(), dev.vc.clone()
    if nan_blocks:
        idx = torch.tensor(nan_blocks, dtype=torch.long, device="cuda")
        kc[idx] = float("nan")
        vc[idx] = float("nan")
    out = to_f64(pg.gqa_paged_decode(dev.q, kc, vc, to_dev(table), dev.ctx, case.max_context_len,
                                     scale=float(case.scale), window=window))
    assert_close(out, ref, W.BF16, "released pages")


@pytest.mark.parametrize("window", [1, 31, 64, 65, 200])
@pytest.mark.parametrize("hq,hkv", [(32, 8), (8, 2), (4, 4), (16, 1)])
@pytest.mark.parametrize("d", [64, 128])
def test_prefill_windows(orc, window, hq, hkv, d):
    p = W.make_prefill_case([1, 31, 32, 33, 100, 7, 64, 129, 300], hq, hkv, d, 16, W.BF16,
                            seed=1400 + window + hq + d)
    say(f"prefill window {window} {hq}/{hkv} d{d}")
    out = to_f64(pg.gqa_varlen_prefill(to_dev(p.q), to_dev(p.k), to_dev(p.v), to_dev(p.cu_seqlens), p.max_seqlen,
                                       scale=float(p.scale), window=window))
    ref = orc.gqa_varlen_prefill(p.q, p.k, p.v, p.cu_seqlens, p.scale, window=window)
    assert_close(out, ref, W.BF16, f"prefill window {window} {hq}/{hkv} d{d}")


@pytest.mark.parametrize("window", [1, 5, 64, 129, 700])
@pytest.mark.parametrize("d,hq,hkv", [(128, 32, 8), (64, 8, 2), (128, 16, 1)])
def test_extend_windows(orc, window, d, hq, hkv):
    c = W.make_extend_case([0, 1, 31, 64, 100, 7, 650], [1, 33, 64, 5, 129, 40, 70], hq, hkv, d, 16, W.BF16,
                           seed=1500 + window + d + hq)
    say(f"extend window {window} d{d} {hq}/{hkv}")
    dev = DevExtend(c)
    out = to_f64(pg.gqa_paged_extend(dev.q, dev.cu_q, dev.kc, dev.vc, dev.table, dev.ctx, c.max_q_len,
                                     c.max_context_len, scale=float(c.scale), window=window))
    kc = W.nan_pool(c.num_blocks, c.num_kv_heads, c.block_size, c.head_dim, c.dtype)
    vc = W.nan_pool(c.num_blocks, c.num_kv_heads, c.block_size, c.head_dim, c.dtype)
    orc.paged_kv_write(c.k, c.v, c.cu_ctx, c.start_pos, c.block_table, kc, vc)
    ref = orc.gqa_paged_extend(c.q, c.cu_q, kc, vc, c.block_table, c.context_lens, c.scale, window=window)
    assert_close(out, ref, W.BF16, f"extend window {window} d{d}")


@pytest.mark.parametrize("bs", [8, 16, 32])
def test_extend_released_pages_are_not_read(orc, bs):
    """Multi-token queries with a window: pages wholly before every query's window
    released (table entries outside the pool, blocks NaN); a 64-key block of the
    kernel can start inside such pages when they are smaller than the block."""
    window = 100
    c = W.make_extend_case([3000, 700, 64, 1500, 37], [4, 40, 5, 1, 130], 32, 8, 128, bs, W.BF16, seed=1700 + bs)
    dev = DevExtend(c)
    ref = oracle_extend(orc, c, window=window)
    table = c.block_table.copy()
    nan_blocks = []
    for b, ctx in enumerate(c.context_lens):
        lo = max(0, int(ctx) - int(c.q_lens[b]) - window + 1)   # the first new row's window edge
        first_kept_page = lo // bs
        nan_blocks += table[b, :first_kept_page].tolist()
        table[b, :first_kept_page] = -1
    assert nan_blocks
    say(f"extend window with released pages bs{bs}")
    kc, vc = dev.kc.clone(), dev.vc.clone()
    idx = torch.tensor(nan_blocks, dtype=torch.long, device="cuda")
    kc[idx] = float("nan")
    vc[idx] = float("nan")
    out = to_f64(pg.gqa_paged_extend(dev.q, dev.cu_q, kc, vc, to_dev(table), dev.ctx, c.max_q_len,
                                     c.max_context_len, scale=float(c.scale), window=window))
    assert_close(out, ref, W.BF16, f"extend released pages bs{bs}")


def test_window_covering_everything_is_full_attention():
    """A window at least the longest context changes nothing: bit-identical outputs."""
    case = W.make_decode_case(LENS, 32, 8, 128, 16, W.BF16, seed=1600)
    dev = DevDecode(case)
    say("window >= context is full attention")
    a = pg.gqa_paged_decode(dev.q, dev.kc, dev.vc, dev.table, dev.ctx, case.max_context_len, scale=float(case.scale))
    b = pg.gqa_paged_decode(dev.q, dev.kc, dev.vc, dev.table, dev.ctx, case.max_context_len, scale=float(case.scale),
                            window=case.max_context_len)
    p = W.make_prefill_case([100, 300, 7], 32, 8, 128, 16, W.BF16, seed=1601)
    args = (to_dev(p.q), to_dev(p.k), to_dev(p.v), to_dev(p.cu_seqlens), p.max_seqlen)
    c = pg.gqa_varlen_prefill(*args, scale=float(p.scale))
    d = pg.gqa_varlen_prefill(*args, scale=float(p.scale), window=300)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(c.view(torch.int16), d.view(torch.int16))


def test_long_context_window_workload(orc):
    """The long-context decode workload (B = 8, ctx 32768, Hq 64) with a 4096-token window."""
    case = W.make_workload("long_ctx_decode")
    say("long-context decode, window 4096")
    dev = DevDecode(case)
    out = to_f64(pg.gqa_paged_decode(dev.q, dev.kc, dev.vc, dev.table, dev.ctx, case.max_context_len,
                                     scale=float(case.scale), window=4096))
    assert_close(out, _oracle_decode(orc, case, 4096), W.BF16, "long ctx window 4096")
