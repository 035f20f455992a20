"""Low-precision (FP8 E4M3) KV pages on the GPU: the quantising write bit-exact
against the oracle's (codes and row scales), and decode over FP8 pages against
the oracle's attention over the dequantised cache."""

import numpy as np
import pytest
import torch

import workload as W
import paged_gqa_kv_02_amd as pg
from gpu_helpers import assert_close, say, to_bits, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _dev_pools(nb, hkv, bs, d):
    kc = torch.full((nb, hkv, bs, d), 0x7F, dtype=torch.uint8, device="cuda")
    ks = torch.full((nb, hkv, bs), float("nan"), dtype=torch.float32, device="cuda")
    return kc, kc.clone(), ks, ks.clone()


def _host_pools(nb, hkv, bs, d):
    kc = np.full((nb, hkv, bs, d), 0x7F, dtype=np.uint8)
    ks = np.full((nb, hkv, bs), np.nan, dtype=np.float32)
    return kc, kc.copy(), ks, ks.copy()


def _write_both(orc, c):
    nb, hkv, bs, d = c.num_blocks, c.num_kv_heads, c.block_size, c.head_dim
    dk, dv, dks, dvs = _dev_pools(nb, hkv, bs, d)
    pg.paged_kv_write_fp8(to_dev(c.k), to_dev(c.v), to_dev(c.cu_ctx), to_dev(c.start_pos), to_dev(c.block_table),
                          dk, dv, dks, dvs)
    hk, hv, hks, hvs = _host_pools(nb, hkv, bs, d)
    orc.paged_kv_write_fp8(c.k, c.v, c.cu_ctx, c.start_pos, c.block_table, hk, hv, hks, hvs)
    return (dk, dv, dks, dvs), (hk, hv, hks, hvs)


def _special_rows(c):
    """Overwrite a few K/V rows with the cases the codes hinge on: a row whose
    scale is exactly 1 (max 448) holding the midpoints between neighbouring codes
    (ties) and subnormal-range values, an all-zero row, a row with one large value."""
    d = c.head_dim
    codes = np.arange(0x7F, dtype=np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    row = np.resize(np.concatenate([mids, -mids[::-1]]), d).astype(np.float32)
    row[0] = 448.0
    for arr, t, h, r in ((c.k, 0, 0, row), (c.v, 1, 0, -row), (c.k, 2, 0, np.zeros(d, np.float32)),
                         (c.v, 2, 0, np.full(d, 1e-3, np.float32) * np.eye(1, d, 5, dtype=np.float32)[0] * 5e4)):
        if t < arr.shape[0]:
            arr[t, h] = W.f32_to_bf16_bits(r)


@pytest.mark.parametrize("d,bs,hkv", [(128, 16, 8), (64, 16, 2), (32, 1, 4), (16, 256, 1), (128, 256, 2)])
def test_write_bit_exact(orc, d, bs, hkv):
    c = W.make_decode_case([1, 17, 96, 203, 3], 2 * hkv, hkv, d, bs, W.BF16, seed=2000 + d + bs)
    _special_rows(c)
    say(f"fp8 write d{d} bs{bs} hkv{hkv}")
    dev, host = _write_both(orc, c)
    for g, h, name in zip(dev, host, ("k codes", "v codes", "k scales", "v scales")):
        got = to_bits(g)
        if got.dtype == np.float32:
            assert np.array_equal(got.view(np.uint32), h.view(np.uint32)), name
        else:
            assert np.array_equal(got, h), name


def _decode_case_fp8(orc, c, window=0, num_splits=0):
    dev, host = _write_both(orc, c)
    dk, dv, dks, dvs = dev
    hk, hv, hks, hvs = host
    out = pg.gqa_paged_decode_fp8(to_dev(c.q), dk, dv, dks, dvs, to_dev(c.block_table), to_dev(c.context_lens),
                                  c.max_context_len, scale=float(c.scale), window=window, num_splits=num_splits)
    qd = c.q.view(np.uint16).astype(np.uint32) << 16
    ref = orc.gqa_paged_decode(qd.view(np.float32).astype(np.float64), orc.dequantize_fp8(hk, hks),
                               orc.dequantize_fp8(hv, hvs), c.block_table, c.context_lens, c.scale, window=window)
    return to_f64(out), ref


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 4), (8, 2), (32, 8), (16, 1), (32, 1), (64, 1)])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_shapes(orc, hq, hkv, d):
    c = W.make_decode_case([1, 17, 96, 203, 3, 700], hq, hkv, d, 16, W.BF16, seed=2100 + hq + hkv + d)
    say(f"fp8 decode {hq}/{hkv} d{d}")
    out, ref = _decode_case_fp8(orc, c)
    assert_close(out, ref, W.BF16, f"fp8 decode {hq}/{hkv} d{d}")


@pytest.mark.parametrize("bs", [16, 32, 64, 128, 256])
def test_decode_block_sizes(orc, bs):
    c = W.make_decode_case([1, bs - 1, bs, bs + 1, 3 * bs + 5, 300], 32, 8, 128, bs, W.BF16, seed=2200 + bs)
    say(f"fp8 decode bs{bs}")
    out, ref = _decode_case_fp8(orc, c)
    assert_close(out, ref, W.BF16, f"fp8 decode bs{bs}")


@pytest.mark.parametrize("window,num_splits", [(0, 1), (0, 7), (0, 1000), (100, 0), (1, 0), (513, 37)])
def test_decode_windows_and_splits(orc, window, num_splits):
    c = W.make_decode_case([5, 64, 65, 1000, 2100, 129], 32, 8, 128, 16, W.BF16, seed=2300 + window + num_splits)
    say(f"fp8 decode window {window} splits {num_splits}")
    out, ref = _decode_case_fp8(orc, c, window=window, num_splits=num_splits)
    assert_close(out, ref, W.BF16, f"fp8 window {window} splits {num_splits}")


def test_decode_sharpened_queries(orc):
    c = W.make_decode_case([40, 300, 1000], 32, 8, 128, 16, W.BF16, seed=2400)
    c.q = W.f32_to_bf16_bits(W.bf16_bits_to_f32(c.q) * np.float32(4.0))
    say("fp8 decode sharpened")
    out, ref = _decode_case_fp8(orc, c)
    assert np.abs(ref).max() > 0.5
    assert_close(out, ref, W.BF16, "fp8 sharpened")


@pytest.mark.parametrize("key", ["llama3_8b_decode", "long_ctx_decode"])
def test_workload(orc, key):
    """The decode workloads with FP8 pages, in the launch configuration the benchmark times."""
    c = W.make_workload(key)
    say(f"fp8 decode workload {key}")
    out, ref = _decode_case_fp8(orc, c)
    e = assert_close(out, ref, W.BF16, f"fp8 {key}")
    say(f"fp8 {key}: {e}")


# ---- several new tokens per sequence over FP8 pages (gqa_paged_extend_fp8) ----

def _extend_case_fp8(orc, c, window=0, context_lens=None, workspace=None):
    """Device result and the oracle's multi-token attention over the dequantised
    cache (fp64, bf16 queries widened exactly)."""
    dev, host = _write_both(orc, c)
    dk, dv, dks, dvs = dev
    hk, hv, hks, hvs = host
    ctx = c.context_lens if context_lens is None else np.asarray(context_lens, np.int32)
    kw = {} if workspace is None else {"workspace": workspace}
    out = pg.gqa_paged_extend_fp8(to_dev(c.q), to_dev(c.cu_q), dk, dv, dks, dvs, to_dev(c.block_table),
                                  to_dev(ctx), c.max_q_len, int(ctx.max()) if len(ctx) else 0,
                                  scale=float(c.scale), window=window, **kw)
    qd = (c.q.view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = orc.gqa_paged_extend(qd, c.cu_q, orc.dequantize_fp8(hk, hks), orc.dequantize_fp8(hv, hvs),
                               c.block_table, ctx, c.scale, window=window)
    return to_f64(out), ref


EXT_PREFIX = [0, 1, 31, 64, 100, 7, 250]
EXT_QLENS = [1, 33, 64, 5, 129, 40, 16]


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2), (32, 8), (16, 1), (64, 1)])
@pytest.mark.parametrize("d", [64, 128])
def test_extend_shapes(orc, hq, hkv, d):
    c = W.make_extend_case(EXT_PREFIX, EXT_QLENS, hq, hkv, d, 16, W.BF16, seed=2500 + hq * 10 + hkv + d)
    say(f"fp8 extend {hq}/{hkv} d{d}")
    out, ref = _extend_case_fp8(orc, c)
    assert_close(out, ref, W.BF16, f"fp8 extend {hq}/{hkv} d{d}")


@pytest.mark.parametrize("d,bs", [(128, 8), (128, 16), (128, 64), (128, 256), (64, 16), (64, 32), (64, 256)])
def test_extend_block_sizes(orc, d, bs):
    c = W.make_extend_case([0, bs - 1, bs, 3 * bs + 1, 70], [bs + 1, 1, 2 * bs, 64, 97], 8, 2, d, bs, W.BF16,
                           seed=2600 + bs + d)
    say(f"fp8 extend bs{bs} d{d}")
    out, ref = _extend_case_fp8(orc, c)
    assert_close(out, ref, W.BF16, f"fp8 extend bs{bs} d{d}")


def test_extend_single_token_equals_decode(orc):
    """q_len = 1 everywhere: FP8 decode over the same pages, both against the oracle."""
    c = W.make_extend_case([0, 15, 16, 300, 1000, 2047], [1] * 6, 32, 8, 128, 16, W.BF16, seed=2610)
    say("fp8 extend q_len=1 vs fp8 decode")
    out, ref = _extend_case_fp8(orc, c)
    assert_close(out, ref, W.BF16, "fp8 extend q_len=1")
    dc = W.DecodeCase(name="x", dtype=W.BF16, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                      context_lens=c.context_lens, cu_ctx=c.cu_ctx, q=c.q, k=c.k, v=c.v,
                      block_table=c.block_table, num_blocks=c.num_blocks, scale=c.scale)
    dec, dref = _decode_case_fp8(orc, dc)
    assert np.array_equal(dref, ref)
    assert_close(dec, ref, W.BF16, "fp8 decode")


def test_extend_edges(orc):
    """Empty sequences, a context shorter than its query count (rows with no key
    give 0), and a sequence with no context at all."""
    c = W.make_extend_case([5, 0, 40, 3, 0, 16], [0, 0, 70, 9, 4, 33], 8, 2, 128, 16, W.BF16, seed=2620)
    ctx = c.context_lens.copy()
    ctx[3] = 4
    ctx[4] = 0
    say("fp8 extend edges")
    out, ref = _extend_case_fp8(orc, c, context_lens=ctx)
    qa = int(c.cu_q[3])
    assert (ref[qa:qa + 5] == 0).all() and (out[qa:qa + 5] == 0).all()
    assert (out[int(c.cu_q[4]):int(c.cu_q[5])] == 0).all()
    assert_close(out, ref, W.BF16, "fp8 extend edges")


def test_extend_sharpened_queries(orc):
    c = W.make_extend_case([10, 200, 63], [100, 17, 65], 32, 8, 128, 16, W.BF16, seed=2630)
    c.q = W.f32_to_bf16_bits(W.bf16_bits_to_f32(c.q) * np.float32(4.0))
    say("fp8 extend sharpened")
    out, ref = _extend_case_fp8(orc, c)
    assert np.abs(ref).max() > 0.5
    assert_close(out, ref, W.BF16, "fp8 extend sharpened")


@pytest.mark.parametrize("q_len,window,d", [(4, 0, 128), (7, 300, 128), (37, 1000, 64), (40, 0, 64)])
def test_extend_key_split_and_window(orc, q_len, window, d):
    """Few query tokens over long contexts (the library splits the key range),
    with and without a window; also with no workspace (no split)."""
    prefix = [3000, 17, 1024 - q_len, 1025 - q_len, 2048, 4000, 64, 2500]
    c = W.make_extend_case(prefix, [q_len] * len(prefix), 8, 2, d, 16, W.BF16, seed=2640 + q_len + window + d)
    assert pg.gqa_paged_extend_workspace_size(c.batch, c.total_q, c.max_q_len, 8, 2, d, c.max_context_len) > 0
    say(f"fp8 extend key split q_len={q_len} window={window} d{d}")
    out, ref = _extend_case_fp8(orc, c, window=window)
    assert_close(out, ref, W.BF16, "fp8 split")
    out1, _ = _extend_case_fp8(orc, c, window=window, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    assert_close(out1, ref, W.BF16, "fp8 no split")


@pytest.mark.parametrize("key", ["chunked_prefill", "spec_verify"])
def test_extend_workload(orc, key):
    """The multi-token workloads over FP8 pages in the benchmark's launch
    configuration, every output against the oracle."""
    c = W.make_workload(key)
    say(f"fp8 extend workload {key}")
    out, ref = _extend_case_fp8(orc, c)
    e = assert_close(out, ref, W.BF16, f"fp8 extend {key}")
    say(f"fp8 extend {key}: {e}")


@pytest.mark.parametrize("bs", [8, 16, 32])
def test_extend_released_pages_are_not_read(orc, bs):
    """A window over FP8 pages with the pages before every query's window released
    (table entries -1, their codes NaN, their scales NaN)."""
    window = 100
    c = W.make_extend_case([3000, 700, 64, 1500, 37], [4, 40, 5, 1, 130], 32, 8, 128, bs, W.BF16, seed=2700 + bs)
    dev, host = _write_both(orc, c)
    dk, dv, dks, dvs = dev
    hk, hv, hks, hvs = host
    qd = (c.q.view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = orc.gqa_paged_extend(qd, c.cu_q, orc.dequantize_fp8(hk, hks), orc.dequantize_fp8(hv, hvs),
                               c.block_table, c.context_lens, c.scale, window=window)
    table = c.block_table.copy()
    gone = []
    for b, ctx in enumerate(c.context_lens):
        lo = max(0, int(ctx) - int(c.q_lens[b]) - window + 1)
        gone += table[b, :lo // bs].tolist()
        table[b, :lo // bs] = -1
    assert gone
    idx = torch.tensor(gone, dtype=torch.long, device="cuda")
    for pool in (dk, dv):
        pool[idx] = 0x7F
    for pool in (dks, dvs):
        pool[idx] = float("nan")
    say(f"fp8 extend window with released pages bs{bs}")
    out = pg.gqa_paged_extend_fp8(to_dev(c.q), to_dev(c.cu_q), dk, dv, dks, dvs, to_dev(table),
                                  to_dev(c.context_lens), c.max_q_len, c.max_context_len, scale=float(c.scale),
                                  window=window)
    assert_close(to_f64(out), ref, W.BF16, f"fp8 extend released pages bs{bs}")


@pytest.mark.parametrize("hq,hkv,qlens,window", [(24, 2, [2, 1, 2, 2], 0), (32, 1, [1, 1, 1, 1], 0),
                                                 (8, 2, [8, 3, 8, 1], 70), (2, 2, [32, 5, 17, 32], 0)])
def test_extend_packed_rows(orc, hq, hkv, qlens, window):
    """FP8 pages on the packed-rows kernel (query tokens x group <= 32): groups that
    are not powers of two, one token of 32 heads, windows, full 32-row tiles."""
    c = W.make_extend_case([3000, 64, 130, 1], qlens, hq, hkv, 128, 16, W.BF16, seed=2800 + hq + hkv + window)
    say(f"fp8 extend packed {hq}/{hkv} q_lens {qlens} window {window}")
    out, ref = _extend_case_fp8(orc, c, window=window)
    assert_close(out, ref, W.BF16, f"fp8 packed {hq}/{hkv}")
