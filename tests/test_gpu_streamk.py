"""Stream-K shares of the packed-rows kernel (multi-token calls whose tokens times
the group fit one 32-row tile, and one-KV-head decode): every workgroup takes an
equal share of the pairs' work units, pairs cut by a share edge leave fp32
partials that a merge kernel combines.  Checked against the fp64 oracle, against
the same call without a workspace (one workgroup per pair), and for the route
taken (PGQA_LOG)."""

import re

import numpy as np
import pytest
import torch

import workload as W
import paged_gqa_kv_02_amd as pg
from gpu_helpers import DevDecode, DevExtend, assert_close, oracle_decode, oracle_extend, say, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _extend(dev, c, window=0, workspace=None):
    return pg.gqa_paged_extend(dev.q, dev.cu_q, dev.kc, dev.vc, dev.table, dev.ctx, c.max_q_len, c.max_context_len,
                               scale=float(c.scale), window=window, workspace=workspace)


def _route(monkeypatch, capfd, fn):
    """Run fn with the launch log on; return what the library printed."""
    capfd.readouterr()
    monkeypatch.setenv("PGQA_LOG", "1")
    try:
        out = fn()
        torch.cuda.synchronize()
    finally:
        monkeypatch.setenv("PGQA_LOG", "0")
    return out, capfd.readouterr().err


# 1,200 sequences x 2 KV heads: more pairs per scanning thread than it keeps in
# registers, and shares whose pair range (mostly pairs without query rows) runs
# past the pairs handed over in LDS.
_rng = np.random.default_rng(4242)
_MANY_Q = np.where(_rng.random(1200) < 0.75, 0, _rng.choice([1, 2, 4], 1200)).tolist()
_MANY_P = _rng.integers(0, 300, 1200).tolist()


@pytest.mark.parametrize("name,prefix,qlens,hq,hkv,d,window", [
    # one long sequence: every pair is cut into many pieces (hundreds of shares)
    ("one long pair", [100000 - 1], [1], 32, 1, 128, 0),
    ("few long pairs", [60000, 30000], [4, 2], 32, 8, 128, 0),
    # more work units than shares, pairs of every length, empty query rows
    ("ragged", [3000, 0, 61, 64, 1500, 120, 9000, 5, 0, 777], [4, 1, 3, 0, 2, 4, 4, 1, 0, 3], 32, 8, 128, 0),
    ("ragged d64", [3000, 0, 61, 64, 1500, 120, 9000, 5, 0, 777], [4, 1, 3, 0, 2, 4, 4, 1, 0, 3], 32, 8, 64, 0),
    # fewer work units than workgroup slots: empty shares
    ("tiny", [3, 0], [1, 2], 8, 2, 128, 0),
    # a window: each pair's units start at its first row's window edge
    ("window", [20000, 500, 7000, 64], [2, 2, 1, 2], 32, 4, 128, 1000),
    ("window inside a block", [20000, 500, 7000, 64], [2, 2, 1, 2], 32, 4, 128, 37),
    # more than 16 packed rows: 16-row waves (24 rows of G = 12; 8 heads x 4 tokens
    # under a window; one token of 32 heads at d 64)
    ("ragged, 16-row waves", [3000, 0, 61, 64, 1500, 120, 9000, 5, 0, 777], [2, 1, 2, 0, 2, 1, 2, 1, 0, 2], 24, 2,
     128, 0),
    ("window, 16-row waves", [20000, 500, 7000, 64], [4, 3, 1, 4], 64, 8, 128, 1000),
    ("d64, 16-row waves", [9000, 33, 2000, 0], [1, 1, 1, 1], 32, 1, 64, 0),
    ("many pairs, mostly empty", _MANY_P, _MANY_Q, 16, 2, 128, 0),
])
def test_streamk_against_oracle(orc, monkeypatch, capfd, name, prefix, qlens, hq, hkv, d, window):
    c = W.make_extend_case(prefix, qlens, hq, hkv, d, 16, W.BF16, seed=4100 + sum(prefix) % 997 + hq + d + window)
    say(f"stream-K {name}: {hq}/{hkv} d={d} window={window}")
    dev = DevExtend(c)
    out, err = _route(monkeypatch, capfd, lambda: _extend(dev, c, window))
    assert "stream-K shares" in err, err
    # More than 16 packed rows (32 heads of one token here) run in 16-row waves.
    assert ("in 16-row waves" in err) == (max(qlens) * (hq // hkv) > 16), err
    ref = oracle_extend(orc, c, window=window)
    assert_close(to_f64(out), ref, W.BF16, f"stream-K {name}")
    plain = _extend(dev, c, window, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    assert_close(to_f64(plain), ref, W.BF16, f"{name}, one workgroup per pair")


def test_streamk_is_deterministic():
    c = W.make_extend_case([32000, 9000, 20000, 100], [4] * 4, 32, 8, 128, 16, W.BF16, seed=4150)
    dev = DevExtend(c)
    say("stream-K twice")
    a = _extend(dev, c)
    b = _extend(dev, c)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_streamk_workspace_fallback(orc, monkeypatch, capfd):
    """A workspace too small for the shares' partials but large enough for key
    chunks: the packed kernel splits into key chunks instead."""
    c = W.make_extend_case([3000, 17, 4000, 64, 2500, 7000], [4] * 6, 32, 8, 128, 16, W.BF16, seed=4160)
    dev = DevExtend(c)
    full = pg.gqa_paged_extend_workspace_size(c.batch, c.total_q, c.max_q_len, 32, 8, 128, c.max_context_len)
    per_chunk = c.total_q * 32 * (128 + 2) * 4
    assert full > 4 * per_chunk
    ws = torch.empty(4 * per_chunk, dtype=torch.uint8, device="cuda")
    say("stream-K workspace fallback")
    out, err = _route(monkeypatch, capfd, lambda: _extend(dev, c, workspace=ws))
    assert "stream-K" not in err and "key chunks" in err, err
    assert_close(to_f64(out), oracle_extend(orc, c), W.BF16, "key chunks")


def test_streamk_many_pairs_fallback(orc, monkeypatch, capfd):
    """More (sequence, KV head) pairs than one workgroup's scan covers: the
    library keeps one workgroup per pair."""
    rng = np.random.default_rng(4170)
    B = 520                                   # x 8 KV heads = 4160 pairs
    c = W.make_extend_case(rng.integers(0, 80, B), [1] * B, 32, 8, 128, 16, W.BF16, seed=4171)
    dev = DevExtend(c)
    say("stream-K many pairs")
    out, err = _route(monkeypatch, capfd, lambda: _extend(dev, c))
    assert "stream-K" not in err, err
    assert_close(to_f64(out), oracle_extend(orc, c), W.BF16, "4160 pairs")


def test_streamk_fp8_pages(orc, monkeypatch, capfd):
    """FP8 pages on the packed rows: the same shares, against the oracle's
    attention over the dequantised pages."""
    c = W.make_extend_case([30000, 0, 61, 4000, 100], [4, 1, 3, 2, 4], 32, 8, 128, 16, W.BF16, seed=4180)
    nb = c.num_blocks
    dk = torch.full((nb, 8, 16, 128), 0x7F, dtype=torch.uint8, device="cuda")
    ds = torch.full((nb, 8, 16), float("nan"), dtype=torch.float32, device="cuda")
    dv, dvs = dk.clone(), ds.clone()
    table, ctx = to_dev(c.block_table), to_dev(c.context_lens)
    pg.paged_kv_write_fp8(to_dev(c.k), to_dev(c.v), to_dev(c.cu_ctx), to_dev(c.start_pos), table, dk, dv, ds, dvs)
    hk = np.full((nb, 8, 16, 128), 0x7F, dtype=np.uint8)
    hs = np.full((nb, 8, 16), np.nan, dtype=np.float32)
    hv, hvs = hk.copy(), hs.copy()
    orc.paged_kv_write_fp8(c.k, c.v, c.cu_ctx, c.start_pos, c.block_table, hk, hv, hs, hvs)
    qd = (c.q.view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = orc.gqa_paged_extend(qd, c.cu_q, orc.dequantize_fp8(hk, hs), orc.dequantize_fp8(hv, hvs), c.block_table,
                               c.context_lens, c.scale)
    q, cu_q = to_dev(c.q), to_dev(c.cu_q)
    say("stream-K fp8")
    out, err = _route(monkeypatch, capfd, lambda: pg.gqa_paged_extend_fp8(
        q, cu_q, dk, dv, ds, dvs, table, ctx, c.max_q_len, c.max_context_len, scale=float(c.scale)))
    assert "fp8" in err and "stream-K shares" in err and "16-row" not in err, err
    assert_close(to_f64(out), ref, W.BF16, "fp8 stream-K")
    plain = pg.gqa_paged_extend_fp8(q, cu_q, dk, dv, ds, dvs, table, ctx, c.max_q_len, c.max_context_len,
                                    scale=float(c.scale), workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    assert_close(to_f64(plain), ref, W.BF16, "fp8, one workgroup per pair")


def test_mqa_decode_streamk(orc, monkeypatch, capfd):
    """One-KV-head decode with 32 query heads runs the packed kernel's shares."""
    c = W.make_decode_case([1, 9000, 300, 16, 5000, 64, 1], 32, 1, 128, 32, W.BF16, seed=4190)
    dev = DevDecode(c)
    say("MQA decode stream-K")
    out, err = _route(monkeypatch, capfd, lambda: pg.gqa_paged_decode(
        dev.q, dev.kc, dev.vc, dev.table, dev.ctx, c.max_context_len, scale=float(c.scale)))
    assert "stream-K shares" in err and "in 16-row waves" in err, err
    kc = W.nan_pool(c.num_blocks, 1, 32, 128, c.dtype)
    vc = W.nan_pool(c.num_blocks, 1, 32, 128, c.dtype)
    orc.paged_kv_write(c.k, c.v, c.cu_ctx, c.start_pos, c.block_table, kc, vc)
    ref = orc.gqa_paged_decode(c.q, kc, vc, c.block_table, c.context_lens, c.scale)
    assert_close(to_f64(out), ref, W.BF16, "MQA decode")


def test_one_workspace_across_routes(orc, monkeypatch, capfd):
    """One workspace buffer shared, in turn, by the one-KV-head stream-K decode, the
    split-KV decode, the packed stream-K extend and the key-chunk extend, with
    different inputs each time: whatever a route leaves in the buffer, the next
    call's outputs still match the oracle (no route depends on what another wrote).
    The buffer starts as all-ones bytes (NaN floats, -1 ints): no call needs it
    initialised."""
    mqa_a = W.make_decode_case([900, 1, 2500, 64, 0, 5000], 32, 1, 128, 32, W.BF16, seed=811)
    mqa_b = W.make_decode_case([3000, 17, 640, 129], 32, 1, 128, 32, W.BF16, seed=812)
    gqa = W.make_decode_case([700, 33, 2100, 4096, 515], 32, 8, 128, 16, W.BF16, seed=813)
    sk = W.make_extend_case([3000, 0, 61, 1500, 9000], [2, 1, 2, 2, 1], 32, 2, 128, 16, W.BF16, seed=814)
    chunks = W.make_extend_case([20000, 3000], [96, 40], 32, 8, 128, 16, W.BF16, seed=815)
    need = max(pg.gqa_paged_decode_workspace_size(6, 32, 1, 128, 0),
               pg.gqa_paged_decode_workspace_size(5, 32, 8, 128, 5),
               pg.gqa_paged_extend_workspace_size(sk.batch, int(sk.q_lens.sum()), int(sk.q_lens.max()), 32, 2, 128,
                                                  int(sk.context_lens.max())),
               pg.gqa_paged_extend_workspace_size(chunks.batch, int(chunks.q_lens.sum()), int(chunks.q_lens.max()),
                                                  32, 8, 128, int(chunks.context_lens.max())))
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    dm_a, dm_b, dg = DevDecode(mqa_a), DevDecode(mqa_b), DevDecode(gqa)
    de_sk, de_ch = DevExtend(sk), DevExtend(chunks)

    def dec(dev, c, splits=0):
        return pg.gqa_paged_decode(dev.q, dev.kc, dev.vc, dev.table, dev.ctx, c.max_context_len,
                                   scale=float(c.scale), num_splits=splits, workspace=ws)

    steps = [
        ("MQA stream-K decode A", lambda: dec(dm_a, mqa_a), lambda: oracle_decode(orc, mqa_a), "stream-K shares"),
        ("split-KV decode", lambda: dec(dg, gqa, 5), lambda: oracle_decode(orc, gqa), None),
        ("packed stream-K extend", lambda: _extend(de_sk, sk, workspace=ws), lambda: oracle_extend(orc, sk),
         "stream-K shares"),
        ("MQA stream-K decode B", lambda: dec(dm_b, mqa_b), lambda: oracle_decode(orc, mqa_b), "stream-K shares"),
        ("key-chunk extend", lambda: _extend(de_ch, chunks, workspace=ws), lambda: oracle_extend(orc, chunks),
         "key chunks"),
        ("MQA stream-K decode A again", lambda: dec(dm_a, mqa_a), lambda: oracle_decode(orc, mqa_a),
         "stream-K shares"),
    ]
    for name, run, ref, route in steps:
        say(f"shared workspace: {name}")
        out, err = _route(monkeypatch, capfd, run)
        if route == "key chunks":
            m = re.search(r"key chunks (\d+) x", err)
            assert m and int(m.group(1)) > 1, (name, err)
        elif route is not None:
            assert route in err, (name, err)
        assert_close(to_f64(out), ref(), W.BF16, f"shared workspace: {name}")
