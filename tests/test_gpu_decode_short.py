"""Decode calls whose every segment is at most two tiles long (latency-bound): one
workgroup per (sequence, KV head) segment writes the outputs directly and no merge
kernel runs.  Against the fp64 oracle, with the route checked in the PGQA_LOG line,
and against the same call with an explicit split count (stream-K shares + merge)."""

import numpy as np
import pytest
import torch

import workload as W
import paged_gqa_kv_02_amd as pg
from gpu_helpers import DevDecode, assert_close, oracle_decode, oracle_pools, say, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _logged(monkeypatch, capfd, fn):
    capfd.readouterr()
    monkeypatch.setenv("PGQA_LOG", "1")
    try:
        out = fn()
        torch.cuda.synchronize()
    finally:
        monkeypatch.setenv("PGQA_LOG", "0")
    return out, capfd.readouterr().err


@pytest.mark.parametrize("hq,hkv,d,bs,dtype,maxlen", [
    (32, 8, 128, 16, W.BF16, 32),     # bf16 d128: 16-token tiles, two tiles
    (64, 8, 128, 16, W.BF16, 17),     # G = 8
    (64, 4, 128, 16, W.BF16, 32),     # G = 16: two-wave workgroups
    (16, 8, 64, 8, W.BF16, 64),       # d 64: 32-token tiles
    (4, 2, 16, 4, W.F32, 11),         # the tiny fp32 shape
])
def test_short_contexts(orc, monkeypatch, capfd, hq, hkv, d, bs, dtype, maxlen):
    rng = np.random.default_rng(3000 + hq + d + maxlen)
    lens = rng.integers(0, maxlen + 1, 37)
    lens[0], lens[1] = 0, maxlen                        # an empty sequence and a full one
    case = W.make_decode_case(lens, hq, hkv, d, bs, dtype, seed=3001 + hq + d)
    say(f"short decode {hq}/{hkv} d{d} max {maxlen}")
    dev = DevDecode(case)
    out, err = _logged(monkeypatch, capfd, dev.decode)
    assert "one workgroup per segment" in err and "no merge" in err, err
    ref = oracle_decode(orc, case)
    assert_close(to_f64(out), ref, dtype, f"short {hq}/{hkv} d{d}")
    split = dev.decode(num_splits=64)
    assert_close(to_f64(split), ref, dtype, f"short {hq}/{hkv} d{d}, 64 splits")


def test_longer_contexts_keep_the_shares(monkeypatch, capfd):
    """Three tiles in the longest segment: the stream-K split and its merge."""
    case = W.make_decode_case([1, 33, 48, 5], 32, 8, 128, 16, W.BF16, seed=3050)
    dev = DevDecode(case)
    _, err = _logged(monkeypatch, capfd, dev.decode)
    assert "one workgroup per segment" not in err and "merge" in err, err


def test_short_contexts_window(orc, monkeypatch, capfd):
    case = W.make_decode_case([0, 1, 5, 31, 32, 20], 32, 8, 128, 16, W.BF16, seed=3060)
    dev = DevDecode(case)
    out, err = _logged(monkeypatch, capfd, lambda: pg.gqa_paged_decode(
        dev.q, dev.kc, dev.vc, dev.table, dev.ctx, case.max_context_len, scale=float(case.scale), window=7))
    assert "one workgroup per segment" in err, err
    kc, vc = oracle_pools(orc, case)
    ref = orc.gqa_paged_decode(case.q, kc, vc, case.block_table, case.context_lens, case.scale, window=7)
    assert_close(to_f64(out), ref, W.BF16, "short window 7")


def test_short_contexts_fp8(orc, monkeypatch, capfd):
    """FP8 pages (32-token tiles): contexts up to 64, against the oracle over the
    dequantised pages."""
    c = W.make_decode_case([0, 64, 17, 33, 1, 50], 32, 8, 128, 16, W.BF16, seed=3070)
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
    out, err = _logged(monkeypatch, capfd, lambda: pg.gqa_paged_decode_fp8(
        to_dev(c.q), dk, dv, ds, dvs, table, ctx, c.max_context_len, scale=float(c.scale)))
    assert "fp8" in err and "one workgroup per segment" in err, err
    qd = (c.q.view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = orc.gqa_paged_decode(qd, orc.dequantize_fp8(hk, hs), orc.dequantize_fp8(hv, hvs), c.block_table,
                               c.context_lens, c.scale)
    assert_close(to_f64(out), ref, W.BF16, "short fp8")
