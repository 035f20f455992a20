"""The debugging aids on the GPU: pgqa_check_contents finds every kind of broken
promise about device array contents (and reports nothing on valid inputs),
PGQA_DEBUG_CHECKS turns a broken promise into an error before the call, and
PGQA_LOG prints each launch's route."""

import numpy as np
import pytest
import torch

import workload as W
import paged_gqa_kv_02_amd as pg
from paged_gqa_kv_02_amd import ops
from gpu_helpers import DevDecode, DevExtend, say, to_dev

pytestmark = pytest.mark.gpu


def _decode_check(c, table=None, ctx=None, window=0, max_ctx=None):
    table = c.block_table if table is None else table
    ctx = c.context_lens if ctx is None else ctx
    return pg.check_contents(c.batch, block_table=to_dev(table), context_lens=to_dev(ctx), num_blocks=c.num_blocks,
                             block_size=c.block_size,
                             max_context_len=c.max_context_len if max_ctx is None else max_ctx, window=window)


def _extend_check(c, table=None, ctx=None, cu=None, window=0):
    table = c.block_table if table is None else table
    ctx = c.context_lens if ctx is None else ctx
    cu = c.cu_q if cu is None else cu
    return pg.check_contents(c.batch, block_table=to_dev(table), context_lens=to_dev(ctx), cu_rows=to_dev(cu),
                             total_rows=c.total_q, max_rows=c.max_q_len, num_blocks=c.num_blocks,
                             block_size=c.block_size, max_context_len=c.max_context_len, window=window)


def test_valid_workloads_pass():
    for key in ("llama3_8b_decode", "long_ctx_decode", "mqa_decode"):
        c = W.make_workload(key)
        say(f"check contents: {key}")
        assert _decode_check(c)["flags"] == 0
    for key in ("chunked_prefill", "spec_verify"):
        c = W.make_workload(key)
        say(f"check contents: {key}")
        assert _extend_check(c)["flags"] == 0
        r = pg.check_contents(c.batch, block_table=to_dev(c.block_table), cu_rows=to_dev(c.cu_ctx),
                              start_pos=to_dev(c.start_pos), total_rows=int(c.cu_ctx[-1]), num_blocks=c.num_blocks,
                              block_size=c.block_size)
        assert r["flags"] == 0
    p = W.make_workload("varlen_prefill")
    r = pg.check_contents(len(p.cu_seqlens) - 1, cu_rows=to_dev(p.cu_seqlens), total_rows=int(p.cu_seqlens[-1]),
                          max_rows=p.max_seqlen)
    assert r == {"flags": 0, "first_bad_sequence": None, "bad_block_ids": 0, "bad_sequences": 0, "problems": []}


def test_bad_block_ids():
    c = W.make_decode_case([1, 17, 96, 203, 3, 700], 8, 2, 128, 16, W.BF16, seed=3000)
    t = c.block_table.copy()
    t[3, 5] = -1                    # page 5 of 13 used pages
    t[5, 0] = c.num_blocks          # one past the pool
    t[5, 43] = c.num_blocks + 7     # page 43 of 44
    t[0, 1] = -5                    # past sequence 0's single page: never read
    say("check contents: bad block ids")
    r = _decode_check(c, table=t)
    assert r["flags"] == 1 and r["first_bad_sequence"] == 3 and r["bad_block_ids"] == 3 and r["bad_sequences"] == 2


def test_window_ignores_released_pages():
    c = W.make_decode_case([1000, 700, 64], 8, 2, 128, 16, W.BF16, seed=3001)
    t = c.block_table.copy()
    t[0, :(1000 - 100) // 16] = -1       # wholly before the window of 100
    t[1, :(700 - 100) // 16] = -1
    say("check contents: released pages under a window")
    assert _decode_check(c, table=t, window=100)["flags"] == 0
    assert _decode_check(c, table=t)["flags"] == 1
    t[0, (1000 - 100) // 16] = -1        # the page holding the window's first key
    r = _decode_check(c, table=t, window=100)
    assert r["flags"] == 1 and r["first_bad_sequence"] == 0 and r["bad_block_ids"] == 1


def test_bad_lengths_and_offsets():
    c = W.make_extend_case([0, 31, 64, 100], [5, 33, 1, 7], 8, 2, 128, 16, W.BF16, seed=3002)
    ctx = c.context_lens.copy()
    ctx[2] = c.max_context_len + 1
    ctx[1] = -3
    say("check contents: lengths and offsets")
    r = _extend_check(c, ctx=ctx)
    assert r["flags"] & 2 and r["first_bad_sequence"] == 1 and r["bad_sequences"] == 2
    ctx = c.context_lens.copy()
    ctx[3] = 6                           # 7 new rows, 6 cached positions
    r = _extend_check(c, ctx=ctx)
    assert r["flags"] == 8 and r["first_bad_sequence"] == 3
    cu = c.cu_q.copy()
    cu[2] = cu[1] - 1                    # decreasing
    r = _extend_check(c, cu=cu)
    assert r["flags"] & 4 and r["first_bad_sequence"] == 1
    cu = c.cu_q.copy()
    cu[-1] += 1                          # does not end at total_q
    assert _extend_check(c, cu=cu)["flags"] & 4
    sp = c.start_pos.copy()
    sp[0] = c.block_table.shape[1] * c.block_size   # a write past the table row
    r = pg.check_contents(c.batch, block_table=to_dev(c.block_table), cu_rows=to_dev(c.cu_ctx),
                          start_pos=to_dev(sp), total_rows=int(c.cu_ctx[-1]), num_blocks=c.num_blocks,
                          block_size=c.block_size)
    assert r["flags"] == 2 and r["first_bad_sequence"] == 0


def test_debug_mode_raises_before_the_call(monkeypatch):
    c = W.make_decode_case([1, 17, 96], 8, 2, 128, 16, W.BF16, seed=3003)
    dev = DevDecode(c)
    t = c.block_table.copy()
    t[2, 1] = 10 ** 6
    monkeypatch.setattr(ops, "DEBUG_CHECKS", True)
    say("debug checks: decode with a bad table")
    out = pg.gqa_paged_decode(dev.q, dev.kc, dev.vc, dev.table, dev.ctx, c.max_context_len, scale=float(c.scale))
    with pytest.raises(pg.ContractError, match="block id outside the pool"):
        pg.gqa_paged_decode(dev.q, dev.kc, dev.vc, to_dev(t), dev.ctx, c.max_context_len, scale=float(c.scale))
    e = W.make_extend_case([0, 40], [5, 9], 8, 2, 128, 16, W.BF16, seed=3004)
    de = DevExtend(e)
    ctx = e.context_lens.copy()
    ctx[1] = 3
    with pytest.raises(pg.ContractError, match="fewer cached positions"):
        pg.gqa_paged_extend(de.q, de.cu_q, de.kc, de.vc, de.table, to_dev(ctx), e.max_q_len, e.max_context_len,
                            scale=float(e.scale))
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()


def test_launch_log(monkeypatch, capfd):
    c = W.make_decode_case([1, 17, 96], 8, 2, 128, 16, W.BF16, seed=3005)
    dev = DevDecode(c)
    e = W.make_extend_case([0, 40], [5, 9], 8, 2, 128, 16, W.BF16, seed=3006)
    de = DevExtend(e)
    capfd.readouterr()
    monkeypatch.setenv("PGQA_LOG", "1")
    say("launch log")
    pg.gqa_paged_decode(dev.q, dev.kc, dev.vc, dev.table, dev.ctx, c.max_context_len, scale=float(c.scale))
    de.extend()
    torch.cuda.synchronize()
    err = capfd.readouterr().err
    assert "pgqa: decode B=3 Hq=8 Hkv=2 d=128 bs=16 bf16" in err
    assert "pgqa: extend B=2 rows=14 Hq=8 Hkv=2 d=128" in err
    monkeypatch.setenv("PGQA_LOG", "0")
    pg.gqa_paged_decode(dev.q, dev.kc, dev.vc, dev.table, dev.ctx, c.max_context_len, scale=float(c.scale))
    torch.cuda.synchronize()
    assert "pgqa:" not in capfd.readouterr().err


def test_garbage_contents_are_reported_not_followed():
    """Extreme values in every array: each is reported, and the check reads nothing
    outside the arrays (lengths are cut to the table row)."""
    c = W.make_extend_case([0, 31, 64], [5, 33, 1], 8, 2, 128, 16, W.BF16, seed=3007)
    big = 2 ** 31 - 1
    ctx = np.array([big, -big - 1, 7], dtype=np.int32)
    cu = np.array([0, big, 5, 7], dtype=np.int32)
    t = np.full_like(c.block_table, -7)
    say("check contents: garbage")
    r = pg.check_contents(c.batch, block_table=to_dev(t), context_lens=to_dev(ctx), cu_rows=to_dev(cu),
                          total_rows=c.total_q, max_rows=c.max_q_len, num_blocks=c.num_blocks,
                          block_size=c.block_size, max_context_len=c.max_context_len, window=big)
    assert r["flags"] == 1 | 2 | 4 | 8 and r["first_bad_sequence"] == 0 and r["bad_sequences"] == 3
    sp = np.array([big, -5, 0], dtype=np.int32)
    r = pg.check_contents(c.batch, block_table=to_dev(t), cu_rows=to_dev(cu), start_pos=to_dev(sp),
                          total_rows=c.total_q, num_blocks=c.num_blocks, block_size=c.block_size)
    assert r["flags"] & 2 and r["flags"] & 4 and r["bad_sequences"] == 3
