"""Paged GQA decode on the GPU against the fp64 oracle."""

import numpy as np
import pytest
import torch

import workload as W
from gpu_helpers import DevDecode, assert_close, oracle_decode, say, to_bits, to_dev, to_f64

pytestmark = pytest.mark.gpu

DECODE_WORKLOADS = ["tiny_f32", "llama3_8b_decode", "long_ctx_decode", "mqa_decode"]


@pytest.mark.parametrize("key", DECODE_WORKLOADS)
def test_workload_matches_oracle(orc, key):
    """Full-size workloads, in the launch configuration the benchmark times (library split choice)."""
    case = W.make_workload(key)
    say(f"decode {key} B={case.batch} Hq={case.num_q_heads} Hkv={case.num_kv_heads}")
    dev = DevDecode(case)
    out = to_f64(dev.decode())
    torch.cuda.synchronize()
    ref = oracle_decode(orc, case)
    e = assert_close(out, ref, case.dtype, key)
    say(f"decode {key}: {e}")


@pytest.mark.parametrize("key", ["llama3_8b_decode", "mqa_decode"])
def test_sharpened_queries(orc, key):
    """q scaled by 4 (exact in bf16) makes the softmax peaked and the outputs O(1)."""
    case = W.make_workload(key)
    q4 = W.f32_to_bf16_bits(W.bf16_bits_to_f32(case.q) * np.float32(4.0))
    case.q = q4
    say(f"decode sharpened {key}")
    out = to_f64(DevDecode(case).decode())
    ref = oracle_decode(orc, case)
    assert np.abs(ref).max() > 0.5
    assert_close(out, ref, case.dtype, f"sharpened {key}")


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("hq,hkv", [(4, 4), (4, 2), (8, 2), (16, 2), (8, 1), (16, 1), (32, 1), (64, 1)])
def test_shapes(orc, dtype, d, hq, hkv):
    lens = [1, 17, 96, 203, 3]
    case = W.make_decode_case(lens, hq, hkv, d, 16, dtype, seed=hq * 100 + hkv * 10 + d)
    say(f"decode shape {dtype} d{d} {hq}/{hkv}")
    out = to_f64(DevDecode(case).decode())
    assert_close(out, oracle_decode(orc, case), dtype, f"{dtype} d{d} {hq}/{hkv}")


@pytest.mark.parametrize("bs", [1, 2, 4, 8, 16, 32, 64, 256])
def test_block_sizes(orc, bs):
    case = W.make_decode_case([1, bs, bs + 1, 3 * bs - 1, 150], 8, 2, 128, bs, W.BF16, seed=300 + bs)
    say(f"decode bs{bs}")
    out = to_f64(DevDecode(case).decode())
    assert_close(out, oracle_decode(orc, case), W.BF16, f"bs{bs}")


def test_edge_contexts(orc):
    """Empty, single-token, page- and tile-aligned and ragged contexts in one batch."""
    lens = [0, 1, 15, 16, 17, 31, 32, 33, 64, 65, 0, 1000]
    case = W.make_decode_case(lens, 32, 8, 128, 16, W.BF16, seed=41)
    say("decode edge contexts")
    out = to_f64(DevDecode(case).decode())
    ref = oracle_decode(orc, case)
    assert np.all(out[0] == 0) and np.all(out[10] == 0), "empty context must give zeros"
    assert_close(out, ref, W.BF16, "edge contexts")


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 64, 997, 4096])
def test_split_counts(orc, splits):
    """Any split of the work gives the oracle's answer and is deterministic run to run."""
    case = W.make_decode_case([700, 33, 2100, 1, 0, 4096, 515], 32, 8, 128, 16, W.BF16, seed=51)
    say(f"decode splits={splits}")
    dev = DevDecode(case)
    a = dev.decode(num_splits=splits)
    b = dev.decode(num_splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "not deterministic"
    assert_close(to_f64(a), oracle_decode(orc, case), W.BF16, f"splits={splits}")


def test_placement_invariance():
    """Another page permutation, a bigger pool and extra table columns: bit-identical output."""
    case = W.make_decode_case([300, 45, 1024, 7], 32, 8, 128, 16, W.BF16, seed=61)
    say("decode placement invariance")
    base = DevDecode(case).decode(num_splits=5)
    table, nb = W.place_pages(np.random.default_rng(5), case.context_lens, 16, pool_factor=3.0, extra_cols=9)
    moved = DevDecode(case, table=table, num_blocks=nb).decode(num_splits=5)
    torch.cuda.synchronize()
    assert torch.equal(base.view(torch.int16), moved.view(torch.int16))


def test_batch_independence():
    """A sequence's output does not depend on the rest of its batch (single share each)."""
    case = W.make_decode_case([300, 45, 1024, 7], 8, 2, 128, 16, W.BF16, seed=62)
    say("decode batch independence")
    full = DevDecode(case).decode(num_splits=1)
    for b in range(case.batch):
        a, e = int(case.cu_ctx[b]), int(case.cu_ctx[b + 1])
        one = W.make_decode_case([int(case.context_lens[b])], 8, 2, 128, 16, W.BF16, seed=63)
        one.q, one.k, one.v = case.q[b:b + 1].copy(), case.k[a:e].copy(), case.v[a:e].copy()
        alone = DevDecode(one).decode(num_splits=1)
        torch.cuda.synchronize()
        assert torch.equal(alone[0].view(torch.int16), full[b].view(torch.int16)), f"sequence {b}"


def test_gqa_equals_repeated_mha():
    """GQA(32, 8) on the GPU equals MHA(32) with each KV head repeated 4 times, bit for
    bit: with one share per call every (sequence, KV head) segment is computed whole,
    and a query head's scores, weights and sums take the same steps in either grouping."""
    case = W.make_decode_case([130, 77], 32, 8, 128, 16, W.BF16, seed=64)
    mha = W.make_decode_case([130, 77], 32, 32, 128, 16, W.BF16, seed=64)
    mha.q = case.q
    mha.k = np.repeat(case.k, 4, axis=1)
    mha.v = np.repeat(case.v, 4, axis=1)
    say("decode GQA vs repeated MHA")
    g = DevDecode(case).decode(num_splits=1)
    m = DevDecode(mha).decode(num_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(g.view(torch.int16), m.view(torch.int16))


def test_workspace_reuse(orc):
    """One workspace reused across calls (different split counts and batches,
    stale partials from the previous call left in it): outputs stay correct."""
    import paged_gqa_kv_02_amd as pg
    case = W.make_decode_case([700, 33, 2100, 1, 0, 4096, 515], 32, 8, 128, 16, W.BF16, seed=71)
    small = W.make_decode_case([300, 45], 32, 8, 128, 16, W.BF16, seed=72)
    dev, dev_s = DevDecode(case), DevDecode(small)
    ws = pg.decode_workspace(case.batch, 32, 8, 128, 0)
    ref = oracle_decode(orc, case)
    ref_s = oracle_decode(orc, small)
    for splits in (0, 3, 97, 0):
        say(f"decode workspace reuse splits={splits}")
        out = pg.gqa_paged_decode(dev.q, dev.kc, dev.vc, dev.table, dev.ctx, case.max_context_len,
                                  scale=float(case.scale), num_splits=splits, workspace=ws)
        out_s = pg.gqa_paged_decode(dev_s.q, dev_s.kc, dev_s.vc, dev_s.table, dev_s.ctx, small.max_context_len,
                                    scale=float(small.scale), num_splits=splits, workspace=ws)
        torch.cuda.synchronize()
        assert_close(to_f64(out), ref, W.BF16, f"reuse splits={splits}")
        assert_close(to_f64(out_s), ref_s, W.BF16, f"reuse small splits={splits}")


@pytest.mark.parametrize("hq,d,bs", [(32, 128, 16), (32, 64, 8), (64, 128, 4), (32, 128, 256)])
def test_one_kv_head_matrix_core_route(orc, hq, d, bs):
    """One KV head and Hq a multiple of 32 run on the matrix cores (query heads as
    tile rows; G = 32: the batch's key blocks in equal stream-K shares, G = 64: key
    chunks of 20 blocks of 64): empty, one-token, page- and chunk-edge and long
    contexts against the oracle, sharpened queries too, deterministic, and within
    tolerance of the split-KV kernel (an explicit split count keeps that path)."""
    lens = [0, 1, bs - 1, bs, bs + 1, 1023, 1024, 1025, 1279, 1280, 1281, 2561, 3000, 5000]
    case = W.make_decode_case(lens, hq, 1, d, bs, W.BF16, seed=hq * 7 + d + bs)
    say(f"decode one KV head hq={hq} d{d} bs{bs}")
    dev = DevDecode(case)
    out = dev.decode()
    again = dev.decode()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), again.view(torch.int16)), "not deterministic"
    ref = oracle_decode(orc, case)
    assert_close(to_f64(out), ref, W.BF16, f"one KV head hq={hq} d{d} bs{bs}")
    assert not to_f64(out)[0].any(), "empty context must give zeros"
    split = dev.decode(num_splits=97)
    torch.cuda.synchronize()
    assert_close(to_f64(split), ref, W.BF16, "split-KV path")
    q4 = W.f32_to_bf16_bits(W.bf16_bits_to_f32(case.q) * np.float32(4.0))
    case.q = q4
    sharp = to_f64(DevDecode(case).decode())
    assert_close(sharp, oracle_decode(orc, case), W.BF16, "sharpened")


def test_one_kv_head_many_sequences(orc, monkeypatch, capfd):
    """More sequences than the stream-K scan takes (4,096 pairs): the one-KV-head
    route falls back to key chunks, still against the oracle."""
    rng = np.random.default_rng(1480)
    lens = rng.integers(0, 120, 4100)
    case = W.make_decode_case(lens, 32, 1, 128, 16, W.BF16, seed=1481)
    say("decode one KV head, 4100 sequences")
    dev = DevDecode(case)
    capfd.readouterr()
    monkeypatch.setenv("PGQA_LOG", "1")
    out = dev.decode()
    torch.cuda.synchronize()
    monkeypatch.setenv("PGQA_LOG", "0")
    err = capfd.readouterr().err
    assert "stream-K" not in err and "extend B=4100" in err, err
    assert_close(to_f64(out), oracle_decode(orc, case), W.BF16, "4100 sequences")
