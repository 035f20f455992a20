"""The seeded input generator: rounding, recipe, and the pages' paging figures."""

import json
import math
from pathlib import Path

import numpy as np
import pytest
import torch

import workload as W

GOLDEN = Path(__file__).resolve().parent / "golden"


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(200_000, dtype=np.float32)
    # add exact ties (low 16 bits == 0x8000) with both even and odd kept parts
    ties = (np.arange(1, 2001, dtype=np.uint32) << np.uint32(16)) | np.uint32(0x8000)
    x = np.concatenate([x, ties.view(np.float32), -ties.view(np.float32)])
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    # widening back is exact
    assert np.array_equal(W.f32_to_bf16_bits(W.bf16_bits_to_f32(ours)), ours)


def test_same_seed_same_inputs():
    a = W.make_decode_case([7, 3], 4, 2, 16, 4, W.BF16, seed=5)
    b = W.make_decode_case([7, 3], 4, 2, 16, 4, W.BF16, seed=5)
    for f in ("q", "k", "v", "block_table"):
        assert np.array_equal(getattr(a, f), getattr(b, f))


def test_tiny_workload_recipe():
    c = W.make_workload("tiny_f32")
    assert c.context_lens.tolist() == [5, 11]
    assert c.num_blocks == 8 and c.block_size == 4
    assert c.q.shape == (2, 4, 16) and c.k.shape == (16, 2, 16) and c.q.dtype == np.float32
    assert c.scale == np.float32(0.25)
    # sequence 0 takes permutation[0:2], sequence 1 permutation[2:5], the rest unused
    rng = np.random.default_rng(1)
    rng.standard_normal(size=(2, 4, 16), dtype=np.float32)
    rng.standard_normal(size=(16, 2, 16), dtype=np.float32)
    rng.standard_normal(size=(16, 2, 16), dtype=np.float32)
    perm = rng.permutation(8)
    assert c.block_table[0, :2].tolist() == perm[0:2].tolist()
    assert c.block_table[1, :3].tolist() == perm[2:5].tolist()
    assert c.block_table[0, 2] == -1


@pytest.mark.parametrize("key,lo,hi,n", [("llama3_8b_decode", 512, 4096, 64),
                                         ("mqa_decode", 16, 8192, 256),
                                         ("varlen_prefill", 64, 1024, 32),
                                         ("chunked_prefill", 0, 3072, 16),
                                         ("spec_verify", 508, 4092, 64),
                                         ("shared_prefix_decode", 64, 2048, 64)])
def test_length_recipes(key, lo, hi, n):
    lens = W.workload_lengths(key, np.random.default_rng(W.WORKLOADS[key].seed))
    assert lens.shape == (n,) and lens.min() >= lo and lens.max() <= hi


def test_mqa_lengths_lognormal_median():
    lens = W.workload_lengths("mqa_decode", np.random.default_rng(4))
    assert 700 <= np.median(lens) <= 1400


def test_long_context_pool_size():
    lens = W.workload_lengths("long_ctx_decode", np.random.default_rng(3))
    table, nb = W.place_pages(np.random.default_rng(0), lens, 16)
    assert nb == 20480 and table.shape == (8, 2048)
    used = table[table >= 0]
    assert len(np.unique(used)) == used.size == 16384 and used.max() < nb


def test_paging_waste_below_one_block():
    """Paged placement wastes fewer than block_size slots per sequence, unlike a
    contiguous max-length reservation (the pages' 2048-reserved/10-used example)."""
    g = json.loads((GOLDEN / "fragmentation.json").read_text())
    for ex in g["contiguous"]:
        assert ex["reserved"] - ex["used"] == ex["wasted"]
        bs = g["block_size"]
        pages = W.pages_needed([ex["used"]], bs)[0]
        waste = pages * bs - ex["used"]
        assert 0 <= waste < bs < ex["wasted"]
    lens = np.random.default_rng(7).integers(1, 300, size=50)
    for bs in (1, 4, 16, 32):
        pages = W.pages_needed(lens, bs)
        assert np.all(pages * bs - lens < bs) and np.all(pages * bs >= lens)


def test_gqa_cache_reduction_factor():
    """Pool bytes shrink by Hq / Hkv against one KV head per query head."""
    g = json.loads((GOLDEN / "gqa_cache_reduction.json").read_text())
    for case in g["cases"]:
        gqa = W.nan_pool(3, case["num_kv_heads"], 16, 8, W.BF16).nbytes
        mha = W.nan_pool(3, case["num_q_heads"], 16, 8, W.BF16).nbytes
        assert mha // gqa == case["reduction"] and mha % gqa == 0


def test_kv_bytes_and_flops_accounting():
    c = W.make_decode_case([10, 20], 8, 2, 16, 4, W.BF16, 3)
    assert c.kv_bytes() == 30 * 2 * 16 * 2 * 2
    assert c.flops() == 30 * 8 * 4 * 16
    p = W.make_prefill_case([3, 4], 4, 2, 8, 4, W.BF16, 3)
    assert p.flops() == (6 + 10) * 4 * 4 * 8


def test_shared_prefix_case_accounting():
    c = W.make_shared_prefix_case(20, [3, 5], 4, 2, 8, 4, W.BF16, 9)
    row = 2 * 8 * 2 * 2
    assert c.logical_kv_bytes() == (23 + 25) * row and c.unique_kv_bytes() == (20 + 8) * row
    u = c.logical(np.random.default_rng(0))
    assert u.context_lens.tolist() == [23, 25]
    # sample 1 reads the prompt, then its own continuation rows
    assert np.array_equal(u.k[23:43], c.k_prompt) and np.array_equal(u.k[43:48], c.k_cont[3:8])
