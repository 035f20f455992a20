"""Packed varlen prefill on the GPU (bf16 MFMA) against the fp64 oracle."""

import json
from pathlib import Path

import numpy as np
import pytest
import torch

import workload as W
import paged_gqa_kv_02_amd as pg
from gpu_helpers import DevDecode, assert_close, say, to_dev, to_f64

pytestmark = pytest.mark.gpu

GOLDEN = Path(__file__).resolve().parent / "golden"


def _gpu_prefill(p: W.PrefillCase, causal=True):
    return pg.gqa_varlen_prefill(to_dev(p.q), to_dev(p.k), to_dev(p.v), to_dev(p.cu_seqlens), p.max_seqlen,
                                 scale=float(p.scale), causal=causal)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 4), (8, 2), (32, 8), (16, 1)])
@pytest.mark.parametrize("d", [64, 128])
def test_small_batches(orc, causal, hq, hkv, d):
    lens = [1, 31, 32, 33, 100, 7, 64, 129]
    p = W.make_prefill_case(lens, hq, hkv, d, 16, W.BF16, seed=hq * 10 + hkv + d, causal=causal)
    say(f"prefill small causal={causal} {hq}/{hkv} d{d}")
    out = to_f64(_gpu_prefill(p, causal))
    ref = orc.gqa_varlen_prefill(p.q, p.k, p.v, p.cu_seqlens, p.scale, causal=causal)
    assert_close(out, ref, W.BF16, f"prefill causal={causal} {hq}/{hkv} d{d}")


def test_packing_example(orc):
    g = json.loads((GOLDEN / "packing_3_9_5.json").read_text())
    p = W.make_prefill_case(g["lengths"], 32, 8, 128, 16, W.BF16, seed=5)
    say("prefill packing 3+9+5")
    out = to_f64(_gpu_prefill(p))
    assert out.shape[0] == g["total_tokens"]
    ref = orc.gqa_varlen_prefill(p.q, p.k, p.v, p.cu_seqlens, p.scale)
    assert_close(out, ref, W.BF16, "packing example")


def test_empty_sequences_in_batch(orc):
    p = W.make_prefill_case([0, 40, 0, 3, 0], 8, 2, 128, 16, W.BF16, seed=6)
    say("prefill with empty sequences")
    out = to_f64(_gpu_prefill(p))
    ref = orc.gqa_varlen_prefill(p.q, p.k, p.v, p.cu_seqlens, p.scale)
    assert_close(out, ref, W.BF16, "empty sequences")


def test_workload_every_output(orc):
    """The full varlen prefill workload (32 sequences, 16K packed rows) in the
    benchmark's launch configuration, every output element against the oracle."""
    p = W.make_workload("varlen_prefill")
    say(f"prefill workload T={p.total_tokens}")
    out = to_f64(_gpu_prefill(p))
    torch.cuda.synchronize()
    ref = orc.gqa_varlen_prefill(p.q, p.k, p.v, p.cu_seqlens, p.scale)
    e = assert_close(out, ref, W.BF16, "prefill workload")
    say(f"prefill workload: {e}")


def test_decode_equals_last_prefill_row(orc):
    """Decode over pages written from a prefill batch equals each sequence's last causal row."""
    p = W.make_prefill_case([70, 513, 1, 260], 32, 8, 128, 16, W.BF16, seed=8)
    say("cross path prefill -> decode")
    pre = to_f64(_gpu_prefill(p))
    last = p.cu_seqlens[1:] - 1
    case = W.DecodeCase(name="x", dtype=W.BF16, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                        context_lens=p.lengths, cu_ctx=p.cu_seqlens, q=np.ascontiguousarray(p.q[last]), k=p.k,
                        v=p.v, block_table=p.block_table, num_blocks=p.num_blocks, scale=p.scale)
    dec = to_f64(DevDecode(case).decode())
    ref = orc.gqa_varlen_prefill(p.q, p.k, p.v, p.cu_seqlens, p.scale, rows=last.astype(np.int32))
    assert_close(dec, ref, W.BF16, "decode of last rows")
    assert_close(pre[last], ref, W.BF16, "prefill last rows")


@pytest.mark.parametrize("batch", [64, 65])
def test_tile_list_boundary(orc, batch):
    """64 (sequence, KV head) pairs per XCD is the largest batch whose query tiles are
    listed densely per XCD (a wave-wide scan of the pairs' lengths); 65 falls back to
    one level per query tile of the longest sequence.  Ragged, empty and one-row
    sequences on both sides of that boundary."""
    rng = np.random.default_rng(batch)
    lens = rng.integers(0, 200, size=batch)
    lens[::7] = 0
    lens[3::11] = 1
    p = W.make_prefill_case(lens.tolist(), 16, 8, 64, 16, W.BF16, seed=batch)
    say(f"prefill tile-list boundary B={batch}")
    out = to_f64(_gpu_prefill(p))
    ref = orc.gqa_varlen_prefill(p.q, p.k, p.v, p.cu_seqlens, p.scale)
    assert_close(out, ref, W.BF16, f"tile-list boundary B={batch}")
