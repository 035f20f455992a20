"""Parity at the sizes the boundary allows at its extremes: one 256K-token
context (decode, and few query tokens over it through the key split), the
largest decode batch, and a long packed prefill sequence, each checked against
the fp64 oracle (all outputs, or sampled rows the oracle evaluates one by one)."""

import numpy as np
import pytest
import torch

import workload as W
import paged_gqa_kv_02_amd as pg
from gpu_helpers import DevDecode, DevExtend, assert_close, oracle_decode, oracle_extend, say, to_dev, to_f64

pytestmark = pytest.mark.gpu

LONG = 262144


def test_decode_256k_context(orc):
    case = W.make_decode_case([LONG, 5], 32, 8, 128, 16, W.BF16, seed=3000)
    say(f"decode {LONG}-token context")
    out = to_f64(DevDecode(case).decode())
    assert_close(out, oracle_decode(orc, case), W.BF16, "decode 256K")


def test_few_queries_over_256k_context(orc):
    c = W.make_extend_case([LONG - 4, 3000], [4, 4], 32, 8, 128, 16, W.BF16, seed=3001)
    assert pg.gqa_paged_extend_workspace_size(c.batch, c.total_q, c.max_q_len, 32, 8, 128, c.max_context_len) > 0
    say(f"multi-token (4 queries) over a {LONG}-token context")
    out = to_f64(DevExtend(c).extend())
    assert_close(out, oracle_extend(orc, c), W.BF16, "extend 256K")


def test_largest_decode_batch(orc):
    lens = np.random.default_rng(3002).integers(1, 65, size=8192).astype(np.int32)
    case = W.make_decode_case(lens, 8, 2, 64, 16, W.BF16, seed=3002)
    say("decode batch 8192")
    out = to_f64(DevDecode(case).decode())
    assert_close(out, oracle_decode(orc, case), W.BF16, "decode B=8192")


def test_long_prefill_sequence(orc):
    p = W.make_prefill_case([16384, 100], 32, 8, 128, 16, W.BF16, seed=3003)
    say("prefill 16384-token sequence")
    out = to_f64(pg.gqa_varlen_prefill(to_dev(p.q), to_dev(p.k), to_dev(p.v), to_dev(p.cu_seqlens), p.max_seqlen,
                                       scale=float(p.scale)))
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 16383, 16384, 16483],
                                     np.random.default_rng(0).integers(0, 16384, 40)])).astype(np.int32)
    ref = orc.gqa_varlen_prefill(p.q, p.k, p.v, p.cu_seqlens, p.scale, rows=rows)
    assert_close(out[rows], ref, W.BF16, "prefill 16K rows")
