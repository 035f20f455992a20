"""The hot path captured in a HIP graph (as bench.py replays it): every replay
matches the eager launch bit for bit, with other GPU work and synchronisations
between the replays, and matches the oracle."""

import numpy as np
import pytest
import torch

import paged_gqa_kv_02_amd as pg
import workload as W
from gpu_helpers import DevDecode, assert_close, oracle_decode, say, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _newest_token_write(case):
    """Inputs of the per-step paged write of each sequence's newest token."""
    live = [b for b in range(case.batch) if case.context_lens[b] > 0]
    last = case.cu_ctx[1:][live] - 1
    k_new, v_new = to_dev(np.ascontiguousarray(case.k[last])), to_dev(np.ascontiguousarray(case.v[last]))
    cu_new = to_dev(np.arange(len(live) + 1, dtype=np.int32))
    sp_new = to_dev((case.context_lens[live] - 1).astype(np.int32))
    table = to_dev(np.ascontiguousarray(case.block_table[live]))
    return k_new, v_new, cu_new, sp_new, table


def test_decode_step_graph_replays(orc):
    case = W.make_decode_case([700, 33, 2100, 1, 0, 4096, 515, 64], 32, 8, 128, 16, W.BF16, seed=81)
    dev = DevDecode(case)
    k_new, v_new, cu_new, sp_new, wtable = _newest_token_write(case)
    ws = pg.decode_workspace(case.batch, 32, 8, 128, 0)
    out = torch.empty_like(dev.q)

    def step():
        pg.paged_kv_write(k_new, v_new, cu_new, sp_new, wtable, dev.kc, dev.vc)
        pg.gqa_paged_decode(dev.q, dev.kc, dev.vc, dev.table, dev.ctx, case.max_context_len,
                            scale=float(case.scale), out=out, workspace=ws)

    say("graph: eager decode step")
    step()
    torch.cuda.synchronize()
    eager = out.clone()
    assert_close(to_f64(eager), oracle_decode(orc, case), W.BF16, "eager step")

    say("graph: capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        say(f"graph: replay {r}")
        out.fill_(0)
        other = dev.decode(num_splits=7)          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {r} differs from eager"
        assert other.isfinite().all()


def test_prefill_graph_replays(orc):
    p = W.make_prefill_case([70, 513, 1, 260, 0, 33], 32, 8, 128, 16, W.BF16, seed=82)
    q, k, v = to_dev(p.q), to_dev(p.k), to_dev(p.v)
    cu = to_dev(p.cu_seqlens)
    out = torch.empty_like(q)

    def call():
        pg.gqa_varlen_prefill(q, k, v, cu, p.max_seqlen, scale=float(p.scale), causal=True, out=out)

    say("graph: eager prefill")
    call()
    torch.cuda.synchronize()
    eager = out.clone()
    ref = orc.gqa_varlen_prefill(p.q, p.k, p.v, p.cu_seqlens, p.scale, causal=True)
    assert_close(to_f64(eager), ref, W.BF16, "eager prefill")
    say("graph: capture prefill")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for r in range(3):
        say(f"graph: prefill replay {r}")
        out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"prefill replay {r} differs"
