"""gqa_paged_decode_noalloc (the library's own per-GPU scratch in place of the
caller's workspace) against gqa_paged_decode, through the C ABI: two calls in a
row, the second on a smaller batch, then the one-KV-head matrix-core route and an
explicit split count.  The two entry points run the same kernels with the same
split, so their outputs must be bit-identical."""

import numpy as np
import pytest
import torch

import workload as W
from paged_gqa_kv_02_amd import _lib
from gpu_helpers import DevDecode, assert_close, oracle_decode, say, to_f64

pytestmark = pytest.mark.gpu


def _noalloc(dev: DevDecode, num_splits: int = 0) -> torch.Tensor:
    c = dev.case
    out = torch.empty_like(dev.q)
    B, hq, d = dev.q.shape
    nb, hkv, bs, _ = dev.kc.shape
    st = _lib.lib().gqa_paged_decode_noalloc(
        dev.q.data_ptr(), dev.kc.data_ptr(), dev.vc.data_ptr(), dev.table.data_ptr(), dev.table.shape[1],
        dev.ctx.data_ptr(), B, hq, hkv, d, bs, nb, int(c.max_context_len), float(c.scale), 0,
        _lib.PGQA_BF16 if dev.q.dtype == torch.bfloat16 else _lib.PGQA_F32, out.data_ptr(), int(num_splits),
        torch.cuda.current_stream().cuda_stream)
    assert st == 0, f"gqa_paged_decode_noalloc returned {_lib.STATUS.get(st, st)}"
    return out


def _same(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.int16), b.view(torch.int16)) if a.dtype == torch.bfloat16 else torch.equal(a, b)


def test_two_calls_in_a_row_then_smaller(orc):
    big = W.make_workload("llama3_8b_decode")
    small = W.make_decode_case([5, 70, 300, 1, 0], 32, 8, 128, 16, W.BF16, seed=1401)
    dev_b, dev_s = DevDecode(big), DevDecode(small)
    say("no-alloc decode: llama3_8b_decode")
    got_b = _noalloc(dev_b)
    ref_b = dev_b.decode()
    say("no-alloc decode: smaller batch")
    got_s = _noalloc(dev_s)
    ref_s = dev_s.decode()
    torch.cuda.synchronize()
    assert _same(got_b, ref_b), "large batch differs from gqa_paged_decode"
    assert _same(got_s, ref_s), "small batch differs from gqa_paged_decode"
    assert_close(to_f64(got_s), oracle_decode(orc, small), W.BF16, "no-alloc small batch")


@pytest.mark.parametrize("hq,hkv,d,bs,dtype,splits", [(32, 1, 128, 32, W.BF16, 0), (32, 8, 128, 16, W.BF16, 97),
                                                      (4, 2, 16, 4, W.F32, 0)])
def test_routes(orc, hq, hkv, d, bs, dtype, splits):
    case = W.make_decode_case([1, 33, 1025, 4000, 0, 260], hq, hkv, d, bs, dtype, seed=1410 + hq + hkv)
    dev = DevDecode(case)
    say(f"no-alloc decode {hq}/{hkv} d{d} bs{bs} {dtype} splits={splits}")
    got = _noalloc(dev, splits)
    ref = dev.decode(num_splits=splits)
    again = _noalloc(dev, splits)
    torch.cuda.synchronize()
    assert _same(got, ref) and _same(again, ref)
    assert_close(to_f64(got), oracle_decode(orc, case), dtype, "no-alloc route")
