"""The torch front end refuses tensors that disagree with one another before any
C call: the C ABI sees raw pointers only, so a dtype or shape mismatch caught
nowhere else would make a kernel read or write past a buffer.  CPU tensors are
used throughout: every mismatch is reported before the device check."""

import pytest
import torch

import paged_gqa_kv_02_amd as pg

B, HQ, HKV, D, BS, NB, MAXB = 3, 8, 2, 64, 16, 20, 4
bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32


def _decode_args(**kw):
    a = dict(q=torch.zeros(B, HQ, D, dtype=bf), k_cache=torch.zeros(NB, HKV, BS, D, dtype=bf),
             v_cache=torch.zeros(NB, HKV, BS, D, dtype=bf), block_table=torch.zeros(B, MAXB, dtype=i32),
             context_lens=torch.zeros(B, dtype=i32), max_context_len=BS * MAXB, scale=0.125)
    a.update(kw)
    return a


def test_consistent_decode_reaches_the_device_check():
    with pytest.raises(ValueError, match="on the GPU"):
        pg.gqa_paged_decode(**_decode_args())


@pytest.mark.parametrize("bad,exc", [
    (dict(k_cache=torch.zeros(NB, HKV, BS, D, dtype=f32), v_cache=torch.zeros(NB, HKV, BS, D, dtype=f32)), TypeError),
    (dict(v_cache=torch.zeros(NB, HKV, BS, D, dtype=f32)), TypeError),
    (dict(v_cache=torch.zeros(NB + 1, HKV, BS, D, dtype=bf)), ValueError),
    (dict(out=torch.zeros(B, HQ, D, dtype=f32)), TypeError),
    (dict(out=torch.zeros(B + 1, HQ, D, dtype=bf)), ValueError),
    (dict(context_lens=torch.zeros(B + 1, dtype=i32)), ValueError),
    (dict(block_table=torch.zeros(B - 1, MAXB, dtype=i32)), ValueError),
    (dict(block_table=torch.zeros(B * MAXB, dtype=i32)), ValueError),
    (dict(q=torch.zeros(B, HQ, 2 * D, dtype=bf)), ValueError),
])
def test_decode_mismatches(bad, exc):
    with pytest.raises(exc):
        pg.gqa_paged_decode(**_decode_args(**bad))


def _write_args(**kw):
    T = 10
    a = dict(k=torch.zeros(T, HKV, D, dtype=bf), v=torch.zeros(T, HKV, D, dtype=bf),
             cu_seqlens=torch.tensor([0, 3, 7, 10], dtype=i32), start_pos=torch.zeros(B, dtype=i32),
             block_table=torch.zeros(B, MAXB, dtype=i32), k_cache=torch.zeros(NB, HKV, BS, D, dtype=bf),
             v_cache=torch.zeros(NB, HKV, BS, D, dtype=bf))
    a.update(kw)
    return a


def test_consistent_write_reaches_the_device_check():
    with pytest.raises(ValueError, match="on the GPU"):
        pg.paged_kv_write(**_write_args())


@pytest.mark.parametrize("bad,exc", [
    (dict(k=torch.zeros(10, HKV, D, dtype=f32), v=torch.zeros(10, HKV, D, dtype=f32)), TypeError),
    (dict(k=torch.zeros(10, HKV + 1, D, dtype=bf), v=torch.zeros(10, HKV + 1, D, dtype=bf)), ValueError),
    (dict(v=torch.zeros(9, HKV, D, dtype=bf)), ValueError),
    (dict(cu_seqlens=torch.tensor([0, 10], dtype=i32)), ValueError),
    (dict(block_table=torch.zeros(B + 2, MAXB, dtype=i32)), ValueError),
])
def test_write_mismatches(bad, exc):
    with pytest.raises(exc):
        pg.paged_kv_write(**_write_args(**bad))


def test_write_dtype_mismatch_is_a_type_error():
    with pytest.raises(TypeError):
        pg.paged_kv_write(**_write_args(v=torch.zeros(10, HKV, D, dtype=f32)))


def _prefill_args(**kw):
    T = 12
    a = dict(q=torch.zeros(T, HQ, D, dtype=bf), k=torch.zeros(T, HKV, D, dtype=bf), v=torch.zeros(T, HKV, D, dtype=bf),
             cu_seqlens=torch.tensor([0, 5, 12], dtype=i32), max_seqlen=7, scale=0.125)
    a.update(kw)
    return a


def test_consistent_prefill_reaches_the_device_check():
    with pytest.raises(ValueError, match="on the GPU"):
        pg.gqa_varlen_prefill(**_prefill_args())


@pytest.mark.parametrize("bad,exc", [
    (dict(k=torch.zeros(11, HKV, D, dtype=bf)), ValueError),
    (dict(v=torch.zeros(13, HKV, D, dtype=bf)), ValueError),
    (dict(k=torch.zeros(12, HKV, D, dtype=f32), v=torch.zeros(12, HKV, D, dtype=f32)), TypeError),
    (dict(out=torch.zeros(12, HQ, D, dtype=f32)), TypeError),
    (dict(out=torch.zeros(12, HQ + 1, D, dtype=bf)), ValueError),
])
def test_prefill_mismatches(bad, exc):
    with pytest.raises(exc):
        pg.gqa_varlen_prefill(**_prefill_args(**bad))


def _extend_args(**kw):
    a = dict(q=torch.zeros(9, HQ, D, dtype=bf), cu_q=torch.tensor([0, 2, 5, 9], dtype=i32),
             k_cache=torch.zeros(NB, HKV, BS, D, dtype=bf), v_cache=torch.zeros(NB, HKV, BS, D, dtype=bf),
             block_table=torch.zeros(B, MAXB, dtype=i32), context_lens=torch.zeros(B, dtype=i32), max_q_len=4,
             max_context_len=BS * MAXB, scale=0.125)
    a.update(kw)
    return a


def test_consistent_extend_reaches_the_device_check():
    with pytest.raises(ValueError, match="on the GPU"):
        pg.gqa_paged_extend(**_extend_args())


@pytest.mark.parametrize("bad,exc", [
    (dict(context_lens=torch.zeros(B - 1, dtype=i32)), ValueError),
    (dict(block_table=torch.zeros(B + 1, MAXB, dtype=i32)), ValueError),
    (dict(k_cache=torch.zeros(NB, HKV, BS, D, dtype=f32), v_cache=torch.zeros(NB, HKV, BS, D, dtype=f32)), TypeError),
    (dict(out=torch.zeros(9, HQ, D // 2, dtype=bf)), ValueError),
])
def test_extend_mismatches(bad, exc):
    with pytest.raises(exc):
        pg.gqa_paged_extend(**_extend_args(**bad))


def test_fp8_mismatches():
    u8 = torch.uint8
    kc, vc = torch.zeros(NB, HKV, BS, D, dtype=u8), torch.zeros(NB, HKV, BS, D, dtype=u8)
    ks, vs = torch.zeros(NB, HKV, BS, dtype=f32), torch.zeros(NB, HKV, BS, dtype=f32)
    w = _write_args()
    args = (w["k"], w["v"], w["cu_seqlens"], w["start_pos"], w["block_table"])
    with pytest.raises(ValueError, match="on the GPU"):
        pg.paged_kv_write_fp8(*args, kc, vc, ks, vs)
    with pytest.raises(ValueError):
        pg.paged_kv_write_fp8(*args, kc, vc, torch.zeros(NB, HKV, BS + 1, dtype=f32), vs)
    with pytest.raises(TypeError):
        pg.paged_kv_write_fp8(torch.zeros(10, HKV, D, dtype=f32), torch.zeros(10, HKV, D, dtype=f32), *args[2:],
                              kc, vc, ks, vs)
    d = _decode_args()
    with pytest.raises(ValueError, match="on the GPU"):
        pg.gqa_paged_decode_fp8(d["q"], kc, vc, ks, vs, d["block_table"], d["context_lens"], d["max_context_len"],
                                scale=0.125)
    with pytest.raises(ValueError):
        pg.gqa_paged_decode_fp8(d["q"], kc, vc, ks, vs, d["block_table"], torch.zeros(B + 1, dtype=i32),
                                d["max_context_len"], scale=0.125)
    with pytest.raises(TypeError):
        pg.gqa_paged_decode_fp8(d["q"].float(), kc, vc, ks, vs, d["block_table"], d["context_lens"],
                                d["max_context_len"], scale=0.125)


def test_scale_is_required():
    a = _decode_args()
    del a["scale"]
    with pytest.raises(TypeError):
        pg.gqa_paged_decode(**a)
