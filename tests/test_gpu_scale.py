"""Zero and negative softmax scales on the GPU against the fp64 oracle.

The kernels fold the scale into a positive exponent factor and apply its sign to
the query bits as they load them; a zero scale zeroes the query, so every
visible key gets the same weight.  Masked keys (causal diagonal, ragged tails,
NaN-filled unused slots) must still get weight 0 in every case."""

import numpy as np
import pytest
import torch

import workload as W
import paged_gqa_kv_02_amd as pg
from gpu_helpers import DevDecode, DevExtend, assert_close, oracle_decode, oracle_extend, say, to_dev, to_f64

pytestmark = pytest.mark.gpu

SCALES = [0.0, -0.0883883, -0.35]


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("hq,hkv,d,bs,dtype", [(32, 8, 128, 16, W.BF16), (4, 2, 16, 4, W.F32),
                                               (32, 1, 128, 32, W.BF16), (16, 2, 64, 8, W.BF16)])
def test_decode(orc, scale, hq, hkv, d, bs, dtype):
    case = W.make_decode_case([1, 15, 300, 1100, 0, 77], hq, hkv, d, bs, dtype, seed=1200 + hq + d, scale=scale)
    say(f"decode scale={scale} {hq}/{hkv} d{d} bs{bs} {dtype}")
    dev = DevDecode(case)
    out = to_f64(dev.decode())
    ref = oracle_decode(orc, case)
    assert_close(out, ref, dtype, f"decode scale={scale}")
    if hkv == 1:   # the split-KV kernel as well as the matrix-core route
        assert_close(to_f64(dev.decode(num_splits=37)), ref, dtype, f"decode split scale={scale}")


@pytest.mark.parametrize("scale", SCALES)
def test_decode_fp8(orc, scale):
    case = W.make_decode_case([5, 70, 300, 1], 32, 8, 128, 16, W.BF16, seed=1210, scale=scale)
    say(f"fp8 decode scale={scale}")
    kc, vc, ks, vs = pg.fp8_pools(case.num_blocks, 8, 16, 128)
    pg.paged_kv_write_fp8(to_dev(case.k), to_dev(case.v), to_dev(case.cu_ctx), to_dev(case.start_pos),
                          to_dev(case.block_table), kc, vc, ks, vs)
    got = pg.gqa_paged_decode_fp8(to_dev(case.q), kc, vc, ks, vs, to_dev(case.block_table),
                                  to_dev(case.context_lens), case.max_context_len, scale=float(scale))
    shape = (case.num_blocks, 8, 16, 128)
    hk, hv = np.full(shape, 0x7F, np.uint8), np.full(shape, 0x7F, np.uint8)
    hks, hvs = np.full(shape[:3], np.nan, np.float32), np.full(shape[:3], np.nan, np.float32)
    orc.paged_kv_write_fp8(case.k, case.v, case.cu_ctx, case.start_pos, case.block_table, hk, hv, hks, hvs)
    qd = W.bf16_bits_to_f32(case.q).astype(np.float64)
    ref = orc.gqa_paged_decode(qd, orc.dequantize_fp8(hk, hks), orc.dequantize_fp8(hv, hvs), case.block_table,
                               case.context_lens, scale)
    assert_close(to_f64(got), ref, W.BF16, f"fp8 decode scale={scale}")


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("causal", [True, False])
def test_prefill(orc, scale, causal):
    p = W.make_prefill_case([1, 31, 100, 7, 129], 32, 8, 128, 16, W.BF16, seed=1220, causal=causal, scale=scale)
    say(f"prefill scale={scale} causal={causal}")
    got = pg.gqa_varlen_prefill(to_dev(p.q), to_dev(p.k), to_dev(p.v), to_dev(p.cu_seqlens), p.max_seqlen,
                                scale=float(scale), causal=causal)
    ref = orc.gqa_varlen_prefill(p.q, p.k, p.v, p.cu_seqlens, scale, causal=causal)
    assert_close(to_f64(got), ref, W.BF16, f"prefill scale={scale} causal={causal}")


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("prefix,q_lens,hq,hkv", [([0, 37, 300, 2000], [5, 40, 1, 64], 32, 8),
                                                  ([3000, 17, 4000, 64], [4, 4, 4, 4], 8, 2)])
def test_extend(orc, scale, prefix, q_lens, hq, hkv):
    c = W.make_extend_case(prefix, q_lens, hq, hkv, 128, 16, W.BF16, seed=1230 + hq, scale=scale)
    say(f"extend scale={scale} {hq}/{hkv}")
    out = to_f64(DevExtend(c).extend())
    assert_close(out, oracle_extend(orc, c), W.BF16, f"extend scale={scale}")
    torch.cuda.synchronize()
