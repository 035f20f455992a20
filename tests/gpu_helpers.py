"""Helpers for the GPU parity tests: moving generator arrays to the device bit for
bit, running the HIP calls, and comparing against the oracle."""

from __future__ import annotations

import sys

import numpy as np
import torch

import workload as W
import paged_gqa_kv_02_amd as pg

# Parity bar against the fp64 oracle.
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
BF16_REL_RMS = 1e-2       # guards against near-zero outputs passing the absolute bounds
F32_MAX_ABS = 1e-5


def say(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a failure can be placed."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    if a.dtype in (np.float32, np.int32):
        return torch.from_numpy(a).cuda()
    raise TypeError(a.dtype)


def to_bits(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host array with the same bytes (uint16 bits for bf16)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def nan_pool_dev(num_blocks, hkv, bs, d, dtype: str) -> torch.Tensor:
    shape = (num_blocks, hkv, bs, d)
    if dtype == W.BF16:
        return torch.full(shape, 0x7FC0, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    return torch.full(shape, 0x7FC00000, dtype=torch.int32, device="cuda").view(torch.float32)


class DevDecode:
    """A decode case resident on the GPU, its pools written by the HIP kernel."""

    def __init__(self, case: W.DecodeCase, table=None, num_blocks=None):
        self.case = case
        table = case.block_table if table is None else table
        nb = case.num_blocks if num_blocks is None else num_blocks
        self.q = to_dev(case.q)
        self.table = to_dev(table)
        self.ctx = to_dev(case.context_lens)
        self.kc = nan_pool_dev(nb, case.num_kv_heads, case.block_size, case.head_dim, case.dtype)
        self.vc = nan_pool_dev(nb, case.num_kv_heads, case.block_size, case.head_dim, case.dtype)
        k, v = to_dev(case.k), to_dev(case.v)
        pg.paged_kv_write(k, v, to_dev(case.cu_ctx), to_dev(case.start_pos), self.table, self.kc, self.vc)
        del k, v

    def decode(self, num_splits: int = 0, q: torch.Tensor = None) -> torch.Tensor:
        c = self.case
        return pg.gqa_paged_decode(self.q if q is None else q, self.kc, self.vc, self.table, self.ctx,
                                   c.max_context_len, scale=float(c.scale), num_splits=num_splits)


def oracle_pools(orc, case: W.DecodeCase, table=None, num_blocks=None):
    table = case.block_table if table is None else table
    nb = case.num_blocks if num_blocks is None else num_blocks
    kc = W.nan_pool(nb, case.num_kv_heads, case.block_size, case.head_dim, case.dtype)
    vc = W.nan_pool(nb, case.num_kv_heads, case.block_size, case.head_dim, case.dtype)
    orc.paged_kv_write(case.k, case.v, case.cu_ctx, case.start_pos, table, kc, vc)
    return kc, vc


def oracle_decode(orc, case: W.DecodeCase, q=None) -> np.ndarray:
    kc, vc = oracle_pools(orc, case)
    return orc.gqa_paged_decode(case.q if q is None else q, kc, vc, case.block_table, case.context_lens,
                                case.scale)


def errors(got: np.ndarray, ref: np.ndarray) -> dict:
    err = np.abs(got - ref)
    rms_ref = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    return {"max_abs": float(err.max()) if err.size else 0.0,
            "mean_abs": float(err.mean()) if err.size else 0.0,
            "rel_rms": float(np.sqrt(np.mean(err * err)) / rms_ref) if rms_ref > 0 else 0.0}


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "") -> dict:
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    e = errors(got, ref)
    if dtype == W.BF16:
        ok = (e["max_abs"] <= BF16_MAX_ABS and e["mean_abs"] <= BF16_MEAN_ABS
              and (e["rel_rms"] <= BF16_REL_RMS or np.abs(ref).max() == 0))
    else:
        ok = e["max_abs"] <= F32_MAX_ABS
    assert ok, f"{what}: {e}"
    return e


class DevExtend:
    """A multi-token-query case resident on the GPU, its pools written by the HIP kernel."""

    def __init__(self, case: W.ExtendCase, context_lens=None):
        self.case = case
        self.q = to_dev(case.q)
        self.cu_q = to_dev(case.cu_q)
        self.table = to_dev(case.block_table)
        self.ctx_np = case.context_lens if context_lens is None else np.asarray(context_lens, np.int32)
        self.ctx = to_dev(self.ctx_np)
        self.kc = nan_pool_dev(case.num_blocks, case.num_kv_heads, case.block_size, case.head_dim, case.dtype)
        self.vc = nan_pool_dev(case.num_blocks, case.num_kv_heads, case.block_size, case.head_dim, case.dtype)
        k, v = to_dev(case.k), to_dev(case.v)
        pg.paged_kv_write(k, v, to_dev(case.cu_ctx), to_dev(case.start_pos), self.table, self.kc, self.vc)
        del k, v

    def extend(self) -> torch.Tensor:
        c = self.case
        return pg.gqa_paged_extend(self.q, self.cu_q, self.kc, self.vc, self.table, self.ctx, c.max_q_len,
                                   int(self.ctx_np.max()) if c.batch else 0, scale=float(c.scale))


def oracle_extend(orc, case: W.ExtendCase, rows=None, context_lens=None, window: int = 0) -> np.ndarray:
    kc = W.nan_pool(case.num_blocks, case.num_kv_heads, case.block_size, case.head_dim, case.dtype)
    vc = W.nan_pool(case.num_blocks, case.num_kv_heads, case.block_size, case.head_dim, case.dtype)
    orc.paged_kv_write(case.k, case.v, case.cu_ctx, case.start_pos, case.block_table, kc, vc)
    ctx = case.context_lens if context_lens is None else np.asarray(context_lens, np.int32)
    return orc.gqa_paged_extend(case.q, case.cu_q, kc, vc, case.block_table, ctx, case.scale, rows=rows,
                                window=window)
