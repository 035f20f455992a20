"""Thin torch front end of the C ABI: argument marshalling only.

Every function takes torch tensors on the GPU, checks dtypes / shapes / layout
enough to build the C call, passes ``data_ptr()``s and the current stream's
handle, and raises :class:`PgqaError` on a non-OK status.  All computation runs
in the HIP kernels of libpaged_gqa.so; torch only owns memory and streams.
"""

from __future__ import annotations

import os
from typing import Optional, Tuple

import torch

from ._lib import PGQA_BF16, PGQA_F32, check, lib

# PGQA_DEBUG_CHECKS=1: before each call, check the device arrays' contents
# (block ids, lengths, row offsets) with pgqa_check_contents and raise
# ContractError on a broken promise.  Each check waits for the GPU.
DEBUG_CHECKS = os.environ.get("PGQA_DEBUG_CHECKS", "") not in ("", "0")

_CHECK_FLAGS = {1: "block id outside the pool", 2: "context length or write position out of range",
                4: "bad row offsets", 8: "fewer cached positions than query rows"}
_INT32_MAX = 2 ** 31 - 1


class ContractError(ValueError):
    """A device array breaks a promise the C ABI takes on trust (found by check_contents)."""


def check_contents(batch: int, block_table: Optional[torch.Tensor] = None,
                   context_lens: Optional[torch.Tensor] = None, cu_rows: Optional[torch.Tensor] = None,
                   start_pos: Optional[torch.Tensor] = None, total_rows: int = 0, max_rows: int = -1,
                   num_blocks: int = 0, block_size: int = 1, max_context_len: int = 0, window: int = 0) -> dict:
    """Run pgqa_check_contents on the given device arrays and return its report
    (flags, first bad sequence or None, bad block-table entries, bad sequences)."""
    ts = [t for t in (block_table, context_lens, cu_rows, start_pos) if t is not None]
    _dev(*ts)
    _i32(*ts)
    dev = ts[0].device if ts else torch.device("cuda")
    status = torch.empty(4, dtype=torch.int32, device=dev)
    ptr = lambda t: None if t is None else t.data_ptr()
    st = lib().pgqa_check_contents(ptr(block_table), block_table.shape[1] if block_table is not None else 0,
                                   ptr(context_lens), ptr(cu_rows), ptr(start_pos), int(batch), int(total_rows),
                                   int(max_rows), int(num_blocks), int(block_size), int(max_context_len),
                                   int(window), status.data_ptr(), _stream())
    check("pgqa_check_contents", st)
    f, first, nbad, nseq = status.cpu().tolist()
    return {"flags": f, "first_bad_sequence": None if first == _INT32_MAX else first, "bad_block_ids": nbad,
            "bad_sequences": nseq,
            "problems": [msg for bit, msg in _CHECK_FLAGS.items() if f & bit]}


def _debug(call: str, batch: int, **kw) -> None:
    if not DEBUG_CHECKS:
        return
    r = check_contents(batch, **kw)
    if r["flags"]:
        raise ContractError(f"{call}: {', '.join(r['problems'])} ({r['bad_sequences']} sequence(s), first "
                            f"{r['first_bad_sequence']}; {r['bad_block_ids']} bad block-table entries)")

_DT = {torch.bfloat16: PGQA_BF16, torch.float32: PGQA_F32}


def _dtype(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"expected bfloat16 or float32, got {t.dtype}")
    return _DT[t.dtype]


def _dev(*ts: torch.Tensor) -> None:
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _i32(*ts: torch.Tensor) -> None:
    for t in ts:
        if t.dtype != torch.int32:
            raise TypeError(f"index tensors must be int32, got {t.dtype}")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _same_dtype(what: str, ref: torch.Tensor, *ts: torch.Tensor) -> None:
    for t in ts:
        if t.dtype != ref.dtype:
            raise TypeError(f"{what}: dtype {t.dtype} differs from {ref.dtype}")


def _shape(what: str, t: torch.Tensor, shape) -> None:
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def _rank(what: str, t: torch.Tensor, n: int) -> None:
    if t.dim() != n:
        raise ValueError(f"{what}: expected {n} dimensions, got shape {tuple(t.shape)}")


def _rows(what: str, t: torch.Tensor, n: int) -> None:
    if t.dim() < 1 or t.shape[0] != n:
        raise ValueError(f"{what}: expected {n} rows, got shape {tuple(t.shape)}")


def _table(block_table: torch.Tensor, batch: int) -> None:
    _rank("block_table", block_table, 2)
    _rows("block_table", block_table, batch)


def _pools(k_cache: torch.Tensor, v_cache: torch.Tensor):
    _rank("k_cache", k_cache, 4)
    _shape("v_cache", v_cache, k_cache.shape)
    _same_dtype("v_cache", k_cache, v_cache)
    return k_cache.shape


def _out(out: Optional[torch.Tensor], q: torch.Tensor) -> torch.Tensor:
    if out is None:
        return torch.empty_like(q)
    _shape("out", out, q.shape)
    _same_dtype("out", q, out)
    return out


def paged_kv_write(k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor, start_pos: torch.Tensor,
                   block_table: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor) -> None:
    """Scatter packed k, v [T, Hkv, d] into k_cache, v_cache [num_blocks, Hkv, bs, d] in place."""
    nb, hkv, bs, d = _pools(k_cache, v_cache)
    _rank("k", k, 3)
    _shape("k", k, (k.shape[0], hkv, d))
    _shape("v", v, k.shape)
    _same_dtype("k / v against the cache", k_cache, k, v)
    batch = start_pos.numel()
    _rows("cu_seqlens", cu_seqlens, batch + 1)
    _table(block_table, batch)
    _dev(k, v, cu_seqlens, start_pos, block_table, k_cache, v_cache)
    _i32(cu_seqlens, start_pos, block_table)
    _debug("paged_kv_write", batch, block_table=block_table, cu_rows=cu_seqlens, start_pos=start_pos,
           total_rows=k.shape[0], num_blocks=nb, block_size=bs)
    st = lib().paged_kv_write(k.data_ptr(), v.data_ptr(), cu_seqlens.data_ptr(), start_pos.data_ptr(),
                              block_table.data_ptr(), block_table.shape[1], k_cache.data_ptr(), v_cache.data_ptr(),
                              cu_seqlens.numel() - 1, k.shape[0], nb, bs, hkv, d, _dtype(k), _stream())
    check("paged_kv_write", st)


def paged_kv_gather(k_cache: torch.Tensor, v_cache: torch.Tensor, cu_seqlens: torch.Tensor,
                    start_pos: torch.Tensor, block_table: torch.Tensor, total_tokens: int,
                    k_out: Optional[torch.Tensor] = None,
                    v_out: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Inverse of paged_kv_write: packed [total_tokens, Hkv, d] copies of the cached rows."""
    nb, hkv, bs, d = _pools(k_cache, v_cache)
    batch = start_pos.numel()
    _rows("cu_seqlens", cu_seqlens, batch + 1)
    _table(block_table, batch)
    if k_out is None:
        k_out = torch.empty((total_tokens, hkv, d), dtype=k_cache.dtype, device=k_cache.device)
    if v_out is None:
        v_out = torch.empty((total_tokens, hkv, d), dtype=k_cache.dtype, device=k_cache.device)
    _shape("k_out", k_out, (total_tokens, hkv, d))
    _shape("v_out", v_out, (total_tokens, hkv, d))
    _same_dtype("k_out / v_out against the cache", k_cache, k_out, v_out)
    _dev(k_cache, v_cache, cu_seqlens, start_pos, block_table, k_out, v_out)
    _i32(cu_seqlens, start_pos, block_table)
    _debug("paged_kv_gather", batch, block_table=block_table, cu_rows=cu_seqlens, start_pos=start_pos,
           total_rows=total_tokens, num_blocks=nb, block_size=bs)
    st = lib().paged_kv_gather(k_cache.data_ptr(), v_cache.data_ptr(), cu_seqlens.data_ptr(), start_pos.data_ptr(),
                               block_table.data_ptr(), block_table.shape[1], k_out.data_ptr(), v_out.data_ptr(),
                               cu_seqlens.numel() - 1, total_tokens, nb, bs, hkv, d, _dtype(k_cache), _stream())
    check("paged_kv_gather", st)
    return k_out, v_out


def gqa_paged_decode_workspace_size(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                                    num_splits: int = 0) -> int:
    return int(lib().gqa_paged_decode_workspace_size(batch, num_q_heads, num_kv_heads, head_dim, num_splits))


def decode_workspace(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int, num_splits: int = 0,
                     device=None) -> torch.Tensor:
    """Device workspace for gqa_paged_decode (contents need no initialisation)."""
    n = gqa_paged_decode_workspace_size(batch, num_q_heads, num_kv_heads, head_dim, num_splits)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device or "cuda")


def gqa_paged_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                     context_lens: torch.Tensor, max_context_len: int, scale: float,
                     out: Optional[torch.Tensor] = None, num_splits: int = 0,
                     workspace: Optional[torch.Tensor] = None, window: int = 0) -> torch.Tensor:
    """Decode attention: q [B, Hq, d] over paged K/V -> out [B, Hq, d] (window > 0: the newest
    `window` positions only).  scale is the softmax scale (normally 1/sqrt(d))."""
    _rank("q", q, 3)
    B, hq, d = q.shape
    nb, hkv, bs, d2 = _pools(k_cache, v_cache)
    if d2 != d:
        raise ValueError("head_dim mismatch")
    _same_dtype("k_cache / v_cache against q", q, k_cache)
    _table(block_table, B)
    _shape("context_lens", context_lens, (B,))
    out = _out(out, q)
    if workspace is None:
        workspace = decode_workspace(B, hq, hkv, d, num_splits, q.device)
    _dev(q, k_cache, v_cache, block_table, context_lens, out, workspace)
    _i32(block_table, context_lens)
    _debug("gqa_paged_decode", B, block_table=block_table, context_lens=context_lens, num_blocks=nb, block_size=bs,
           max_context_len=int(max_context_len), window=int(window))
    st = lib().gqa_paged_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(),
                                block_table.shape[1], context_lens.data_ptr(), B, hq, hkv, d, bs, nb,
                                int(max_context_len), float(scale), int(window), _dtype(q), out.data_ptr(),
                                int(num_splits),
                                workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream())
    check("gqa_paged_decode", st)
    return out


def gqa_paged_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                             block_table: torch.Tensor, context_lens: torch.Tensor, max_context_len: int,
                             scale: float, out: torch.Tensor, num_splits: int = 0, window: int = 0) -> torch.Tensor:
    """gqa_paged_decode without a workspace (the library's own per-GPU scratch holds the
    split partials; calls that may overlap on one GPU race).  out is required: nothing
    is allocated (so PGQA_DEBUG_CHECKS, whose check needs a status buffer, skips it)."""
    _rank("q", q, 3)
    B, hq, d = q.shape
    nb, hkv, bs, d2 = _pools(k_cache, v_cache)
    if d2 != d:
        raise ValueError("head_dim mismatch")
    _same_dtype("k_cache / v_cache against q", q, k_cache)
    _table(block_table, B)
    _shape("context_lens", context_lens, (B,))
    out = _out(out, q)
    _dev(q, k_cache, v_cache, block_table, context_lens, out)
    _i32(block_table, context_lens)
    st = lib().gqa_paged_decode_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(),
                                        block_table.shape[1], context_lens.data_ptr(), B, hq, hkv, d, bs, nb,
                                        int(max_context_len), float(scale), int(window), _dtype(q), out.data_ptr(),
                                        int(num_splits), _stream())
    check("gqa_paged_decode_noalloc", st)
    return out


def gqa_varlen_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
                       max_seqlen: int, scale: float, causal: bool = True,
                       out: Optional[torch.Tensor] = None, window: int = 0) -> torch.Tensor:
    """Packed varlen prefill: q [T, Hq, d], k / v [T, Hkv, d] -> out [T, Hq, d]."""
    _rank("q", q, 3)
    _rank("k", k, 3)
    T, hq, d = q.shape
    hkv = k.shape[1]
    _shape("k", k, (T, hkv, d))
    _shape("v", v, k.shape)
    _same_dtype("k / v against q", q, k, v)
    _rank("cu_seqlens", cu_seqlens, 1)
    out = _out(out, q)
    _dev(q, k, v, cu_seqlens, out)
    _i32(cu_seqlens)
    _debug("gqa_varlen_prefill", cu_seqlens.numel() - 1, cu_rows=cu_seqlens, total_rows=T, max_rows=int(max_seqlen))
    st = lib().gqa_varlen_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), cu_seqlens.data_ptr(),
                                  cu_seqlens.numel() - 1, T, int(max_seqlen), hq, hkv, d, float(scale),
                                  int(bool(causal)), int(window), _dtype(q), out.data_ptr(), _stream())
    check("gqa_varlen_prefill", st)
    return out


def gqa_paged_extend_workspace_size(batch: int, total_q: int, max_q_len: int, num_q_heads: int,
                                    num_kv_heads: int, head_dim: int, max_context_len: int) -> int:
    return int(lib().gqa_paged_extend_workspace_size(batch, total_q, max_q_len, num_q_heads, num_kv_heads, head_dim,
                                                     max_context_len))


def extend_workspace(batch: int, total_q: int, max_q_len: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                     max_context_len: int, device=None) -> torch.Tensor:
    """Device workspace for gqa_paged_extend's key split (contents need no initialisation)."""
    n = gqa_paged_extend_workspace_size(batch, total_q, max_q_len, num_q_heads, num_kv_heads, head_dim,
                                        max_context_len)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device or "cuda")


def gqa_paged_extend(q: torch.Tensor, cu_q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                     block_table: torch.Tensor, context_lens: torch.Tensor, max_q_len: int, max_context_len: int,
                     scale: float, out: Optional[torch.Tensor] = None,
                     window: int = 0, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Several new tokens per sequence over its paged cache (chunked prefill on a cached
    prefix, draft verification): q [total_q, Hq, d] -> out [total_q, Hq, d].  The new
    tokens' K/V must already be in the pages; context_lens counts them."""
    _rank("q", q, 3)
    T, hq, d = q.shape
    nb, hkv, bs, d2 = _pools(k_cache, v_cache)
    if d2 != d:
        raise ValueError("head_dim mismatch")
    _same_dtype("k_cache / v_cache against q", q, k_cache)
    _rank("cu_q", cu_q, 1)
    batch = cu_q.numel() - 1
    _table(block_table, batch)
    _shape("context_lens", context_lens, (batch,))
    out = _out(out, q)
    if workspace is None:
        workspace = extend_workspace(cu_q.numel() - 1, T, int(max_q_len), hq, hkv, d, int(max_context_len), q.device)
    _dev(q, cu_q, k_cache, v_cache, block_table, context_lens, out, workspace)
    _i32(cu_q, block_table, context_lens)
    _debug("gqa_paged_extend", batch, block_table=block_table, context_lens=context_lens, cu_rows=cu_q,
           total_rows=T, max_rows=int(max_q_len), num_blocks=nb, block_size=bs, max_context_len=int(max_context_len),
           window=int(window))
    st = lib().gqa_paged_extend(q.data_ptr(), cu_q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                block_table.data_ptr(), block_table.shape[1], context_lens.data_ptr(),
                                cu_q.numel() - 1, T, int(max_q_len), hq, hkv, d, bs, nb, int(max_context_len),
                                float(scale), int(window), _dtype(q), out.data_ptr(), workspace.data_ptr(),
                                workspace.numel() * workspace.element_size(), _stream())
    check("gqa_paged_extend", st)
    return out


def paged_kv_copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor, src_blocks: torch.Tensor,
                         dst_blocks: torch.Tensor) -> None:
    """Copy whole blocks src_blocks[p] -> dst_blocks[p] (all heads, K and V) in place."""
    nb, hkv, bs, d = _pools(k_cache, v_cache)
    if src_blocks.numel() != dst_blocks.numel():
        raise ValueError("src_blocks and dst_blocks differ in length")
    _dev(k_cache, v_cache, src_blocks, dst_blocks)
    _i32(src_blocks, dst_blocks)
    st = lib().paged_kv_copy_blocks(k_cache.data_ptr(), v_cache.data_ptr(), src_blocks.data_ptr(),
                                    dst_blocks.data_ptr(), src_blocks.numel(), nb, bs, hkv, d, _dtype(k_cache),
                                    _stream())
    check("paged_kv_copy_blocks", st)


def fp8_pools(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int, device=None):
    """Empty FP8 page pools: (k_codes, v_codes) uint8 [nb, Hkv, bs, d], (k_scale, v_scale) fp32 [nb, Hkv, bs]."""
    shape = (num_blocks, num_kv_heads, block_size, head_dim)
    dev = device or "cuda"
    return (torch.empty(shape, dtype=torch.uint8, device=dev), torch.empty(shape, dtype=torch.uint8, device=dev),
            torch.empty(shape[:3], dtype=torch.float32, device=dev),
            torch.empty(shape[:3], dtype=torch.float32, device=dev))


def _u8(*ts: torch.Tensor) -> None:
    for t in ts:
        if t.dtype != torch.uint8:
            raise TypeError(f"FP8 code pools are uint8, got {t.dtype}")


def _f32(*ts: torch.Tensor) -> None:
    for t in ts:
        if t.dtype != torch.float32:
            raise TypeError(f"scale pools are float32, got {t.dtype}")


def paged_kv_write_fp8(k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor, start_pos: torch.Tensor,
                       block_table: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                       k_scale: torch.Tensor, v_scale: torch.Tensor) -> None:
    """Quantise packed bf16 k, v [T, Hkv, d] into FP8 code pools and fp32 row-scale pools in place."""
    _u8(k_cache, v_cache)
    _f32(k_scale, v_scale)
    nb, hkv, bs, d = _pools(k_cache, v_cache)
    _shape("k_scale", k_scale, (nb, hkv, bs))
    _shape("v_scale", v_scale, (nb, hkv, bs))
    _rank("k", k, 3)
    _shape("k", k, (k.shape[0], hkv, d))
    _shape("v", v, k.shape)
    if k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise TypeError("rows quantised into FP8 pages are bfloat16")
    batch = start_pos.numel()
    _rows("cu_seqlens", cu_seqlens, batch + 1)
    _table(block_table, batch)
    _dev(k, v, cu_seqlens, start_pos, block_table, k_cache, v_cache, k_scale, v_scale)
    _i32(cu_seqlens, start_pos, block_table)
    _debug("paged_kv_write_fp8", batch, block_table=block_table, cu_rows=cu_seqlens, start_pos=start_pos,
           total_rows=k.shape[0], num_blocks=nb, block_size=bs)
    st = lib().paged_kv_write_fp8(k.data_ptr(), v.data_ptr(), cu_seqlens.data_ptr(), start_pos.data_ptr(),
                                  block_table.data_ptr(), block_table.shape[1], k_cache.data_ptr(), v_cache.data_ptr(),
                                  k_scale.data_ptr(), v_scale.data_ptr(), cu_seqlens.numel() - 1, k.shape[0], nb, bs,
                                  hkv, d, _dtype(k), _stream())
    check("paged_kv_write_fp8", st)


def gqa_paged_decode_fp8(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, k_scale: torch.Tensor,
                         v_scale: torch.Tensor, block_table: torch.Tensor, context_lens: torch.Tensor,
                         max_context_len: int, scale: float, out: Optional[torch.Tensor] = None,
                         num_splits: int = 0, workspace: Optional[torch.Tensor] = None,
                         window: int = 0) -> torch.Tensor:
    """Decode attention over FP8 pages: bf16 q [B, Hq, d] -> bf16 out [B, Hq, d]."""
    _rank("q", q, 3)
    B, hq, d = q.shape
    _u8(k_cache, v_cache)
    _f32(k_scale, v_scale)
    nb, hkv, bs, d2 = _pools(k_cache, v_cache)
    if d2 != d:
        raise ValueError("head_dim mismatch")
    if q.dtype != torch.bfloat16:
        raise TypeError("queries over FP8 pages are bfloat16")
    _shape("k_scale", k_scale, (nb, hkv, bs))
    _shape("v_scale", v_scale, (nb, hkv, bs))
    _table(block_table, B)
    _shape("context_lens", context_lens, (B,))
    out = _out(out, q)
    if workspace is None:
        workspace = decode_workspace(B, hq, hkv, d, num_splits, q.device)
    _dev(q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens, out, workspace)
    _i32(block_table, context_lens)
    _debug("gqa_paged_decode_fp8", B, block_table=block_table, context_lens=context_lens, num_blocks=nb,
           block_size=bs, max_context_len=int(max_context_len), window=int(window))
    st = lib().gqa_paged_decode_fp8(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), k_scale.data_ptr(),
                                    v_scale.data_ptr(), block_table.data_ptr(), block_table.shape[1],
                                    context_lens.data_ptr(), B, hq, hkv, d, bs, nb, int(max_context_len),
                                    float(scale), int(window), out.data_ptr(), int(num_splits), workspace.data_ptr(),
                                    workspace.numel() * workspace.element_size(), _stream())
    check("gqa_paged_decode_fp8", st)
    return out


def gqa_paged_extend_fp8(q: torch.Tensor, cu_q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                         k_scale: torch.Tensor, v_scale: torch.Tensor, block_table: torch.Tensor,
                         context_lens: torch.Tensor, max_q_len: int, max_context_len: int, scale: float,
                         out: Optional[torch.Tensor] = None, window: int = 0,
                         workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """gqa_paged_extend over FP8 pages: bf16 q [total_q, Hq, d] -> bf16 out [total_q, Hq, d]."""
    _rank("q", q, 3)
    T, hq, d = q.shape
    _u8(k_cache, v_cache)
    _f32(k_scale, v_scale)
    nb, hkv, bs, d2 = _pools(k_cache, v_cache)
    if d2 != d:
        raise ValueError("head_dim mismatch")
    if q.dtype != torch.bfloat16:
        raise TypeError("queries over FP8 pages are bfloat16")
    _shape("k_scale", k_scale, (nb, hkv, bs))
    _shape("v_scale", v_scale, (nb, hkv, bs))
    _rank("cu_q", cu_q, 1)
    batch = cu_q.numel() - 1
    _table(block_table, batch)
    _shape("context_lens", context_lens, (batch,))
    out = _out(out, q)
    if workspace is None:
        workspace = extend_workspace(batch, T, int(max_q_len), hq, hkv, d, int(max_context_len), q.device)
    _dev(q, cu_q, k_cache, v_cache, k_scale, v_scale, block_table, context_lens, out, workspace)
    _i32(cu_q, block_table, context_lens)
    _debug("gqa_paged_extend_fp8", batch, block_table=block_table, context_lens=context_lens, cu_rows=cu_q,
           total_rows=T, max_rows=int(max_q_len), num_blocks=nb, block_size=bs, max_context_len=int(max_context_len),
           window=int(window))
    st = lib().gqa_paged_extend_fp8(q.data_ptr(), cu_q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                    k_scale.data_ptr(), v_scale.data_ptr(), block_table.data_ptr(),
                                    block_table.shape[1], context_lens.data_ptr(), batch, T, int(max_q_len), hq,
                                    hkv, d, bs, nb, int(max_context_len), float(scale), int(window), out.data_ptr(),
                                    workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream())
    check("gqa_paged_extend_fp8", st)
    return out
