"""Seeded synthetic inputs for paged grouped-query attention.

This module draws the inputs that both the HIP path and the CPU oracle consume:
sequence lengths, Q/K/V values, and the placement of KV pages in a shuffled
physical pool.  It holds none of the attention arithmetic.

Recipe (the same for every workload):

* ``numpy.random.default_rng(seed)`` (PCG64); draws happen in a fixed order:
  (1) lengths, (2) Q, (3) K, (4) V, (5) ``permutation(pool)``.
* Values are ``standard_normal`` in float32.  For bf16 workloads they are
  rounded once to bf16 (round to nearest, ties to even, on the fp32 bit
  pattern) and handed to both sides as raw ``uint16`` bit patterns, so the
  GPU and the oracle read identical bits.
* K and V are packed token-major, sequence-major: ``[sum(len), Hkv, d]``,
  the packed layout of "Modern LLM Inference" (gozhiyuan.github.io),
  section 8.1, selective batching: sequences are concatenated with no padding.
* The physical pool holds ``ceil(1.25 * sum(ceil(len / bs)))`` blocks.
  A permutation of the pool is drawn and its first ``needed`` entries are
  assigned sequence-major, page-minor to the block table, which maps each
  sequence's logical pages to physical blocks ("Advanced Optimizations: MQA,
  GQA, and PagedAttention", section "PagedAttention: The OS Analogy").
  Table entries past a sequence's last page hold -1.
* Pool slots that are never written hold a NaN sentinel, so any read of an
  unused slot shows up in the output.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

F32 = "f32"
BF16 = "bf16"

#: Quiet-NaN bit patterns used to fill never-written pool slots.
NAN_BITS = {BF16: np.uint16(0x7FC0), F32: np.uint32(0x7FC00000)}


def elem_bytes(dtype: str) -> int:
    return 2 if dtype == BF16 else 4


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits.

    Inputs here are finite normal draws, so no NaN/Inf special-casing is needed;
    a NaN input is rejected rather than silently mangled.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.isfinite(x).all():
        raise ValueError("bf16 input rounding expects finite values")
    u = x.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (for reporting only)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _values(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == BF16:
        return f32_to_bf16_bits(x)
    return x


def nan_pool(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int, dtype: str) -> np.ndarray:
    """A KV page pool ``[num_blocks, Hkv, bs, d]`` filled with the NaN sentinel."""
    shape = (num_blocks, num_kv_heads, block_size, head_dim)
    if dtype == BF16:
        return np.full(shape, NAN_BITS[BF16], dtype=np.uint16)
    return np.full(shape, NAN_BITS[F32], dtype=np.uint32).view(np.float32)


def pages_needed(lengths: Sequence[int], block_size: int) -> np.ndarray:
    return np.array([-(-int(n) // block_size) for n in lengths], dtype=np.int64)


def place_pages(rng: np.random.Generator, lengths: Sequence[int], block_size: int,
                pool_blocks: Optional[int] = None, pool_factor: float = 1.25,
                extra_cols: int = 0):
    """Draw the physical placement of every logical page.

    Returns ``(block_table int32 [B, max_pages + extra_cols], num_blocks)``.
    """
    need = pages_needed(lengths, block_size)
    total = int(need.sum())
    if pool_blocks is None:
        pool_blocks = max(1, int(math.ceil(pool_factor * total)))
    if pool_blocks < total:
        raise ValueError("pool smaller than the pages needed")
    perm = rng.permutation(pool_blocks)
    width = int(need.max()) if len(need) else 0
    width = max(width + extra_cols, 1)
    table = np.full((len(lengths), width), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[off:off + n]
        off += int(n)
    return table, int(pool_blocks)


def cu_from_lengths(lengths: Sequence[int]) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


@dataclass
class DecodeCase:
    """One decode batch: one query token per sequence over paged K/V."""
    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    context_lens: np.ndarray      # int32 [B]
    cu_ctx: np.ndarray            # int32 [B+1], prefix sums of context_lens
    q: np.ndarray                 # [B, Hq, d]      (uint16 bf16 bits or float32)
    k: np.ndarray                 # [sum ctx, Hkv, d] packed
    v: np.ndarray                 # [sum ctx, Hkv, d] packed
    block_table: np.ndarray       # int32 [B, max_blocks_per_seq]
    num_blocks: int
    scale: np.float32
    seed: int = 0

    @property
    def batch(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.batch else 0

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def start_pos(self) -> np.ndarray:
        return np.zeros(self.batch, dtype=np.int32)

    def kv_bytes(self) -> int:
        """Bytes of K and V that attention must read (valid tokens only)."""
        return int(self.context_lens.astype(np.int64).sum()) * self.num_kv_heads * self.head_dim * 2 * elem_bytes(self.dtype)

    def flops(self) -> int:
        return int(self.context_lens.astype(np.int64).sum()) * self.num_q_heads * 4 * self.head_dim


@dataclass
class PrefillCase:
    """One packed variable-length prefill batch (block-diagonal causal)."""
    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    lengths: np.ndarray           # int32 [B]
    cu_seqlens: np.ndarray        # int32 [B+1]
    q: np.ndarray                 # [T, Hq, d]
    k: np.ndarray                 # [T, Hkv, d]
    v: np.ndarray                 # [T, Hkv, d]
    block_table: np.ndarray       # int32 [B, max_blocks_per_seq] for the paged copy of K/V
    num_blocks: int
    scale: np.float32
    causal: bool = True
    seed: int = 0

    @property
    def batch(self) -> int:
        return int(self.lengths.shape[0])

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def max_seqlen(self) -> int:
        return int(self.lengths.max()) if self.batch else 0

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    def flops(self) -> int:
        """Algorithmic FLOPs: QK^T and PV over the causal (or full) key range."""
        L = self.lengths.astype(np.int64)
        pairs = (L * (L + 1) // 2).sum() if self.causal else (L * L).sum()
        return int(pairs) * self.num_q_heads * 4 * self.head_dim


def make_decode_case(lengths: Sequence[int], num_q_heads: int, num_kv_heads: int, head_dim: int,
                     block_size: int, dtype: str = BF16, seed: int = 0, *, name: str = "custom",
                     rng: Optional[np.random.Generator] = None, pool_blocks: Optional[int] = None,
                     pool_factor: float = 1.25, extra_cols: int = 0,
                     scale: Optional[float] = None) -> DecodeCase:
    """Decode inputs for given context lengths; draws Q, K, V, then the placement."""
    if rng is None:
        rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, dtype=np.int32)
    B = int(lengths.shape[0])
    T = int(lengths.astype(np.int64).sum())
    q = _values(rng, (B, num_q_heads, head_dim), dtype)
    k = _values(rng, (T, num_kv_heads, head_dim), dtype)
    v = _values(rng, (T, num_kv_heads, head_dim), dtype)
    table, nblk = place_pages(rng, lengths, block_size, pool_blocks=pool_blocks,
                              pool_factor=pool_factor, extra_cols=extra_cols)
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return DecodeCase(name=name, dtype=dtype, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                      head_dim=head_dim, block_size=block_size, context_lens=lengths,
                      cu_ctx=cu_from_lengths(lengths), q=q, k=k, v=v, block_table=table,
                      num_blocks=nblk, scale=np.float32(scale), seed=seed)


def make_prefill_case(lengths: Sequence[int], num_q_heads: int, num_kv_heads: int, head_dim: int,
                      block_size: int = 16, dtype: str = BF16, seed: int = 0, *, name: str = "custom",
                      rng: Optional[np.random.Generator] = None, causal: bool = True,
                      pool_factor: float = 1.25, scale: Optional[float] = None) -> PrefillCase:
    """Packed prefill inputs for given sequence lengths; draws Q, K, V, then the placement."""
    if rng is None:
        rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, dtype=np.int32)
    T = int(lengths.astype(np.int64).sum())
    q = _values(rng, (T, num_q_heads, head_dim), dtype)
    k = _values(rng, (T, num_kv_heads, head_dim), dtype)
    v = _values(rng, (T, num_kv_heads, head_dim), dtype)
    table, nblk = place_pages(rng, lengths, block_size, pool_factor=pool_factor)
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return PrefillCase(name=name, dtype=dtype, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                       head_dim=head_dim, block_size=block_size, lengths=lengths,
                       cu_seqlens=cu_from_lengths(lengths), q=q, k=k, v=v, block_table=table,
                       num_blocks=nblk, scale=np.float32(scale), causal=causal, seed=seed)


@dataclass
class ExtendCase:
    """Several query tokens per sequence over its paged cache (chunked prefill on
    a cached prefix, or draft-token verification): sequence b's q_lens[b] query
    tokens are the last positions of its context_lens[b] cached tokens."""
    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    context_lens: np.ndarray      # int32 [B] (prefix + new tokens)
    q_lens: np.ndarray            # int32 [B]
    cu_ctx: np.ndarray            # int32 [B+1]
    cu_q: np.ndarray              # int32 [B+1]
    q: np.ndarray                 # [sum q_lens, Hq, d]
    k: np.ndarray                 # [sum ctx, Hkv, d] packed
    v: np.ndarray                 # [sum ctx, Hkv, d] packed
    block_table: np.ndarray       # int32 [B, max_blocks_per_seq]
    num_blocks: int
    scale: np.float32
    seed: int = 0

    @property
    def batch(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.cu_q[-1])

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if self.batch else 0

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.batch else 0

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def start_pos(self) -> np.ndarray:
        return np.zeros(self.batch, dtype=np.int32)

    def kv_bytes(self) -> int:
        """Bytes of K and V that must be read (every cached token once)."""
        return int(self.context_lens.astype(np.int64).sum()) * self.num_kv_heads * self.head_dim * 2 * elem_bytes(self.dtype)

    def flops(self) -> int:
        """Algorithmic FLOPs: query i of a sequence attends to prefix + i + 1 keys."""
        n = self.q_lens.astype(np.int64)
        pre = self.context_lens.astype(np.int64) - n
        pairs = (n * pre + n * (n + 1) // 2).sum()
        return int(pairs) * self.num_q_heads * 4 * self.head_dim


def make_extend_case(prefix_lens: Sequence[int], q_lens: Sequence[int], num_q_heads: int, num_kv_heads: int,
                     head_dim: int, block_size: int = 16, dtype: str = BF16, seed: int = 0, *,
                     name: str = "custom", rng: Optional[np.random.Generator] = None,
                     pool_factor: float = 1.25, scale: Optional[float] = None) -> ExtendCase:
    """Multi-token-query inputs; draws Q, K, V, then the placement (like decode)."""
    if rng is None:
        rng = np.random.default_rng(seed)
    prefix = np.asarray(prefix_lens, dtype=np.int32)
    qn = np.asarray(q_lens, dtype=np.int32)
    ctx = (prefix + qn).astype(np.int32)
    T = int(ctx.astype(np.int64).sum())
    Tq = int(qn.astype(np.int64).sum())
    q = _values(rng, (Tq, num_q_heads, head_dim), dtype)
    k = _values(rng, (T, num_kv_heads, head_dim), dtype)
    v = _values(rng, (T, num_kv_heads, head_dim), dtype)
    table, nblk = place_pages(rng, ctx, block_size, pool_factor=pool_factor)
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return ExtendCase(name=name, dtype=dtype, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                      head_dim=head_dim, block_size=block_size, context_lens=ctx, q_lens=qn,
                      cu_ctx=cu_from_lengths(ctx), cu_q=cu_from_lengths(qn), q=q, k=k, v=v,
                      block_table=table, num_blocks=nblk, scale=np.float32(scale), seed=seed)


@dataclass
class SharedPrefixCase:
    """Several samples decoding from one prompt (prefix sharing): every sample's
    context is the prompt followed by its own continuation.  Values only; how the
    pages are shared is decided by the code under test."""
    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    prompt_len: int
    cont_lens: np.ndarray         # int32 [B] tokens each sample added after the fork (>= 1)
    q: np.ndarray                 # [B, Hq, d] one decode query per sample
    k_prompt: np.ndarray          # [prompt_len, Hkv, d]
    v_prompt: np.ndarray
    k_cont: np.ndarray            # [sum cont_lens, Hkv, d], samples concatenated
    v_cont: np.ndarray
    scale: np.float32
    seed: int = 0

    @property
    def batch(self) -> int:
        return int(self.cont_lens.shape[0])

    @property
    def context_lens(self) -> np.ndarray:
        return (self.prompt_len + self.cont_lens).astype(np.int32)

    @property
    def cu_cont(self) -> np.ndarray:
        return cu_from_lengths(self.cont_lens)

    def _row_bytes(self) -> int:
        return self.num_kv_heads * self.head_dim * 2 * elem_bytes(self.dtype)

    def logical_kv_bytes(self) -> int:
        """K/V bytes the samples attend over, each sample's copy of the prompt counted."""
        return int(self.context_lens.astype(np.int64).sum()) * self._row_bytes()

    def unique_kv_bytes(self) -> int:
        """K/V bytes of distinct positions: the prompt once plus every continuation."""
        return (self.prompt_len + int(self.cont_lens.astype(np.int64).sum())) * self._row_bytes()

    def logical(self, rng: np.random.Generator) -> DecodeCase:
        """The same samples as unshared sequences (packed K/V, a placement of their own)."""
        parts_k, parts_v = [], []
        cu = self.cu_cont
        for b in range(self.batch):
            parts_k += [self.k_prompt, self.k_cont[cu[b]:cu[b + 1]]]
            parts_v += [self.v_prompt, self.v_cont[cu[b]:cu[b + 1]]]
        ctx = self.context_lens
        table, nb = place_pages(rng, ctx, self.block_size)
        return DecodeCase(name=self.name + "_unshared", dtype=self.dtype, num_q_heads=self.num_q_heads,
                          num_kv_heads=self.num_kv_heads, head_dim=self.head_dim, block_size=self.block_size,
                          context_lens=ctx, cu_ctx=cu_from_lengths(ctx), q=self.q, k=np.concatenate(parts_k),
                          v=np.concatenate(parts_v), block_table=table, num_blocks=nb, scale=self.scale,
                          seed=self.seed)


def make_shared_prefix_case(prompt_len: int, cont_lens: Sequence[int], num_q_heads: int, num_kv_heads: int,
                            head_dim: int, block_size: int = 16, dtype: str = BF16, seed: int = 0, *,
                            name: str = "custom", rng: Optional[np.random.Generator] = None,
                            scale: Optional[float] = None) -> SharedPrefixCase:
    """Draw order after the lengths: Q, prompt K, prompt V, continuation K, continuation V."""
    if rng is None:
        rng = np.random.default_rng(seed)
    cont = np.asarray(cont_lens, dtype=np.int32)
    B, Tc = int(cont.shape[0]), int(cont.astype(np.int64).sum())
    q = _values(rng, (B, num_q_heads, head_dim), dtype)
    kp = _values(rng, (prompt_len, num_kv_heads, head_dim), dtype)
    vp = _values(rng, (prompt_len, num_kv_heads, head_dim), dtype)
    kc = _values(rng, (Tc, num_kv_heads, head_dim), dtype)
    vc = _values(rng, (Tc, num_kv_heads, head_dim), dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return SharedPrefixCase(name=name, dtype=dtype, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                            head_dim=head_dim, block_size=block_size, prompt_len=int(prompt_len), cont_lens=cont,
                            q=q, k_prompt=kp, v_prompt=vp, k_cont=kc, v_cont=vc, scale=np.float32(scale), seed=seed)


# ---------------------------------------------------------------------------
# The named workloads.
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    key: str
    kind: str            # "decode" or "prefill"
    seed: int
    description: str
    summary: dict = field(default_factory=dict)


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", "decode", 1,
                         "tiny paged GQA decode, fp32: ctx [5, 11], Hq=4, Hkv=2, d=16, bs=4, 8-block pool",
                         {"batch": 2, "num_q_heads": 4, "num_kv_heads": 2, "head_dim": 16, "block_size": 4, "dtype": F32}),
    "llama3_8b_decode": Workload("llama3_8b_decode", "decode", 2,
                                 "Llama-3-8B-shaped GQA decode: B=64, ctx~U[512,4096], Hq=32, Hkv=8, d=128, bs=16, bf16",
                                 {"batch": 64, "num_q_heads": 32, "num_kv_heads": 8, "head_dim": 128, "block_size": 16, "dtype": BF16}),
    "long_ctx_decode": Workload("long_ctx_decode", "decode", 3,
                                "long-context split-KV decode: B=8, ctx=32768, Hq=64, Hkv=8, d=128, bs=16, bf16",
                                {"batch": 8, "num_q_heads": 64, "num_kv_heads": 8, "head_dim": 128, "block_size": 16, "dtype": BF16}),
    "mqa_decode": Workload("mqa_decode", "decode", 4,
                           "MQA decode: B=256, ctx~lognormal(median 1000, sigma 0.8) in [16,8192], Hq=32, Hkv=1, d=128, bs=32, bf16",
                           {"batch": 256, "num_q_heads": 32, "num_kv_heads": 1, "head_dim": 128, "block_size": 32, "dtype": BF16}),
    "varlen_prefill": Workload("varlen_prefill", "prefill", 5,
                               "packed varlen causal prefill: 32 seqs, L~U[64,1024], Hq=32, Hkv=8, d=128, bf16, paged copy bs=16",
                               {"batch": 32, "num_q_heads": 32, "num_kv_heads": 8, "head_dim": 128, "block_size": 16, "dtype": BF16}),
    "chunked_prefill": Workload("chunked_prefill", "extend", 6,
                                "chunked prefill over a paged prefix: 16 seqs, cached prefix~U[0,3072], 512 new tokens each, "
                                "Hq=32, Hkv=8, d=128, bs=16, bf16",
                                {"batch": 16, "num_q_heads": 32, "num_kv_heads": 8, "head_dim": 128, "block_size": 16,
                                 "dtype": BF16, "q_len": 512}),
    "shared_prefix_decode": Workload("shared_prefix_decode", "shared", 8,
                                     "64 samples decoding from one 8003-token prompt (shared pages), each with its "
                                     "own continuation ~U[64,2048]; Hq=32, Hkv=8, d=128, bs=16, bf16",
                                     {"batch": 64, "num_q_heads": 32, "num_kv_heads": 8, "head_dim": 128,
                                      "block_size": 16, "dtype": BF16, "prompt_len": 8003}),
    "spec_verify": Workload("spec_verify", "extend", 7,
                            "draft-token verification: B=64, ctx~U[512,4096] incl. 4 draft tokens each, "
                            "Hq=32, Hkv=8, d=128, bs=16, bf16",
                            {"batch": 64, "num_q_heads": 32, "num_kv_heads": 8, "head_dim": 128, "block_size": 16,
                             "dtype": BF16, "q_len": 4}),
}

WORKLOAD_ORDER: List[str] = ["tiny_f32", "llama3_8b_decode", "long_ctx_decode", "mqa_decode", "varlen_prefill",
                             "chunked_prefill", "spec_verify", "shared_prefix_decode"]


def workload_lengths(key: str, rng: np.random.Generator) -> np.ndarray:
    """Step (1) of the draw order: the sequence / context lengths."""
    if key == "tiny_f32":
        return np.array([5, 11], dtype=np.int32)
    if key == "llama3_8b_decode":
        return rng.integers(512, 4096, size=64, endpoint=True).astype(np.int32)
    if key == "long_ctx_decode":
        return np.full(8, 32768, dtype=np.int32)
    if key == "mqa_decode":
        z = rng.standard_normal(256)
        n = np.rint(np.exp(math.log(1000.0) + 0.8 * z))
        return np.clip(n, 16, 8192).astype(np.int32)
    if key == "varlen_prefill":
        return rng.integers(64, 1024, size=32, endpoint=True).astype(np.int32)
    if key == "chunked_prefill":   # cached prefix lengths
        return rng.integers(0, 3072, size=16, endpoint=True).astype(np.int32)
    if key == "spec_verify":       # cached prefix lengths (the context less the 4 draft tokens)
        return (rng.integers(512, 4096, size=64, endpoint=True) - 4).astype(np.int32)
    if key == "shared_prefix_decode":   # continuation lengths after the shared prompt
        return rng.integers(64, 2048, size=64, endpoint=True).astype(np.int32)
    raise KeyError(key)


def make_workload(key: str):
    """Build the named workload's inputs (a DecodeCase, PrefillCase, ExtendCase or SharedPrefixCase)."""
    w = WORKLOADS[key]
    s = w.summary
    rng = np.random.default_rng(w.seed)
    lengths = workload_lengths(key, rng)
    if w.kind == "decode":
        pool = 8 if key == "tiny_f32" else None
        return make_decode_case(lengths, s["num_q_heads"], s["num_kv_heads"], s["head_dim"],
                                s["block_size"], s["dtype"], w.seed, name=key, rng=rng,
                                pool_blocks=pool)
    if w.kind == "shared":
        return make_shared_prefix_case(s["prompt_len"], lengths, s["num_q_heads"], s["num_kv_heads"],
                                       s["head_dim"], s["block_size"], s["dtype"], w.seed, name=key, rng=rng)
    if w.kind == "extend":
        q_lens = np.full(len(lengths), s["q_len"], dtype=np.int32)
        return make_extend_case(lengths, q_lens, s["num_q_heads"], s["num_kv_heads"], s["head_dim"],
                                s["block_size"], s["dtype"], w.seed, name=key, rng=rng)
    return make_prefill_case(lengths, s["num_q_heads"], s["num_kv_heads"], s["head_dim"],
                             s["block_size"], s["dtype"], w.seed, name=key, rng=rng)
