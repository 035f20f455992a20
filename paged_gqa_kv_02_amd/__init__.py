"""Grouped-query attention over a paged KV cache for AMD Instinct MI355X (gfx950).

The product is the C-ABI library libpaged_gqa.so (include/paged_gqa.h) built
from the HIP sources in csrc/; this package is its thin torch front end.
"""

from ._lib import PgqaError, LIB_PATH
from .blocks import BlockManager
from .ops import (ContractError, check_contents, decode_workspace, extend_workspace, fp8_pools, gqa_paged_decode, gqa_paged_decode_fp8,
                  gqa_paged_decode_noalloc, gqa_paged_extend_fp8,
                  gqa_paged_decode_workspace_size, gqa_paged_extend, gqa_paged_extend_workspace_size,
                  gqa_varlen_prefill, paged_kv_copy_blocks, paged_kv_gather, paged_kv_write, paged_kv_write_fp8)

__all__ = ["PgqaError", "LIB_PATH", "paged_kv_write", "paged_kv_gather", "gqa_paged_decode",
           "gqa_paged_decode_workspace_size", "decode_workspace", "gqa_varlen_prefill", "gqa_paged_extend",
           "paged_kv_copy_blocks", "BlockManager", "fp8_pools", "paged_kv_write_fp8", "gqa_paged_decode_fp8",
           "gqa_paged_extend_workspace_size", "extend_workspace", "gqa_paged_decode_noalloc",
           "gqa_paged_extend_fp8", "check_contents", "ContractError"]
