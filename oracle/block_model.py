"""Plain model of refcounted KV blocks with copy-on-write.

TEST INFRASTRUCTURE ONLY: the reference the native block manager of the HIP
library is compared against, operation by operation.  It shares no code with
that library.

What it follows (the pages, restated):
  - paging: a sequence's KV cache is a list of fixed-size blocks taken from a
    pool, found through its block table; a block is taken only when a new token
    needs one, and a finished request gives its blocks back ("The Ultimate Guide
    to LLM Inference Optimization- Part 2", section "Paged Attention"; "Modern LLM
    Inference", section 8.2, non-contiguous KV blocks);
  - prefix sharing: blocks carry a reference counter, several sequences may point
    at the same blocks, and when sequences diverge only the block being modified
    is copied while the rest stay shared ("Modern LLM Inference", section 8.2,
    "Prefix Sharing (Copy-on-Write)"; the Ultimate Guide, same section: a shared
    prefix is stored once and duplicated only when a request diverges).

Readings where the pages leave a choice open:
  - a block is free exactly when its counter is 0; new blocks (fresh pages and
    copies alike) are the lowest-numbered free ones; a new sequence gets the
    lowest unused id;
  - forking a sequence gives the child the parent's whole table and length,
    adding one reference to each block;
  - appending n tokens writes positions len .. len+n-1.  Only a partly filled
    last block can be modified by that (full blocks are never written again),
    so if that block is shared (counter > 1) it is copied first: a fresh block
    replaces it in this table, the old block loses one reference, and the copy
    (old, new) is reported so that its contents can be copied on the device
    before the new tokens are written.  Pages past the old end get fresh blocks;
  - an append that would need more free blocks than exist fails and changes
    nothing.
"""

from __future__ import annotations

from typing import Dict, List, Optional, Tuple


class OutOfBlocks(RuntimeError):
    pass


class BlockModel:
    def __init__(self, num_blocks: int, block_size: int):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.ref: List[int] = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lengths: Dict[int, int] = {}

    # -- helpers -------------------------------------------------------------
    def free_blocks(self) -> List[int]:
        return [b for b in range(self.num_blocks) if self.ref[b] == 0]

    def _pages(self, length: int) -> int:
        return -(-length // self.block_size)

    # -- operations ------------------------------------------------------------
    def new_sequence(self) -> int:
        sid = 0
        while sid in self.tables:
            sid += 1
        self.tables[sid] = []
        self.lengths[sid] = 0
        return sid

    def fork(self, parent: int) -> int:
        if parent not in self.tables:
            raise KeyError(parent)
        child = self.new_sequence()
        self.tables[child] = list(self.tables[parent])
        self.lengths[child] = self.lengths[parent]
        for b in self.tables[child]:
            self.ref[b] += 1
        return child

    def append(self, seq: int, n: int) -> Optional[Tuple[int, int]]:
        """Make room for n new tokens; returns the (src, dst) block copy, if any."""
        if seq not in self.tables:
            raise KeyError(seq)
        if n < 0:
            raise ValueError("n must be >= 0")
        table, length = self.tables[seq], self.lengths[seq]
        if n == 0:
            return None
        cow = length % self.block_size != 0 and self.ref[table[-1]] > 1
        fresh = self._pages(length + n) - len(table)
        free = self.free_blocks()
        if len(free) < fresh + (1 if cow else 0):
            raise OutOfBlocks(f"need {fresh + cow} blocks, {len(free)} free")
        copy = None
        if cow:
            new = free.pop(0)
            old = table[-1]
            self.ref[old] -= 1
            self.ref[new] = 1
            table[-1] = new
            copy = (old, new)
        for _ in range(fresh):
            b = free.pop(0)
            self.ref[b] = 1
            table.append(b)
        self.lengths[seq] = length + n
        return copy

    def free(self, seq: int) -> None:
        if seq not in self.tables:
            raise KeyError(seq)
        for b in self.tables.pop(seq):
            self.ref[b] -= 1
        del self.lengths[seq]
