"""Python handle on the library's host-side block manager (pgqa_bm_* in
include/paged_gqa.h): refcounted KV blocks with copy-on-write.  Argument
marshalling only; the bookkeeping runs in block_manager.cpp."""

from __future__ import annotations

import ctypes as C
from typing import List, Optional, Sequence, Tuple

import numpy as np

from ._lib import PgqaError, check, lib


class BlockManager:
    """Block tables for sequences that may share prefix blocks."""

    def __init__(self, num_blocks: int, block_size: int):
        self._h = lib().pgqa_bm_create(int(num_blocks), int(block_size))
        if not self._h:
            raise PgqaError("pgqa_bm_create", 1)
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def close(self) -> None:
        if self._h:
            lib().pgqa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def new_sequence(self) -> int:
        out = C.c_int32()
        check("pgqa_bm_new_sequence", lib().pgqa_bm_new_sequence(self._h, C.byref(out)))
        return out.value

    def fork(self, parent: int) -> int:
        out = C.c_int32()
        check("pgqa_bm_fork", lib().pgqa_bm_fork(self._h, int(parent), C.byref(out)))
        return out.value

    def append(self, seq: int, n: int) -> Optional[Tuple[int, int]]:
        """Room for n more tokens; the (src, dst) block copy to run first, if any."""
        s, d = C.c_int32(), C.c_int32()
        check("pgqa_bm_append", lib().pgqa_bm_append(self._h, int(seq), int(n), C.byref(s), C.byref(d)))
        return None if s.value < 0 else (s.value, d.value)

    def free(self, seq: int) -> None:
        check("pgqa_bm_free_sequence", lib().pgqa_bm_free_sequence(self._h, int(seq)))

    def length(self, seq: int) -> int:
        return int(lib().pgqa_bm_sequence_length(self._h, int(seq)))

    def table(self, seq: int) -> List[int]:
        n = lib().pgqa_bm_block_table(self._h, int(seq), None, 0)
        if n < 0:
            raise PgqaError("pgqa_bm_block_table", 1)
        buf = (C.c_int32 * max(n, 1))()
        lib().pgqa_bm_block_table(self._h, int(seq), buf, n)
        return list(buf[:n])

    def refcount(self, block: int) -> int:
        return int(lib().pgqa_bm_refcount(self._h, int(block)))

    def num_free_blocks(self) -> int:
        return int(lib().pgqa_bm_num_free_blocks(self._h))

    def block_tables(self, seqs: Sequence[int], width: Optional[int] = None) -> np.ndarray:
        """int32 [len(seqs), width] block tables (rows padded with -1) for the device calls."""
        rows = [self.table(s) for s in seqs]
        w = max([len(r) for r in rows] + [1]) if width is None else width
        out = np.full((len(rows), w), -1, dtype=np.int32)
        for i, r in enumerate(rows):
            out[i, :len(r)] = r
        return out
