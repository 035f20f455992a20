"""ctypes loader for libpaged_gqa.so (the C ABI declared in include/paged_gqa.h).

There is no fallback: if the library is missing or fails to load, importing the
ops raises, so nothing can silently run a slower or different code path.
"""

from __future__ import annotations

import ctypes as C
import re
from pathlib import Path

PKG = Path(__file__).resolve().parent
LIB_PATH = PKG / "libpaged_gqa.so"
HEADER = PKG.parent / "include" / "paged_gqa.h"

PGQA_F32, PGQA_BF16 = 0, 1
STATUS = {0: "PGQA_OK", 1: "PGQA_EINVAL", 2: "PGQA_ENOTSUP", 3: "PGQA_ENOSPC", 4: "PGQA_EHIP"}

_P, _I, _F, _Z = C.c_void_p, C.c_int32, C.c_float, C.c_size_t

_SIGNATURES = {
    "paged_kv_write": (C.c_int, [_P, _P, _P, _P, _P, _I, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P]),
    "paged_kv_gather": (C.c_int, [_P, _P, _P, _P, _P, _I, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P]),
    "gqa_paged_decode_workspace_size": (_Z, [_I, _I, _I, _I, _I]),
    "gqa_paged_decode": (C.c_int, [_P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P, _I,
                                   _P, _Z, _P]),
    "gqa_paged_decode_noalloc": (C.c_int, [_P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P, _I,
                                           _P]),
    "gqa_varlen_prefill": (C.c_int, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I, _P, _P]),
    "gqa_paged_extend": (C.c_int, [_P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _F, _I,
                                   _I, _P, _P, _Z, _P]),
    "gqa_paged_extend_workspace_size": (_Z, [_I, _I, _I, _I, _I, _I, _I]),
    "paged_kv_copy_blocks": (C.c_int, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "paged_kv_write_fp8": (C.c_int, [_P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P]),
    "gqa_paged_decode_fp8": (C.c_int, [_P, _P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _I,
                                       _P, _Z, _P]),
    "gqa_paged_extend_fp8": (C.c_int, [_P, _P, _P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I, _I, _I,
                                       _I, _F, _I, _P, _P, _Z, _P]),
    "pgqa_check_contents": (C.c_int, [_P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P]),
    "pgqa_bm_create": (_P, [_I, _I]),
    "pgqa_bm_destroy": (None, [_P]),
    "pgqa_bm_new_sequence": (C.c_int, [_P, C.POINTER(_I)]),
    "pgqa_bm_fork": (C.c_int, [_P, _I, C.POINTER(_I)]),
    "pgqa_bm_append": (C.c_int, [_P, _I, _I, C.POINTER(_I), C.POINTER(_I)]),
    "pgqa_bm_free_sequence": (C.c_int, [_P, _I]),
    "pgqa_bm_sequence_length": (_I, [_P, _I]),
    "pgqa_bm_block_table": (_I, [_P, _I, _P, _I]),
    "pgqa_bm_refcount": (_I, [_P, _I]),
    "pgqa_bm_num_free_blocks": (_I, [_P]),
    "pgqa_status_string": (C.c_char_p, [C.c_int]),
}


class PgqaError(RuntimeError):
    def __init__(self, call: str, status: int):
        self.status = status
        super().__init__(f"{call} returned {STATUS.get(status, status)}")


def header_functions() -> list:
    """Names of the functions include/paged_gqa.h declares."""
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(?:int|int32_t|void|size_t|const char\*|pgqa_block_manager\*)\s+(\w+)\s*\(",
                                 text)))


def load(path: Path = LIB_PATH) -> C.CDLL:
    if not Path(path).exists():
        raise ImportError(f"{path} is not built; run `python -m paged_gqa_kv_02_amd.build`")
    lib = C.CDLL(str(path))
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = None


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        _lib = load()
    return _lib


def check(call: str, status: int) -> None:
    if status != 0:
        raise PgqaError(call, status)
