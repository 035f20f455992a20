"""ctypes front end of the fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg use it; the product package never imports it.  This wrapper
only marshals numpy arrays; every step of the computation is in oracle.c.
"""

from __future__ import annotations

import ctypes as C
from pathlib import Path
from typing import Optional

import numpy as np

from .build import LIB, build

F32, BF16, F64 = 0, 1, 2
OK, EINVAL, ERANGE = 0, 1, 2

_P = C.c_void_p
_I = C.c_int32
_D = C.c_double


class OracleError(RuntimeError):
    pass


def _bind(lib: C.CDLL) -> C.CDLL:
    lib.oracle_paged_kv_write.argtypes = [_P, _P, _P, _P, _P, _I, _P, _P, _I, _I, _I, _I, _I, _I]
    lib.oracle_paged_kv_gather.argtypes = [_P, _P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _I]
    lib.oracle_gqa_paged_decode.argtypes = [_P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I, _D, _I, _I,
                                            _P, _P, _I, _I]
    lib.oracle_gqa_varlen_prefill.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _D, _I, _I, _I, _P, _I, _P, _I]
    lib.oracle_gqa_paged_extend.argtypes = [_P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I, _D, _I, _I,
                                            _P, _I, _P, _I]
    lib.oracle_paged_kv_copy_blocks.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I]
    lib.oracle_fp8_e4m3_decode.argtypes = [_P, C.c_int64, _P]
    lib.oracle_fp8_e4m3_encode.argtypes = [_P, C.c_int64, _P]
    lib.oracle_paged_kv_write_fp8.argtypes = [_P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I]
    lib.oracle_dequantize_fp8.argtypes = [_P, _P, C.c_int64, _I, _P]
    for f in ("oracle_paged_kv_write", "oracle_paged_kv_gather", "oracle_paged_kv_copy_blocks", "oracle_gqa_paged_decode",
              "oracle_fp8_e4m3_decode", "oracle_fp8_e4m3_encode", "oracle_paged_kv_write_fp8", "oracle_dequantize_fp8",
              "oracle_gqa_varlen_prefill", "oracle_gqa_paged_extend", "oracle_max_threads"):
        getattr(lib, f).restype = C.c_int
    return lib


class Oracle:
    """One loaded copy of the oracle library (a path lets tests load variants)."""

    def __init__(self, path: Optional[Path] = None):
        path = Path(path) if path is not None else LIB
        if path == LIB and not LIB.exists():
            build()
        self.path = path
        self.lib = _bind(C.CDLL(str(path)))

    # -- helpers -------------------------------------------------------------
    @staticmethod
    def _dtype(arr: np.ndarray) -> int:
        if arr.dtype == np.float64:
            return F64
        if arr.dtype == np.uint16:
            return BF16
        if arr.dtype == np.float32:
            return F32
        raise TypeError(f"oracle inputs are float32 or uint16 bf16 bits, got {arr.dtype}")

    @staticmethod
    def _c(arr: np.ndarray, dtype=None) -> np.ndarray:
        return np.ascontiguousarray(arr, dtype=dtype)

    @staticmethod
    def _ptr(arr: Optional[np.ndarray]):
        return None if arr is None else arr.ctypes.data_as(C.c_void_p)

    def _check(self, rc: int, what: str):
        if rc != OK:
            raise OracleError(f"{what} returned {rc}")

    def max_threads(self) -> int:
        return int(self.lib.oracle_max_threads())

    # -- the calls -----------------------------------------------------------
    def paged_kv_write(self, k, v, cu_seqlens, start_pos, block_table, k_cache, v_cache):
        """Scatter packed K/V into the page pools in place (pools are modified)."""
        k, v = self._c(k), self._c(v)
        dt = self._dtype(k)
        assert v.dtype == k.dtype and k_cache.dtype == k.dtype and v_cache.dtype == k.dtype
        assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
        cu = self._c(cu_seqlens, np.int32)
        sp = self._c(start_pos, np.int32)
        bt = self._c(block_table, np.int32)
        nb, hkv, bs, d = k_cache.shape
        rc = self.lib.oracle_paged_kv_write(self._ptr(k), self._ptr(v), self._ptr(cu), self._ptr(sp),
                                            self._ptr(bt), bt.shape[1], self._ptr(k_cache),
                                            self._ptr(v_cache), len(cu) - 1, nb, bs, hkv, d, dt)
        self._check(rc, "oracle_paged_kv_write")

    # -- low-precision pages (FP8 E4M3 codes + one fp32 scale per (token, KV head) row) --
    def fp8_decode(self, codes):
        c = self._c(codes, np.uint8)
        out = np.empty(c.shape, dtype=np.float64)
        self._check(self.lib.oracle_fp8_e4m3_decode(self._ptr(c), c.size, self._ptr(out)), "oracle_fp8_e4m3_decode")
        return out

    def fp8_encode(self, x):
        x = self._c(x, np.float32)
        out = np.empty(x.shape, dtype=np.uint8)
        self._check(self.lib.oracle_fp8_e4m3_encode(self._ptr(x), x.size, self._ptr(out)), "oracle_fp8_e4m3_encode")
        return out

    def paged_kv_write_fp8(self, k, v, cu_seqlens, start_pos, block_table, k_cache, v_cache, k_scale, v_scale):
        """Quantising paged write in place: uint8 code pools [nb, Hkv, bs, d], fp32 scale pools [nb, Hkv, bs]."""
        k, v = self._c(k), self._c(v)
        dt = self._dtype(k)
        for a in (k_cache, v_cache, k_scale, v_scale):
            assert a.flags.c_contiguous
        assert k_cache.dtype == np.uint8 and k_scale.dtype == np.float32
        cu, sp = self._c(cu_seqlens, np.int32), self._c(start_pos, np.int32)
        bt = self._c(block_table, np.int32)
        nb, hkv, bs, d = k_cache.shape
        rc = self.lib.oracle_paged_kv_write_fp8(self._ptr(k), self._ptr(v), self._ptr(cu), self._ptr(sp),
                                                self._ptr(bt), bt.shape[1], self._ptr(k_cache), self._ptr(v_cache),
                                                self._ptr(k_scale), self._ptr(v_scale), len(cu) - 1, nb, bs, hkv, d,
                                                dt)
        self._check(rc, "oracle_paged_kv_write_fp8")

    def dequantize_fp8(self, codes, scales):
        """fp64 values of a code pool [..., d] with its scale pool [...]."""
        c, s = self._c(codes, np.uint8), self._c(scales, np.float32)
        assert c.shape[:-1] == s.shape
        out = np.empty(c.shape, dtype=np.float64)
        rc = self.lib.oracle_dequantize_fp8(self._ptr(c), self._ptr(s), s.size, c.shape[-1], self._ptr(out))
        self._check(rc, "oracle_dequantize_fp8")
        return out

    def paged_kv_copy_blocks(self, k_cache, v_cache, src, dst):
        """Copy blocks src[i] -> dst[i] (all KV heads, K and V) in place, in order."""
        assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous and k_cache.dtype == v_cache.dtype
        dt = self._dtype(k_cache)
        s, d_ = self._c(src, np.int32), self._c(dst, np.int32)
        assert s.shape == d_.shape
        nb, hkv, bs, d = k_cache.shape
        rc = self.lib.oracle_paged_kv_copy_blocks(self._ptr(k_cache), self._ptr(v_cache), self._ptr(s),
                                                  self._ptr(d_), len(s), nb, bs, hkv, d, dt)
        self._check(rc, "oracle_paged_kv_copy_blocks")

    def paged_kv_gather(self, k_cache, v_cache, block_table, context_lens):
        nb, hkv, bs, d = k_cache.shape
        dt = self._dtype(k_cache)
        bt = self._c(block_table, np.int32)
        cl = self._c(context_lens, np.int32)
        T = int(cl.astype(np.int64).sum())
        k_out = np.zeros((T, hkv, d), dtype=k_cache.dtype)
        v_out = np.zeros((T, hkv, d), dtype=k_cache.dtype)
        rc = self.lib.oracle_paged_kv_gather(self._ptr(self._c(k_cache)), self._ptr(self._c(v_cache)),
                                             self._ptr(bt), bt.shape[1], self._ptr(cl), self._ptr(k_out),
                                             self._ptr(v_out), len(cl), nb, bs, hkv, d, dt)
        self._check(rc, "oracle_paged_kv_gather")
        return k_out, v_out

    def gqa_paged_decode(self, q, k_cache, v_cache, block_table, context_lens, scale,
                         want_probs: bool = False, num_threads: int = 0, window: int = 0):
        """fp64 output [B, Hq, d] (and, if asked, probs [B, Hq, max_ctx]); window > 0 keeps the
        newest `window` positions only."""
        q = self._c(q)
        dt = self._dtype(q)
        B, hq, d = q.shape
        nb, hkv, bs, d2 = k_cache.shape
        assert d2 == d
        bt = self._c(block_table, np.int32)
        cl = self._c(context_lens, np.int32)
        out = np.empty((B, hq, d), dtype=np.float64)
        stride = int(cl.max()) if (want_probs and B) else 0
        probs = np.zeros((B, hq, max(stride, 1)), dtype=np.float64) if want_probs else None
        rc = self.lib.oracle_gqa_paged_decode(self._ptr(q), self._ptr(self._c(k_cache)),
                                              self._ptr(self._c(v_cache)), self._ptr(bt), bt.shape[1],
                                              self._ptr(cl), B, hq, hkv, d, bs, nb, float(scale), int(window),
                                              dt, self._ptr(out), self._ptr(probs), max(stride, 1),
                                              int(num_threads))
        self._check(rc, "oracle_gqa_paged_decode")
        return (out, probs) if want_probs else out

    def gqa_varlen_prefill(self, q, k, v, cu_seqlens, scale, causal=True, rows=None, num_threads: int = 0,
                           window: int = 0):
        """fp64 output [T or len(rows), Hq, d]."""
        q, k, v = self._c(q), self._c(k), self._c(v)
        dt = self._dtype(q)
        T, hq, d = q.shape
        hkv = k.shape[1]
        cu = self._c(cu_seqlens, np.int32)
        r = None if rows is None else self._c(rows, np.int32)
        n = T if r is None else len(r)
        out = np.empty((n, hq, d), dtype=np.float64)
        rc = self.lib.oracle_gqa_varlen_prefill(self._ptr(q), self._ptr(k), self._ptr(v), self._ptr(cu),
                                                len(cu) - 1, hq, hkv, d, float(scale), int(bool(causal)),
                                                int(window), dt, self._ptr(r), n, self._ptr(out), int(num_threads))
        self._check(rc, "oracle_gqa_varlen_prefill")
        return out


    def gqa_paged_extend(self, q, cu_q, k_cache, v_cache, block_table, context_lens, scale, rows=None,
                         num_threads: int = 0, window: int = 0):
        """fp64 output [total_q or len(rows), Hq, d]: each query row over its sequence's cached keys up to
        its position."""
        q = self._c(q)
        dt = self._dtype(q)
        Tq, hq, d = q.shape
        nb, hkv, bs, d2 = k_cache.shape
        assert d2 == d
        cq = self._c(cu_q, np.int32)
        bt = self._c(block_table, np.int32)
        cl = self._c(context_lens, np.int32)
        r = None if rows is None else self._c(rows, np.int32)
        n = Tq if r is None else len(r)
        out = np.empty((n, hq, d), dtype=np.float64)
        rc = self.lib.oracle_gqa_paged_extend(self._ptr(q), self._ptr(cq), self._ptr(self._c(k_cache)),
                                              self._ptr(self._c(v_cache)), self._ptr(bt), bt.shape[1],
                                              self._ptr(cl), len(cl), hq, hkv, d, bs, nb, float(scale),
                                              int(window), dt, self._ptr(r), n, self._ptr(out), int(num_threads))
        self._check(rc, "oracle_gqa_paged_extend")
        return out


_default: Optional[Oracle] = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
