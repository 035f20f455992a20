"""The C ABI on the CPU: the library loads, exports what the header declares, and
rejects bad arguments on the host before any HIP call (no GPU needed)."""

import ctypes as C
import subprocess

import pytest

from paged_gqa_kv_02_amd import _lib as L

EINVAL, ENOTSUP, ENOSPC = 1, 2, 3
F32, BF16 = 0, 1

# Fake, 16-byte-aligned, non-null "device pointers": validation never dereferences them.
P = [0x10000 * (i + 1) for i in range(12)]


@pytest.fixture(scope="module")
def lib(built_lib):
    return L.load(built_lib)


def test_header_declares_the_calls():
    names = L.header_functions()
    for n in ("paged_kv_write", "paged_kv_gather", "gqa_paged_decode", "gqa_paged_decode_workspace_size",
              "gqa_varlen_prefill", "gqa_paged_extend", "paged_kv_copy_blocks", "pgqa_bm_create", "pgqa_bm_append",
              "gqa_paged_decode_noalloc", "gqa_paged_extend_fp8", "pgqa_check_contents", "gqa_paged_decode_fp8", "paged_kv_write_fp8",
              "pgqa_bm_fork", "pgqa_bm_free_sequence", "pgqa_status_string"):
        assert n in names


def test_every_declared_symbol_is_exported(built_lib):
    out = subprocess.run(["nm", "-D", "--defined-only", str(built_lib)], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for n in L.header_functions():
        assert n in exported, f"{n} declared in paged_gqa.h but not exported"


def test_status_strings(lib):
    for s in range(5):
        assert lib.pgqa_status_string(s)
    assert b"unknown" in lib.pgqa_status_string(99)


def _write(lib, **kw):
    a = dict(k=P[0], v=P[1], cu=P[2], sp=P[3], bt=P[4], maxb=4, kc=P[5], vc=P[6], batch=2, T=10, nb=8, bs=16,
             hkv=2, d=128, dt=BF16)
    a.update(kw)
    return lib.paged_kv_write(a["k"], a["v"], a["cu"], a["sp"], a["bt"], a["maxb"], a["kc"], a["vc"], a["batch"],
                              a["T"], a["nb"], a["bs"], a["hkv"], a["d"], a["dt"], None)


def test_write_validation(lib):
    assert _write(lib, k=None) == EINVAL
    assert _write(lib, k=P[0] + 4) == EINVAL          # misaligned element pointer
    assert _write(lib, cu=P[2] + 2) == EINVAL         # misaligned index pointer
    assert _write(lib, batch=-1) == EINVAL
    assert _write(lib, nb=0) == EINVAL
    assert _write(lib, d=96) == ENOTSUP
    assert _write(lib, bs=24) == ENOTSUP
    assert _write(lib, bs=512) == ENOTSUP
    assert _write(lib, dt=7) == ENOTSUP
    assert _write(lib, batch=0) == 0                  # nothing to do: OK without touching HIP
    assert _write(lib, T=0) == 0


def _decode(lib, **kw):
    a = dict(q=P[0], kc=P[1], vc=P[2], bt=P[3], maxb=4, cl=P[4], batch=2, hq=8, hkv=2, d=128, bs=16, nb=8,
             maxctx=64, scale=0.125, win=0, dt=BF16, out=P[5], splits=0, ws=P[6], wsb=1 << 30)
    a.update(kw)
    return lib.gqa_paged_decode(a["q"], a["kc"], a["vc"], a["bt"], a["maxb"], a["cl"], a["batch"], a["hq"],
                                a["hkv"], a["d"], a["bs"], a["nb"], a["maxctx"], a["scale"], a["win"], a["dt"],
                                a["out"], a["splits"], a["ws"], a["wsb"], None)


def test_decode_validation(lib):
    assert _decode(lib, hq=6, hkv=4) == EINVAL         # Hq % Hkv != 0
    assert _decode(lib, maxctx=65) == EINVAL           # beyond max_blocks_per_seq * block_size
    assert _decode(lib, maxctx=-1) == EINVAL
    assert _decode(lib, out=None) == EINVAL
    assert _decode(lib, q=P[0] + 8) == EINVAL
    assert _decode(lib, splits=-1) == EINVAL
    assert _decode(lib, scale=float("nan")) == EINVAL
    assert _decode(lib, win=-1) == EINVAL
    assert _decode(lib, d=80) == ENOTSUP
    assert _decode(lib, hq=24, hkv=2) == ENOTSUP       # group 12 not built
    assert _decode(lib, hq=256, hkv=2) == ENOTSUP      # group 128 not built
    assert _decode(lib, bs=3) == ENOTSUP
    assert _decode(lib, dt=5) == ENOTSUP
    assert _decode(lib, batch=9000) == ENOTSUP
    need = lib.gqa_paged_decode_workspace_size(2, 8, 2, 128, 0)
    assert need > 0
    assert _decode(lib, wsb=need - 1) == ENOSPC
    assert _decode(lib, ws=None, wsb=0) == ENOSPC
    assert _decode(lib, batch=0) == 0


def _decode_noalloc(lib, **kw):
    a = dict(q=P[0], kc=P[1], vc=P[2], bt=P[3], maxb=4, cl=P[4], batch=2, hq=8, hkv=2, d=128, bs=16, nb=8,
             maxctx=64, scale=0.125, win=0, dt=BF16, out=P[5], splits=0)
    a.update(kw)
    return lib.gqa_paged_decode_noalloc(a["q"], a["kc"], a["vc"], a["bt"], a["maxb"], a["cl"], a["batch"], a["hq"],
                                        a["hkv"], a["d"], a["bs"], a["nb"], a["maxctx"], a["scale"], a["win"],
                                        a["dt"], a["out"], a["splits"], None)


def test_decode_noalloc_validation(lib):
    """The allocation-free decode checks its arguments like gqa_paged_decode, and refuses
    sizes whose partials would not fit its 128 MiB scratch, before any HIP call."""
    assert _decode_noalloc(lib, hq=6, hkv=4) == EINVAL
    assert _decode_noalloc(lib, out=None) == EINVAL
    assert _decode_noalloc(lib, scale=float("inf")) == EINVAL
    assert _decode_noalloc(lib, d=80) == ENOTSUP
    assert _decode_noalloc(lib, batch=9000) == ENOTSUP
    assert _decode_noalloc(lib, batch=0) == 0
    limit = 128 << 20
    # 8,000 sequences x 8 KV heads, G = 4, d = 128: (4096 + 64000) x 4 x 130 x 4 bytes > 128 MiB
    assert lib.gqa_paged_decode_workspace_size(8000, 32, 8, 128, 0) > limit
    assert _decode_noalloc(lib, batch=8000, hq=32, hkv=8, maxb=1, maxctx=16) == ENOSPC
    assert lib.gqa_paged_decode_workspace_size(7500, 32, 8, 128, 0) <= limit
    assert _decode_noalloc(lib, splits=200000, hq=32, hkv=8) == ENOSPC


def test_workspace_size_formula(lib):
    # (splits + B * Hkv) pieces x G heads x (d + 2) floats, then B + 1 int32 tile prefix sums
    assert lib.gqa_paged_decode_workspace_size(64, 32, 8, 128, 100) == (100 + 512) * 4 * 130 * 4 + 65 * 4
    assert lib.gqa_paged_decode_workspace_size(8, 64, 8, 128, 0) == (4096 + 64) * 8 * 130 * 4 + 9 * 4
    assert lib.gqa_paged_decode_workspace_size(2, 6, 4, 128, 0) == 0
    assert lib.gqa_paged_decode_workspace_size(-1, 8, 2, 128, 0) == 0


def _prefill(lib, **kw):
    a = dict(q=P[0], k=P[1], v=P[2], cu=P[3], batch=3, T=17, maxs=9, hq=32, hkv=8, d=128, scale=0.088,
             causal=1, win=0, dt=BF16, out=P[4])
    a.update(kw)
    return lib.gqa_varlen_prefill(a["q"], a["k"], a["v"], a["cu"], a["batch"], a["T"], a["maxs"], a["hq"],
                                  a["hkv"], a["d"], a["scale"], a["causal"], a["win"], a["dt"], a["out"], None)


def test_prefill_validation(lib):
    assert _prefill(lib, hq=30) == EINVAL
    assert _prefill(lib, T=-1) == EINVAL
    assert _prefill(lib, cu=None) == EINVAL
    assert _prefill(lib, out=P[4] + 2) == EINVAL
    assert _prefill(lib, win=-3) == EINVAL
    assert _prefill(lib, causal=0, win=8) == EINVAL     # a window needs the causal mask
    assert _prefill(lib, dt=F32) == ENOTSUP             # bf16 MFMA path only
    assert _prefill(lib, d=32) == ENOTSUP
    assert _prefill(lib, hq=24, hkv=8) == ENOTSUP       # group 3
    assert _prefill(lib, batch=0) == 0
    assert _prefill(lib, T=0) == 0


def _extend(lib, **kw):
    a = dict(q=P[0], cu=P[1], kc=P[2], vc=P[3], bt=P[4], maxb=4, cl=P[5], batch=2, T=12, maxq=9, hq=32, hkv=8,
             d=128, bs=16, nb=8, maxctx=64, scale=0.088, win=0, dt=BF16, out=P[6], ws=None, wsb=0)
    a.update(kw)
    return lib.gqa_paged_extend(a["q"], a["cu"], a["kc"], a["vc"], a["bt"], a["maxb"], a["cl"], a["batch"],
                                a["T"], a["maxq"], a["hq"], a["hkv"], a["d"], a["bs"], a["nb"], a["maxctx"],
                                a["scale"], a["win"], a["dt"], a["out"], a["ws"], a["wsb"], None)


def test_extend_validation(lib):
    assert _extend(lib, hq=30) == EINVAL                # Hq % Hkv != 0
    assert _extend(lib, T=-1) == EINVAL
    assert _extend(lib, maxq=-1) == EINVAL
    assert _extend(lib, maxctx=65) == EINVAL            # beyond max_blocks_per_seq * block_size
    assert _extend(lib, nb=0) == EINVAL
    assert _extend(lib, cu=None) == EINVAL
    assert _extend(lib, cl=P[5] + 2) == EINVAL
    assert _extend(lib, out=P[6] + 2) == EINVAL
    assert _extend(lib, scale=float("inf")) == EINVAL
    assert _extend(lib, win=-1) == EINVAL
    assert _extend(lib, ws=P[7] + 8, wsb=1024) == EINVAL    # misaligned workspace
    assert _extend(lib, dt=F32) == ENOTSUP              # bf16 MFMA path only
    assert _extend(lib, d=32) == ENOTSUP
    assert _extend(lib, hq=24, hkv=8) == ENOTSUP        # group 3
    assert _extend(lib, bs=2, maxctx=8) == ENOTSUP      # a 4-row load would cross pages
    assert _extend(lib, d=64, bs=4, maxctx=16) == ENOTSUP
    assert _extend(lib, bs=12) == ENOTSUP
    assert _extend(lib, batch=0) == 0
    assert _extend(lib, T=0) == 0
    assert _extend(lib, maxq=0) == 0


def _copy(lib, **kw):
    a = dict(kc=P[0], vc=P[1], src=P[2], dst=P[3], n=3, nb=8, bs=16, hkv=2, d=128, dt=BF16)
    a.update(kw)
    return lib.paged_kv_copy_blocks(a["kc"], a["vc"], a["src"], a["dst"], a["n"], a["nb"], a["bs"], a["hkv"],
                                    a["d"], a["dt"], None)


def test_copy_blocks_validation(lib):
    assert _copy(lib, n=-1) == EINVAL
    assert _copy(lib, nb=0) == EINVAL
    assert _copy(lib, kc=None) == EINVAL
    assert _copy(lib, vc=P[1] + 8) == EINVAL
    assert _copy(lib, src=None) == EINVAL
    assert _copy(lib, dst=P[3] + 1) == EINVAL
    assert _copy(lib, d=48) == ENOTSUP
    assert _copy(lib, bs=24) == ENOTSUP
    assert _copy(lib, dt=9) == ENOTSUP
    assert _copy(lib, n=0) == 0


def _decode8(lib, **kw):
    a = dict(q=P[0], kc=P[1], vc=P[2], ks=P[7], vs=P[8], bt=P[3], maxb=4, cl=P[4], batch=2, hq=8, hkv=2, d=128,
             bs=16, nb=8, maxctx=64, scale=0.125, win=0, out=P[5], splits=0, ws=P[6], wsb=1 << 30)
    a.update(kw)
    return lib.gqa_paged_decode_fp8(a["q"], a["kc"], a["vc"], a["ks"], a["vs"], a["bt"], a["maxb"], a["cl"],
                                    a["batch"], a["hq"], a["hkv"], a["d"], a["bs"], a["nb"], a["maxctx"], a["scale"],
                                    a["win"], a["out"], a["splits"], a["ws"], a["wsb"], None)


def test_fp8_decode_validation(lib):
    assert _decode8(lib, hq=6, hkv=4) == EINVAL
    assert _decode8(lib, ks=None) == EINVAL
    assert _decode8(lib, vs=P[8] + 2) == EINVAL
    assert _decode8(lib, maxctx=65) == EINVAL
    assert _decode8(lib, win=-1) == EINVAL
    assert _decode8(lib, d=32) == ENOTSUP              # FP8 pages: head_dim 64 or 128
    assert _decode8(lib, bs=8, maxctx=32) == ENOTSUP   # FP8 pages: block_size >= 16
    assert _decode8(lib, hq=24, hkv=2) == ENOTSUP
    assert _decode8(lib, wsb=16) == ENOSPC
    assert _decode8(lib, batch=0) == 0


def test_fp8_write_validation(lib):
    def w(**kw):
        a = dict(k=P[0], v=P[1], cu=P[2], sp=P[3], bt=P[4], maxb=4, kc=P[5], vc=P[6], ks=P[7], vs=P[8], batch=2,
                 T=10, nb=8, bs=16, hkv=2, d=128, dt=BF16)
        a.update(kw)
        return lib.paged_kv_write_fp8(a["k"], a["v"], a["cu"], a["sp"], a["bt"], a["maxb"], a["kc"], a["vc"],
                                      a["ks"], a["vs"], a["batch"], a["T"], a["nb"], a["bs"], a["hkv"], a["d"],
                                      a["dt"], None)
    assert w(ks=None) == EINVAL
    assert w(k=P[0] + 4) == EINVAL
    assert w(dt=F32) == ENOTSUP
    assert w(d=96) == ENOTSUP
    assert w(batch=0) == 0


def _extend8(lib, **kw):
    a = dict(q=P[0], cu=P[1], kc=P[2], vc=P[3], ks=P[7], vs=P[8], bt=P[4], maxb=4, cl=P[5], batch=2, T=12, maxq=9,
             hq=32, hkv=8, d=128, bs=16, nb=8, maxctx=64, scale=0.088, win=0, out=P[6], ws=None, wsb=0)
    a.update(kw)
    return lib.gqa_paged_extend_fp8(a["q"], a["cu"], a["kc"], a["vc"], a["ks"], a["vs"], a["bt"], a["maxb"], a["cl"],
                                    a["batch"], a["T"], a["maxq"], a["hq"], a["hkv"], a["d"], a["bs"], a["nb"],
                                    a["maxctx"], a["scale"], a["win"], a["out"], a["ws"], a["wsb"], None)


def test_fp8_extend_validation(lib):
    assert _extend8(lib, ks=None) == EINVAL
    assert _extend8(lib, vs=None) == EINVAL
    assert _extend8(lib, ks=P[7] + 2) == EINVAL
    assert _extend8(lib, hq=30) == EINVAL
    assert _extend8(lib, maxctx=65) == EINVAL
    assert _extend8(lib, cu=None) == EINVAL
    assert _extend8(lib, out=P[6] + 2) == EINVAL
    assert _extend8(lib, win=-1) == EINVAL
    assert _extend8(lib, scale=float("nan")) == EINVAL
    # Scale pools of 4 GiB or more (32-bit offsets in the kernel).
    assert _extend8(lib, nb=1 << 19, bs=256, hkv=8, hq=32, maxb=1 << 10, maxctx=64) == EINVAL
    assert _extend8(lib, d=32) == ENOTSUP
    assert _extend8(lib, hq=24, hkv=8) == ENOTSUP
    assert _extend8(lib, bs=4, maxctx=16) == ENOTSUP         # one 1 KB load of 128-byte code rows spans 8 rows
    assert _extend8(lib, d=64, bs=8, maxctx=32) == ENOTSUP   # 16 rows of 64-byte codes
    assert _extend8(lib, batch=0) == 0
    assert _extend8(lib, T=0) == 0


def test_extend_workspace_size(lib):
    def shares(nw, d):   # per share: its cut record, two partial slots of 32 rows (output, then m and l)
        return nw * 16 + 2 * nw * 32 * (d + 2) * 4
    # Packed rows (q_len x group <= 32): room for the stream-K partials of one share per
    # workgroup slot (two per CU; without a GPU the library assumes 256 CUs), whatever
    # the context lengths ...
    assert lib.gqa_paged_extend_workspace_size(8, 32, 4, 64, 8, 128, 32768) == shares(512, 128)
    assert lib.gqa_paged_extend_workspace_size(64, 256, 4, 32, 8, 128, 200) == shares(512, 128)
    # ... but no more shares than the call has work units: 2 pairs x (1 block + 3)
    assert lib.gqa_paged_extend_workspace_size(2, 2, 1, 8, 1, 64, 10) == shares(8, 64)
    # 8 sequences x 8 KV heads of 40 query tokens (not packed): far fewer pieces than the
    # GPU has slots, so the long contexts are split into key chunks
    n = lib.gqa_paged_extend_workspace_size(8, 320, 40, 64, 8, 128, 32768)
    assert n > 0 and n % (320 * 64 * 130 * 4) == 0
    # 16 sequences x 512 query tokens fill the GPU without a split
    assert lib.gqa_paged_extend_workspace_size(16, 8192, 512, 32, 8, 128, 3584) == 0
    assert lib.gqa_paged_extend_workspace_size(2, 8, 4, 30, 8, 128, 4096) == 0     # Hq % Hkv != 0


def test_build_entry_point(monkeypatch, built_lib):
    """__graft_entry__.build() runs end to end: the HIP build step is replaced by
    the library already built (hipcc takes minutes), the oracle is really
    compiled, and the package imports and loads the library."""
    import __graft_entry__ as entry
    from paged_gqa_kv_02_amd import build as hip_build
    monkeypatch.setattr(hip_build, "build", lambda jobs=0: hip_build.LIB)
    entry.build()


def test_check_contents_validation(lib):
    def c(**kw):
        a = dict(bt=P[0], maxb=4, cl=P[1], cu=None, sp=None, batch=2, T=0, maxr=-1, nb=8, bs=16, maxctx=64, win=0,
                 st=P[2])
        a.update(kw)
        return lib.pgqa_check_contents(a["bt"], a["maxb"], a["cl"], a["cu"], a["sp"], a["batch"], a["T"], a["maxr"],
                                       a["nb"], a["bs"], a["maxctx"], a["win"], a["st"], None)
    assert c(st=None) == EINVAL
    assert c(st=P[2] + 2) == EINVAL
    assert c(batch=-1) == EINVAL
    assert c(win=-1) == EINVAL
    assert c(sp=P[3]) == EINVAL            # a write check needs the row offsets
    assert c(nb=0) == EINVAL
    assert c(maxb=0) == EINVAL
    assert c(cl=P[1] + 1) == EINVAL
    assert c(bs=12) == ENOTSUP
    assert c(bs=512) == ENOTSUP
