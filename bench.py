#!/usr/bin/env python3
"""Benchmark of the paged GQA hot path on one MI355X.

Headline: decode KV-read GB/s on the Llama-3-8B-shaped decode workload (B = 64,
context lengths U[512, 4096], Hq = 32, Hkv = 8, d = 128, block_size 16, bf16).
One step = the decode step of the hot path on that batch:
  1. paged_kv_write of each sequence's newest token (position ctx-1) into its page,
  2. gqa_paged_decode over every cached position (split-KV + merge kernels).
``value`` = algorithmic K/V bytes read per step / wall time per step, the three
kernels launched one by one (``--graph`` replays each step as a captured HIP
graph instead).  ``roofline`` times the decode call alone (split + merge) with
HIP events on its stream, in a second pass.

Before any timing (the headline's W warm-up steps included) each item first runs
untimed calls for at least ``--settle-ms`` milliseconds (default 100): after the
CPU-side set-up of an item the GPU has idled and needs tens of milliseconds of
sustained work to reach its working clocks.  The timed regions are unchanged.

Inputs stay resident in HBM.  Every decode-type item rotates over several copies
of its page pools (4 for the decode batches, 4 for the long-context pools), so
the 256 MB Infinity Cache cannot serve a call from the previous one.

Secondary items, each with the roofline that bounds it:
  tiny        the 2-sequence fp32 workload: latency only (launch-bound)
  long_ctx    8 x 32K-token contexts, Hq 64 / Hkv 8, full attention (split-KV)
  window      the same pools with a 4096-token window (local attention)
  mqa         B = 256 lognormal contexts, 32 query heads on one KV head
  prefill     packed varlen causal prefill (paged write + MFMA prefill)
  chunked_prefill / spec_verify   multi-token queries over the paged cache
  fp8         the headline batch over FP8 pages (quantising write + FP8 decode)
  shared      64 samples decoding from one shared prompt (copy-on-write pages)
and the fp64 CPU oracle timed on the same inputs (headline step, plus one call
of the tiny, long-context, MQA and prefill workloads) as a reported baseline.

``--only LEG[,LEG]`` runs just those items (used for the per-item rocprofv3
counter runs); ``--record-traffic DIR`` turns such runs into
profiles/traffic_counters.json (no GPU needed).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
COPIES = 4

LEGS = ["decode", "tiny", "long_ctx", "window", "mqa", "prefill", "chunked_prefill", "spec_verify", "fp8",
        "fp8_spec", "shared"]

_DECODE_SRC = ["paged_gqa_kv_02_amd/csrc/decode.hip", "paged_gqa_kv_02_amd/csrc/device_common.hpp",
               "paged_gqa_kv_02_amd/csrc/launch.hpp"]
_PREFILL_SRC = ["paged_gqa_kv_02_amd/csrc/prefill.hip", "paged_gqa_kv_02_amd/csrc/device_common.hpp",
                "paged_gqa_kv_02_amd/csrc/launch.hpp"]

# Traffic parts: part -> (workload, kernels whose FETCH_SIZE / WRITE_SIZE add up to
# one timed call of that item, sources they are built from).  Each part's
# counters come from a run of this script with --only <part>.
TRAFFIC_PARTS = {
    "decode": ("llama3_8b_decode", ["decode_split_kernel<2,128,4,1,2>", "decode_merge_kernel<2,128,4>"],
               _DECODE_SRC),
    "long_ctx": ("long_ctx_decode", ["decode_split_kernel<2,128,8,1,2>", "decode_merge_kernel<2,128,8>"],
                 _DECODE_SRC),
    "window": ("long_ctx_decode, window 4096",
               ["decode_split_kernel<2,128,8,1,2>", "decode_merge_kernel<2,128,8>"], _DECODE_SRC),
    "mqa": ("mqa_decode", ["prefill_kernel<128,1,true,false,true,true>", "sk_merge_kernel<128>"],
            _DECODE_SRC + _PREFILL_SRC[:1]),
    "prefill": ("varlen_prefill", ["prefill_kernel<128,4,false,false,false,false>"], _PREFILL_SRC),
    "chunked_prefill": ("chunked_prefill", ["prefill_kernel<128,4,true,false,false,false>"], _PREFILL_SRC),
    "spec_verify": ("spec_verify", ["prefill_kernel<128,1,true,false,true,false>", "sk_merge_kernel<128>"],
                    _PREFILL_SRC),
    "fp8_spec": ("spec_verify over FP8 pages", ["prefill_kernel<128,1,true,true,true,false>", "sk_merge_kernel<128>"],
                 _PREFILL_SRC),
    "fp8": ("llama3_8b_decode over FP8 pages", ["decode_split_kernel<2,128,4,1,1>", "decode_merge_kernel<2,128,4>"],
            _DECODE_SRC),
    "shared": ("shared_prefix_decode", ["decode_split_kernel<2,128,4,1,2>", "decode_merge_kernel<2,128,4>"],
               _DECODE_SRC),
}


def _args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                    help="untimed calls of each item before its warm-up and timing, so the GPU is at its working clocks")
    ap.add_argument("--only", default="", help=f"comma list of items to run ({', '.join(LEGS)}); default: all")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing leg")
    for leg in LEGS[1:]:
        ap.add_argument(f"--no-{leg.replace('_', '-')}", action="store_true", help=f"skip the {leg} item")
    ap.add_argument("--no-extend", action="store_true", help="skip both multi-token items")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum oracle timing budget (headline step)")
    ap.add_argument("--num-splits", type=int, default=0, help="decode work shares (0 = the library's choice)")
    ap.add_argument("--graph", action="store_true",
                    help="replay each headline step as a captured HIP graph instead of launching its kernels one by one")
    ap.add_argument("--record-traffic", metavar="DIR",
                    help="write profiles/traffic_counters.json from the rocprofv3 --pmc runs under DIR "
                         "(DIR/fetch_<item>, DIR/write_<item>); no GPU needed")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (scale for HBM byte counters)")
    return ap.parse_args(argv)


def selected_legs(args) -> list:
    """Items to run: --only wins; otherwise every item not switched off."""
    if args.only:
        legs = [x.strip() for x in args.only.split(",") if x.strip()]
        bad = [x for x in legs if x not in LEGS]
        if bad:
            raise SystemExit(f"unknown item(s) {bad}; known: {LEGS}")
        return legs
    out = ["decode"]
    for leg in LEGS[1:]:
        if getattr(args, "no_" + leg):
            continue
        if leg in ("chunked_prefill", "spec_verify") and args.no_extend:
            continue
        out.append(leg)
    return out


def _sources_hash(here: str, sources) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(here, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(path: str) -> dict:
    """HBM bytes per timed call of each item, from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE record (profiles/), each counter scaled by what it reads for a plain
    copy of known size.  None for an item not recorded, or whose kernel sources have
    changed since the counters were taken."""
    here = os.path.dirname(os.path.abspath(__file__))
    out = {p: None for p in TRAFFIC_PARTS}
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return out
    cal = rec["copy_calibration"]
    for part in TRAFFIC_PARTS:
        r = rec.get(part)
        if not r or _sources_hash(here, r["sources"]) != r["sha256_16"]:
            continue
        out[part] = int(sum(k["fetch_kib"] * 1024 * cal["fetch_factor"] + k["write_kib"] * 1024 * cal["write_factor"]
                            for k in r["kernels"].values()))
    return out


def _kernel_short(name: str) -> str:
    n = name.replace("void ", "").replace("pgqa::", "").replace("(anonymous namespace)::", "")
    return n.split("(")[0].replace(" ", "")


def _counter_means(d: str, counter: str) -> dict:
    """Mean per dispatch of one counter, per kernel (counter instances of a dispatch summed)."""
    import csv
    from collections import defaultdict
    per = defaultdict(float)
    with open(os.path.join(d, "pmc_counter_collection.csv")) as f:
        for x in csv.DictReader(f):
            if x["Counter_Name"] == counter:
                per[(_kernel_short(x["Kernel_Name"]), int(x["Dispatch_Id"]))] += float(x["Counter_Value"])
    agg = defaultdict(list)
    for (k, _), v in per.items():
        agg[k].append(v)
    return {k: sum(v) / len(v) for k, v in agg.items()}


def record_traffic(root: str, path: str) -> dict:
    """Write the per-dispatch FETCH_SIZE / WRITE_SIZE means (KiB) of each item's
    kernels into `path`, with the hash of the sources they were built from (the
    copy calibration already there is kept).  `root` holds, per item, the output
    of
      rocprofv3 --pmc FETCH_SIZE -d ROOT/fetch_<item> -o pmc -- python3 bench.py --only <item>
          --steps 20 --warmup 4 --no-cpu-baseline
    and the same with WRITE_SIZE into ROOT/write_<item>.  Items without both runs
    are left as they were."""
    here = os.path.dirname(os.path.abspath(__file__))
    with open(path) as f:
        rec = json.load(f)
    for part, (workload, kernels, sources) in TRAFFIC_PARTS.items():
        fd, wd = os.path.join(root, f"fetch_{part}"), os.path.join(root, f"write_{part}")
        if not (os.path.isfile(os.path.join(fd, "pmc_counter_collection.csv"))
                and os.path.isfile(os.path.join(wd, "pmc_counter_collection.csv"))):
            continue
        fetch, write = _counter_means(fd, "FETCH_SIZE"), _counter_means(wd, "WRITE_SIZE")
        rec[part] = {"workload": workload, "sources": sources, "sha256_16": _sources_hash(here, sources),
                     "kernels": {k: {"fetch_kib": round(fetch[k], 2), "write_kib": round(write[k], 2)}
                                 for k in kernels}}
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return rec


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _events(torch, n):
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]


SETTLE_MS = 100.0   # untimed work before each item's timing (see _settle)


def _settle(torch, f, ms=None, min_calls=0):
    """Untimed calls f(0), f(1), ... until at least `ms` milliseconds of wall time have
    passed and at least min_calls were made.  After the CPU-side set-up of an item the
    GPU has idled and runs below its working clocks for tens of milliseconds of
    sustained work (varlen prefill measured 175 -> 148 us per call over the first
    ~40 ms), so every timing starts after this phase; nothing inside a timed region
    changes.  Returns the number of calls made."""
    ms = SETTLE_MS if ms is None else ms
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = 0
    while i < min_calls or (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(4):
            f(i)
            i += 1
        torch.cuda.synchronize()
    return i


def _timed_calls(torch, f, n, warm=5):
    """Mean / median / p10 / p90 microseconds of f(i) over n calls, HIP events on the current stream."""
    _settle(torch, f, min_calls=warm)
    evs = _events(torch, n)
    for i in range(n):
        evs[i][0].record()
        f(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) for a, b in evs]) * 1e3
    return {"mean": float(us.mean()), "median": float(np.median(us)), "p10": float(np.percentile(us, 10)),
            "p90": float(np.percentile(us, 90))}


def _hbm_roof(nbytes, us, traffic=None):
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic}


def _mfma_roof(flops, us, traffic=None):
    tf = flops / (us * 1e-6) / 1e12
    return {"bound": "mfma", "achieved": round(tf, 2), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4), "traffic": traffic}


def _decode_pools(torch, pg, T, case, copies):
    table = T.to_dev(case.block_table)
    k_all, v_all = T.to_dev(case.k), T.to_dev(case.v)
    cu_all, sp0 = T.to_dev(case.cu_ctx), T.to_dev(case.start_pos)
    pools = []
    for _ in range(copies):
        kc = T.nan_pool_dev(case.num_blocks, case.num_kv_heads, case.block_size, case.head_dim, case.dtype)
        vc = T.nan_pool_dev(case.num_blocks, case.num_kv_heads, case.block_size, case.head_dim, case.dtype)
        pg.paged_kv_write(k_all, v_all, cu_all, sp0, table, kc, vc)
        pools.append((kc, vc))
    del k_all, v_all
    torch.cuda.synchronize()
    return table, pools


def decode_leg(args, torch, pg, W, T):
    case = W.make_workload("llama3_8b_decode")
    B, hq, hkv, d = case.batch, case.num_q_heads, case.num_kv_heads, case.head_dim
    kv_bytes = case.kv_bytes()
    log(f"decode workload: B={B} ctx sum={int(case.context_lens.sum())} KV bytes={kv_bytes}")
    table, pools = _decode_pools(torch, pg, T, case, COPIES)
    ctx = T.to_dev(case.context_lens)
    # newest token of every sequence (its K/V is written by each step)
    last = case.cu_ctx[1:] - 1
    k_new, v_new = T.to_dev(np.ascontiguousarray(case.k[last])), T.to_dev(np.ascontiguousarray(case.v[last]))
    cu_new = T.to_dev(np.arange(B + 1, dtype=np.int32))
    sp_new = T.to_dev((case.context_lens - 1).astype(np.int32))
    q = T.to_dev(case.q)
    out = torch.empty_like(q)
    ws = pg.decode_workspace(B, hq, hkv, d, args.num_splits, q.device)
    scale = float(case.scale)
    maxctx = case.max_context_len

    def step(i, ev=None):
        kc, vc = pools[i % COPIES]
        pg.paged_kv_write(k_new, v_new, cu_new, sp_new, table, kc, vc)
        if ev is not None:
            ev[0].record()
        pg.gqa_paged_decode(q, kc, vc, table, ctx, maxctx, scale=scale, out=out, num_splits=args.num_splits,
                            workspace=ws)
        if ev is not None:
            ev[1].record()

    # Clock settle (untimed, not counted as warm-up steps), then the W warm-up steps.
    _settle(torch, step)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # One HIP graph per pool copy: paged write + split + merge, replayed as one launch.
    graphs = None
    if args.graph:
        graphs = []
        for i in range(COPIES):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(i)
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % COPIES].replay()
        torch.cuda.synchronize()

    # Timed region: exactly --steps steps between two synchronisations.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graphs is not None:
        for i in range(args.steps):
            graphs[i % COPIES].replay()
    else:
        for i in range(args.steps):
            step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # The decode call alone (split + merge), HIP events on the stream it runs on.
    evs = _events(torch, args.steps)
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    dec_us = np.array([a.elapsed_time(b) for a, b in evs]) * 1e3
    return {
        "case": case, "kv_bytes": kv_bytes, "ms_per_step": ms_per_step,
        "call_us": {"mean": float(dec_us.mean()), "median": float(np.median(dec_us)),
                    "p10": float(np.percentile(dec_us, 10)), "p90": float(np.percentile(dec_us, 90))},
        "out": out,
    }


def tiny_leg(args, torch, pg, W, T):
    """The 2-sequence fp32 workload: a launch-latency-bound call (no roofline)."""
    case = W.make_workload("tiny_f32")
    table, pools = _decode_pools(torch, pg, T, case, 1)
    ctx, q = T.to_dev(case.context_lens), T.to_dev(case.q)
    out = torch.empty_like(q)
    ws = pg.decode_workspace(case.batch, case.num_q_heads, case.num_kv_heads, case.head_dim, 0, q.device)
    f = lambda i: pg.gqa_paged_decode(q, *pools[0], table, ctx, case.max_context_len, scale=float(case.scale),
                                      out=out, workspace=ws)
    us = _timed_calls(torch, f, max(20, args.steps // 2))
    return {"workload": "tiny_f32", "dtype": "f32", "call_us": {k: round(v, 2) for k, v in us.items()},
            "bound": "launch latency (4 KB of K/V)", "out": out}


class _LongCtx:
    """The long-context pools (8 x 32K tokens), written once and shared by the
    full-attention and the windowed items."""
    case = None
    pools = None


def _long_ctx_pools(torch, pg, W, T):
    if _LongCtx.pools is None:
        case = W.make_workload("long_ctx_decode")
        table, pools = _decode_pools(torch, pg, T, case, COPIES)
        _LongCtx.case, _LongCtx.pools, _LongCtx.table = case, pools, table
    return _LongCtx.case, _LongCtx.table, _LongCtx.pools


def long_ctx_leg(args, torch, pg, W, T, traffic=None):
    """Full attention over 8 x 32768 cached tokens (Hq 64, Hkv 8): 1 GiB of K/V per call,
    split across the GPU and merged; four pool copies in rotation."""
    case, table, pools = _long_ctx_pools(torch, pg, W, T)
    q, ctx = T.to_dev(case.q), T.to_dev(case.context_lens)
    out = torch.empty_like(q)
    ws = pg.decode_workspace(case.batch, case.num_q_heads, case.num_kv_heads, case.head_dim, 0, q.device)
    f = lambda i: pg.gqa_paged_decode(q, *pools[i % COPIES], table, ctx, case.max_context_len,
                                      scale=float(case.scale), out=out, workspace=ws)
    us = _timed_calls(torch, f, max(20, args.steps // 2))
    kvb = case.kv_bytes()
    return {"workload": "long_ctx_decode", "batch": case.batch, "context": 32768, "num_q_heads": case.num_q_heads,
            "num_kv_heads": case.num_kv_heads, "kv_bytes_per_call": kvb,
            "call_us": {k: round(v, 2) for k, v in us.items()},
            "tokens_per_s": round(case.batch / (us["mean"] * 1e-6), 1), "roofline": _hbm_roof(kvb, us["mean"], traffic),
            "out": out}


def window_leg(args, torch, pg, W, T, window=4096, traffic=None):
    """Local-attention decode on the long-context pools: each sequence attends to its
    newest `window` positions only, so the pages before the window are never read.
    Bytes = the K/V inside the windows (134 MB per call); the calls rotate over the
    four pool copies (537 MB of windows, more than the Infinity Cache holds)."""
    case, table, pools = _long_ctx_pools(torch, pg, W, T)
    q, ctx = T.to_dev(case.q), T.to_dev(case.context_lens)
    out = torch.empty_like(q)
    ws = pg.decode_workspace(case.batch, case.num_q_heads, case.num_kv_heads, case.head_dim, 0, q.device)
    f = lambda i: pg.gqa_paged_decode(q, *pools[i % COPIES], table, ctx, case.max_context_len,
                                      scale=float(case.scale), out=out, workspace=ws, window=window)
    us = _timed_calls(torch, f, max(20, args.steps // 2))
    row = case.num_kv_heads * case.head_dim * 2 * 2
    kv_w = int(np.minimum(case.context_lens, window).astype(np.int64).sum()) * row
    return {"workload": "long_ctx_decode", "window": window, "kv_bytes_in_window": kv_w,
            "call_us": {k: round(v, 2) for k, v in us.items()}, "roofline": _hbm_roof(kv_w, us["mean"], traffic)}


def mqa_leg(args, torch, pg, W, T, traffic=None):
    """MQA decode (B = 256, lognormal contexts, 32 query heads on one KV head,
    bs 32).  With one KV head and a group of 32 the library routes the call to
    the matrix-core multi-token kernel (the query heads form the packed rows of
    one 32-row MFMA tile, two waves sharing every key block, the batch's key
    blocks cut into one equal stream-K share per workgroup slot, cut sequences
    merged afterwards); the VALU
    split kernel on the same pools (forced by an explicit 1,024-share split) is
    timed beside it.  Calls rotate over four pool copies.  Bytes = the K/V read."""
    case = W.make_workload("mqa_decode")
    table, pools = _decode_pools(torch, pg, T, case, COPIES)
    q, ctx = T.to_dev(case.q), T.to_dev(case.context_lens)
    out = torch.empty_like(q)
    ws = pg.decode_workspace(case.batch, case.num_q_heads, case.num_kv_heads, case.head_dim, 0, q.device)

    def run(splits, o):
        f = lambda i: pg.gqa_paged_decode(q, *pools[i % COPIES], table, ctx, case.max_context_len,
                                          scale=float(case.scale), out=o, workspace=ws, num_splits=splits)
        return _timed_calls(torch, f, max(20, args.steps // 2))

    us = run(0, out)
    us_split = run(1024, torch.empty_like(q))
    kvb = case.kv_bytes()
    return {
        "workload": "mqa_decode", "batch": case.batch, "num_q_heads": case.num_q_heads,
        "num_kv_heads": case.num_kv_heads, "block_size": case.block_size, "kv_bytes_per_call": kvb,
        "route": "matrix-core multi-token kernel (query heads as the packed rows of one MFMA tile)",
        "call_us": {k: round(v, 2) for k, v in us.items()}, "split_kernel_us_mean": round(us_split["mean"], 2),
        "speedup_vs_split_kernel": round(us_split["mean"] / us["mean"], 3),
        "tokens_per_s": round(case.batch / (us["mean"] * 1e-6), 1), "roofline": _hbm_roof(kvb, us["mean"], traffic),
        "out": out,
    }


def prefill_leg(args, torch, pg, W, T, traffic=None):
    p = W.make_workload("varlen_prefill")
    q, k, v = T.to_dev(p.q), T.to_dev(p.k), T.to_dev(p.v)
    cu = T.to_dev(p.cu_seqlens)
    sp = T.to_dev(np.zeros(p.batch, np.int32))
    table = T.to_dev(p.block_table)
    kc = T.nan_pool_dev(p.num_blocks, p.num_kv_heads, p.block_size, p.head_dim, p.dtype)
    vc = T.nan_pool_dev(p.num_blocks, p.num_kv_heads, p.block_size, p.head_dim, p.dtype)
    out = torch.empty_like(q)
    scale = float(p.scale)

    def step(ev=None):
        pg.paged_kv_write(k, v, cu, sp, table, kc, vc)
        if ev is not None:
            ev[0].record()
        pg.gqa_varlen_prefill(q, k, v, cu, p.max_seqlen, scale=scale, causal=True, out=out)
        if ev is not None:
            ev[1].record()

    _settle(torch, lambda i: step(), min_calls=max(3, args.warmup // 4))
    n = max(10, args.steps // 4)
    evs = _events(torch, n)
    t0 = time.perf_counter()
    for i in range(n):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    us = np.array([a.elapsed_time(b) for a, b in evs]) * 1e3
    # The same call back to back (no paged write between): the kernel in steady state.
    b2b = _timed_calls(torch, lambda i: pg.gqa_varlen_prefill(q, k, v, cu, p.max_seqlen, scale=scale, causal=True,
                                                              out=out), n)
    flops = p.flops()
    return {
        "workload": "varlen_prefill", "tokens": p.total_tokens, "flops_per_call": flops,
        "call_us": {"mean": round(float(us.mean()), 2), "median": round(float(np.median(us)), 2)},
        "back_to_back_us": {k_: round(v_, 2) for k_, v_ in b2b.items()},
        "back_to_back_tflops": round(flops / (b2b["mean"] * 1e-6) / 1e12, 2),
        "ms_per_step": wall * 1e3 / n, "tflops": round(flops / (us.mean() * 1e-6) / 1e12, 2),
        "tokens_per_s": round(p.total_tokens / (us.mean() * 1e-6), 1),
        "roofline": _mfma_roof(flops, float(us.mean()), traffic), "out": out,
    }


def extend_leg(key, args, torch, pg, W, T, traffic=None, fp8=False):
    """One multi-token step on a named workload: write the new tokens' K/V into
    their pages, then gqa_paged_extend over prefix + new tokens.  HIP events
    bracket the extend call; two pool copies alternate between steps.  fp8: the
    same over FP8 pages (quantising write, gqa_paged_extend_fp8); bytes are then
    the codes and row scales stored."""
    c = W.make_workload(key)
    q, cu_q = T.to_dev(c.q), T.to_dev(c.cu_q)
    table, ctx = T.to_dev(c.block_table), T.to_dev(c.context_lens)
    pools = []
    for _ in range(2):
        if fp8:
            p4 = pg.fp8_pools(c.num_blocks, c.num_kv_heads, c.block_size, c.head_dim)
            pg.paged_kv_write_fp8(T.to_dev(c.k), T.to_dev(c.v), T.to_dev(c.cu_ctx), T.to_dev(c.start_pos), table,
                                  *p4)
            pools.append(p4)
            continue
        kc = T.nan_pool_dev(c.num_blocks, c.num_kv_heads, c.block_size, c.head_dim, c.dtype)
        vc = T.nan_pool_dev(c.num_blocks, c.num_kv_heads, c.block_size, c.head_dim, c.dtype)
        pg.paged_kv_write(T.to_dev(c.k), T.to_dev(c.v), T.to_dev(c.cu_ctx), T.to_dev(c.start_pos), table, kc, vc)
        pools.append((kc, vc))
    new_rows = np.concatenate([np.arange(c.cu_ctx[b + 1] - c.q_lens[b], c.cu_ctx[b + 1])
                               for b in range(c.batch)]).astype(np.int64)
    k_new, v_new = T.to_dev(np.ascontiguousarray(c.k[new_rows])), T.to_dev(np.ascontiguousarray(c.v[new_rows]))
    sp_new = T.to_dev((c.context_lens - c.q_lens).astype(np.int32))
    out = torch.empty_like(q)
    scale = float(c.scale)

    def step(i, ev=None):
        pool = pools[i % 2]
        if fp8:
            pg.paged_kv_write_fp8(k_new, v_new, cu_q, sp_new, table, *pool)
        else:
            pg.paged_kv_write(k_new, v_new, cu_q, sp_new, table, *pool)
        if ev is not None:
            ev[0].record()
        if fp8:
            pg.gqa_paged_extend_fp8(q, cu_q, *pool, table, ctx, c.max_q_len, c.max_context_len, scale=scale, out=out)
        else:
            pg.gqa_paged_extend(q, cu_q, *pool, table, ctx, c.max_q_len, c.max_context_len, scale=scale, out=out)
        if ev is not None:
            ev[1].record()

    _settle(torch, step, min_calls=max(4, args.warmup // 4))
    n = max(10, args.steps // 4)
    evs = _events(torch, n)
    t0 = time.perf_counter()
    for i in range(n):
        step(i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    us = float(np.mean([a.elapsed_time(b) for a, b in evs]) * 1e3)
    flops, kv = c.flops(), c.kv_bytes()
    if fp8:
        kv = kv // (2 * c.head_dim) * (c.head_dim + 4)   # per token and KV head: d code bytes + a 4-byte scale
    # Bound by arithmetic intensity against the ridge point (peak FLOP/s / peak B/s).
    mfma = flops / kv > BF16_MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    return {
        "workload": key, "kv_format": "fp8 e4m3 + fp32 row scale" if fp8 else "bf16", "batch": c.batch,
        "query_tokens": c.total_q, "flops_per_call": flops,
        "kv_bytes_per_call": kv, "call_us_mean": round(us, 2), "ms_per_step": wall * 1e3 / n,
        "tflops": round(flops / (us * 1e-6) / 1e12, 2), "kv_gbs": round(kv / (us * 1e-6) / 1e9, 2),
        "query_tokens_per_s": round(c.total_q / (us * 1e-6), 1),
        "roofline": _mfma_roof(flops, us, traffic) if mfma else _hbm_roof(kv, us, traffic),
    }


def fp8_leg(args, torch, pg, W, T, traffic=None):
    """Decode of the headline workload over FP8 pages (codes + one fp32 scale per
    token and KV head), written by the quantising paged write.  Step = quantising
    write of the 64 newest tokens + FP8 decode; the decode call is event-timed.
    Bytes = codes + row scales actually stored (264 B per token and KV head for
    d 128, against 512 B in bf16)."""
    case = W.make_workload("llama3_8b_decode")
    B, hq, hkv, d, bs = case.batch, case.num_q_heads, case.num_kv_heads, case.head_dim, case.block_size
    table, ctx = T.to_dev(case.block_table), T.to_dev(case.context_lens)
    pools = []
    for _ in range(COPIES):
        kc, vc, ks, vs = pg.fp8_pools(case.num_blocks, hkv, bs, d)
        pg.paged_kv_write_fp8(T.to_dev(case.k), T.to_dev(case.v), T.to_dev(case.cu_ctx), T.to_dev(case.start_pos),
                              table, kc, vc, ks, vs)
        pools.append((kc, vc, ks, vs))
    last = case.cu_ctx[1:] - 1
    k_new, v_new = T.to_dev(np.ascontiguousarray(case.k[last])), T.to_dev(np.ascontiguousarray(case.v[last]))
    cu_new = T.to_dev(np.arange(B + 1, dtype=np.int32))
    sp_new = T.to_dev((case.context_lens - 1).astype(np.int32))
    q = T.to_dev(case.q)
    out = torch.empty_like(q)
    ws = pg.decode_workspace(B, hq, hkv, d, 0, q.device)
    scale, maxctx = float(case.scale), case.max_context_len

    def step(i, ev=None):
        kc, vc, ks, vs = pools[i % COPIES]
        pg.paged_kv_write_fp8(k_new, v_new, cu_new, sp_new, table, kc, vc, ks, vs)
        if ev is not None:
            ev[0].record()
        pg.gqa_paged_decode_fp8(q, kc, vc, ks, vs, table, ctx, maxctx, scale=scale, out=out, workspace=ws)
        if ev is not None:
            ev[1].record()

    _settle(torch, step, min_calls=args.warmup)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    evs = _events(torch, args.steps)
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in evs]) * 1e3)
    tokens = int(case.context_lens.astype(np.int64).sum())
    stored = tokens * hkv * 2 * (d + 4)
    return {
        "workload": "llama3_8b_decode", "kv_format": "fp8 e4m3 + fp32 row scale", "bytes_per_call": stored,
        "bf16_equivalent_bytes": case.kv_bytes(), "call_us_mean": round(us, 2), "ms_per_step": ms_step,
        "kv_gbs": round(stored / (us * 1e-6) / 1e9, 2),
        "bf16_equivalent_gbs": round(case.kv_bytes() / (us * 1e-6) / 1e9, 2),
        "roofline": _hbm_roof(stored, us, traffic),
    }


def shared_prefix_leg(args, torch, pg, W, T, traffic=None):
    """Decode over pages shared by samples of one prompt.  The library's block
    manager builds the tables (prompt stored once, its partly filled last block
    copied on write by each sample), then each step rewrites every sample's newest
    token and decodes, as in the headline step; steps rotate over four copies of
    the shared pools.  The same samples laid out with no sharing are decoded too
    (one pool copy: 2.4 GB, far beyond the Infinity Cache), for the comparison and
    a bitwise check."""
    c = W.make_workload("shared_prefix_decode")
    B, hq, hkv, d, bs, P = c.batch, c.num_q_heads, c.num_kv_heads, c.head_dim, c.block_size, c.prompt_len
    pool = -(-P // bs) + int(sum(-(-int(n) // bs) + 1 for n in c.cont_lens)) + 8
    bm = pg.BlockManager(pool, bs)
    kc = T.nan_pool_dev(pool, hkv, bs, d, c.dtype)
    vc = T.nan_pool_dev(pool, hkv, bs, d, c.dtype)
    root = bm.new_sequence()
    bm.append(root, P)
    pg.paged_kv_write(T.to_dev(c.k_prompt), T.to_dev(c.v_prompt), T.to_dev(np.array([0, P], np.int32)),
                      T.to_dev(np.zeros(1, np.int32)), T.to_dev(bm.block_tables([root])), kc, vc)
    kids = [bm.fork(root) for _ in range(B)]
    cps = [cp for cp in (bm.append(s, int(n)) for s, n in zip(kids, c.cont_lens)) if cp is not None]
    if cps:
        pg.paged_kv_copy_blocks(kc, vc, T.to_dev(np.array([a for a, _ in cps], np.int32)),
                                T.to_dev(np.array([b for _, b in cps], np.int32)))
    table = T.to_dev(bm.block_tables(kids))
    pg.paged_kv_write(T.to_dev(c.k_cont), T.to_dev(c.v_cont), T.to_dev(c.cu_cont), T.to_dev(np.full(B, P, np.int32)),
                      table, kc, vc)
    bm.free(root)
    blocks_used = pool - bm.num_free_blocks()
    pools = [(kc, vc)] + [(kc.clone(), vc.clone()) for _ in range(COPIES - 1)]
    ctx_np = c.context_lens
    ctx = T.to_dev(ctx_np)
    last = c.cu_cont[1:] - 1
    k_new, v_new = T.to_dev(np.ascontiguousarray(c.k_cont[last])), T.to_dev(np.ascontiguousarray(c.v_cont[last]))
    cu_new = T.to_dev(np.arange(B + 1, dtype=np.int32))
    sp_new = T.to_dev((ctx_np - 1).astype(np.int32))
    q = T.to_dev(c.q)
    scale, maxctx = float(c.scale), int(ctx_np.max())
    ws = pg.decode_workspace(B, hq, hkv, d, 0, q.device)

    def timed(pools_, table_, out, n):
        def step(i, ev=None):
            kc_, vc_ = pools_[i % len(pools_)]
            pg.paged_kv_write(k_new, v_new, cu_new, sp_new, table_, kc_, vc_)
            if ev is not None:
                ev[0].record()
            pg.gqa_paged_decode(q, kc_, vc_, table_, ctx, maxctx, scale=scale, out=out, workspace=ws)
            if ev is not None:
                ev[1].record()
        _settle(torch, step, min_calls=max(5, args.warmup // 2))
        evs = _events(torch, n)
        t0 = time.perf_counter()
        for i in range(n):
            step(i, evs[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return np.array([a.elapsed_time(b) for a, b in evs]), wall * 1e3 / n

    out_sh = torch.empty_like(q)
    ms_sh, step_sh = timed(pools, table, out_sh, max(20, args.steps // 2))
    res = {"workload": "shared_prefix_decode", "batch": B, "prompt_len": P, "blocks_used": blocks_used,
           "cow_copies": len(cps)}
    logical, unique = c.logical_kv_bytes(), c.unique_kv_bytes()
    us = float(ms_sh.mean() * 1e3)
    if "shared" not in args.only.split(","):   # the unshared comparison (left out of a counter run)
        u = c.logical(np.random.default_rng(c.seed))
        ukc = T.nan_pool_dev(u.num_blocks, hkv, bs, d, c.dtype)
        uvc = T.nan_pool_dev(u.num_blocks, hkv, bs, d, c.dtype)
        utable = T.to_dev(u.block_table)
        pg.paged_kv_write(T.to_dev(u.k), T.to_dev(u.v), T.to_dev(u.cu_ctx), T.to_dev(u.start_pos), utable, ukc, uvc)
        out_un = torch.empty_like(q)
        ms_un, _ = timed([(ukc, uvc)], utable, out_un, max(10, args.steps // 4))
        res.update({"blocks_unshared": int((u.block_table >= 0).sum()),
                    "unshared_call_us_mean": round(float(ms_un.mean() * 1e3), 2),
                    "speedup_vs_unshared": round(float(ms_un.mean() / ms_sh.mean()), 3),
                    "bit_identical_to_unshared": bool(torch.equal(out_sh.view(torch.int16), out_un.view(torch.int16)))})
    res.update({"logical_kv_bytes": logical, "unique_kv_bytes": unique, "call_us_mean": round(us, 2),
                "ms_per_step": step_sh, "logical_kv_gbs": round(logical / (us * 1e-6) / 1e9, 2),
                "roofline": dict(_hbm_roof(unique, us, traffic),
                                 bytes="unique K/V bytes (prompt once + continuations), the HBM floor")})
    return res


def _oracle_timed(fn, min_s):
    """Seconds per call of fn (repeated until min_s of wall time), and its last result."""
    reps, t0 = 0, time.perf_counter()
    while True:
        ref = fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_s or reps >= 1000:
            return el / reps, reps, el, ref


def cpu_baseline(args, W, gpu):
    """The fp64 oracle, as it stands, on the inputs the GPU items use: the headline
    decode step (write + decode, repeated for at least --cpu-seconds), then one call
    of the tiny, long-context, MQA and packed-prefill workloads (a bounded sample:
    each is a single call, or repeated up to about a second when it is shorter).
    Returns the cpu_baseline object and the oracle outputs for the parity check."""
    import oracle
    orc = oracle.default()
    refs = {}

    def pools(case):
        kc = W.nan_pool(case.num_blocks, case.num_kv_heads, case.block_size, case.head_dim, case.dtype)
        vc = W.nan_pool(case.num_blocks, case.num_kv_heads, case.block_size, case.head_dim, case.dtype)
        orc.paged_kv_write(case.k, case.v, case.cu_ctx, case.start_pos, case.block_table, kc, vc)
        return kc, vc

    case = W.make_workload("llama3_8b_decode")
    kc, vc = pools(case)
    last = case.cu_ctx[1:] - 1
    cu_new = np.arange(case.batch + 1, dtype=np.int32)
    sp_new = (case.context_lens - 1).astype(np.int32)
    k_new, v_new = np.ascontiguousarray(case.k[last]), np.ascontiguousarray(case.v[last])

    def step():
        orc.paged_kv_write(k_new, v_new, cu_new, sp_new, case.block_table, kc, vc)
        return orc.gqa_paged_decode(case.q, kc, vc, case.block_table, case.context_lens, case.scale)

    per_step, reps, el, refs["decode"] = _oracle_timed(step, args.cpu_seconds)
    out = {"value": round(case.kv_bytes() / per_step / 1e9, 3), "unit": "GB/s", "cores": orc.max_threads(),
           "kind": "oracle", "seconds_per_step": per_step,
           "sample": f"the full decode step of the same workload (paged write of the 64 newest tokens + "
                     f"fp64 decode of all 64 sequences), repeated {reps}x over {el:.1f} s",
           "per_config": {}}
    for key, leg in (("tiny_f32", "tiny"), ("long_ctx_decode", "long_ctx"), ("mqa_decode", "mqa")):
        c = W.make_workload(key)
        ck, cv = pools(c)
        s, reps, el, refs[leg] = _oracle_timed(
            lambda: orc.gqa_paged_decode(c.q, ck, cv, c.block_table, c.context_lens, c.scale), 1.0)
        e = {"oracle_s_per_call": s, "sample": f"one decode call of the whole workload, repeated {reps}x over {el:.2f} s"}
        if leg in gpu:
            e["gpu_us_per_call"] = gpu[leg]
            e["oracle_over_gpu"] = round(s / (gpu[leg] * 1e-6), 1)
        out["per_config"][key] = e
    p = W.make_workload("varlen_prefill")
    s, reps, el, refs["prefill"] = _oracle_timed(
        lambda: orc.gqa_varlen_prefill(p.q, p.k, p.v, p.cu_seqlens, p.scale, causal=True), 0.0)
    e = {"oracle_s_per_call": s, "sample": "one causal prefill call of the whole packed batch (16,209 rows)"}
    if "prefill" in gpu:
        e["gpu_us_per_call"] = gpu["prefill"]
        e["oracle_over_gpu"] = round(s / (gpu["prefill"] * 1e-6), 1)
    out["per_config"]["varlen_prefill"] = e
    return out, refs


def main(argv=None):
    global SETTLE_MS
    args = _args(argv)
    SETTLE_MS = max(0.0, args.settle_ms)
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        return 2
    here = os.path.dirname(os.path.abspath(__file__))
    if args.record_traffic:
        rec = record_traffic(args.record_traffic, os.path.join(here, "profiles", "traffic_counters.json"))
        print(json.dumps({k: rec.get(k) for k in TRAFFIC_PARTS}), flush=True)
        return 0
    legs = selected_legs(args)
    sys.path.insert(0, here)
    sys.path.insert(0, os.path.join(here, "tests"))
    import torch
    import workload as W
    import paged_gqa_kv_02_amd as pg
    import gpu_helpers as T
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.calibrate_copy:
        # A plain copy of known size: its FETCH_SIZE / WRITE_SIZE per dispatch give
        # the counter-to-bytes scale used for the kernels' HBM traffic.
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "dispatches": 5}), flush=True)
        return 0

    traffic = recorded_traffic(os.path.join(here, "profiles", "traffic_counters.json"))
    line = {"metric": "decode KV-read GB/s (Llama-3-8B-shaped GQA decode, B=64)", "value": None, "unit": "GB/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1), bf16-rounded)",
            "settle_ms": args.settle_ms}
    outs, gpu_us = {}, {}
    if "decode" in legs:
        dec = decode_leg(args, torch, pg, W, T)
        kv, case = dec["kv_bytes"], dec["case"]
        outs["decode"] = dec["out"]
        line.update({
            "value": round(kv / (dec["ms_per_step"] * 1e-3) / 1e9, 2), "ms_per_step": round(dec["ms_per_step"], 5),
            "config": {"workload": "llama3_8b_decode", "batch": case.batch, "num_q_heads": case.num_q_heads,
                       "num_kv_heads": case.num_kv_heads, "head_dim": case.head_dim, "block_size": case.block_size,
                       "context_lens": W.WORKLOADS["llama3_8b_decode"].description, "kv_bytes_per_step": kv,
                       "tokens_per_step": case.batch, "launch": "hip_graph" if args.graph else "eager"},
            "tokens_per_s": round(case.batch / (dec["ms_per_step"] * 1e-3), 1),
            "decode_call_us": {k: round(v, 2) for k, v in dec["call_us"].items()},
            "roofline": dict(_hbm_roof(kv, dec["call_us"]["mean"], traffic["decode"]),
                             kernel="gqa_paged_decode (split + merge kernels, one call)"),
        })
    if "tiny" in legs:
        log("tiny fp32 leg")
        r = tiny_leg(args, torch, pg, W, T)
        outs["tiny"] = r.pop("out")
        gpu_us["tiny"] = r["call_us"]["mean"]
        line["tiny"] = r
    if "long_ctx" in legs:
        log("long-context leg")
        r = long_ctx_leg(args, torch, pg, W, T, traffic["long_ctx"])
        outs["long_ctx"] = r.pop("out")
        gpu_us["long_ctx"] = r["call_us"]["mean"]
        line["long_ctx"] = r
    if "window" in legs:
        log("sliding window leg")
        line["window"] = window_leg(args, torch, pg, W, T, traffic=traffic["window"])
    _LongCtx.pools = None
    torch.cuda.empty_cache()
    if "mqa" in legs:
        log("mqa decode leg")
        r = mqa_leg(args, torch, pg, W, T, traffic["mqa"])
        outs["mqa"] = r.pop("out")
        gpu_us["mqa"] = r["call_us"]["mean"]
        line["mqa"] = r
    if "prefill" in legs:
        log("prefill leg")
        r = prefill_leg(args, torch, pg, W, T, traffic["prefill"])
        outs["prefill"] = r.pop("out")
        gpu_us["prefill"] = r["call_us"]["mean"]
        line["prefill"] = r
    for key in ("chunked_prefill", "spec_verify"):
        if key in legs:
            log(f"extend leg {key}")
            line.setdefault("extend", {})[key] = extend_leg(key, args, torch, pg, W, T, traffic[key])
    if "fp8" in legs:
        log("fp8 pages leg")
        line["fp8"] = fp8_leg(args, torch, pg, W, T, traffic["fp8"])
        if "decode_call_us" in line:
            line["fp8"]["speedup_vs_bf16_call"] = round(line["decode_call_us"]["mean"] / line["fp8"]["call_us_mean"], 3)
    if "fp8_spec" in legs:
        log("fp8 pages, multi-token leg")
        line["fp8_spec_verify"] = extend_leg("spec_verify", args, torch, pg, W, T, traffic["fp8_spec"], fp8=True)
    if "shared" in legs:
        log("shared prefix leg")
        line["shared_prefix"] = shared_prefix_leg(args, torch, pg, W, T, traffic["shared"])
    if not args.no_cpu_baseline and "decode" in legs:
        log("cpu baseline leg (oracle)")
        cb, refs = cpu_baseline(args, W, gpu_us)
        line["cpu_baseline"] = cb
        line["parity_vs_oracle"] = {}
        for leg, out in outs.items():
            e = T.errors(T.to_f64(out), refs[leg])
            line["parity_vs_oracle"][leg] = {k: float(f"{v:.3e}") for k, v in e.items()}
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
