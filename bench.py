#!/usr/bin/env python3
"""Benchmark of the paged GQA hot path on one MI355X.

Headline: decode KV-read GB/s on the Llama-3-8B-shaped decode workload (B = 64,
context lengths U[512, 4096], Hq = 32, Hkv = 8, d = 128, block_size 16, bf16).
One step = the decode step of the hot path on that batch:
  1. paged_kv_write of each sequence's newest token (position ctx-1) into its page,
  2. gqa_paged_decode over every cached position (split-KV + merge kernels).
``value`` = algorithmic K/V bytes read per step / wall time per step, the three
kernels launched one by one (``--graph`` replays each step as a captured HIP
graph instead; on this stack that is ~3 % slower).  ``roofline`` times the decode
call alone (split + merge) with HIP events on its stream, in a second pass.

Inputs stay resident in HBM.  Four copies of the page pools (about 0.77 GB each)
are used round-robin, so the 256 MB Infinity Cache cannot serve a step from the
previous one.  Secondary line items: the packed varlen causal prefill workload
(paged write + MFMA prefill) in TFLOP/s; multi-token queries over the paged
cache (chunked prefill of 512-token chunks on cached prefixes, and checking 4
draft tokens per sequence), each with the roofline its arithmetic intensity
puts it under; decode of 64 samples over the pages of one shared prompt
(prefix sharing with copy-on-write), against the same samples unshared;
local-attention decode (4096-token window) on the long-context workload;
decode of the headline batch over FP8 pages (quantising write + FP8 decode); and
the fp64 CPU oracle on the same decode batch as a reported baseline.
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


def _args():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing leg")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill line item")
    ap.add_argument("--no-extend", action="store_true", help="skip the multi-token (extend) line items")
    ap.add_argument("--no-shared", action="store_true", help="skip the shared-prefix decode line item")
    ap.add_argument("--no-window", action="store_true", help="skip the sliding-window decode line item")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8-page decode line item")
    ap.add_argument("--no-mqa", action="store_true", help="skip the one-KV-head (MQA) decode line item")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum oracle timing budget")
    ap.add_argument("--decode-workload", default="llama3_8b_decode",
                    choices=["llama3_8b_decode", "long_ctx_decode", "mqa_decode", "tiny_f32"],
                    help="decode workload to time (the headline is llama3_8b_decode)")
    ap.add_argument("--num-splits", type=int, default=0,
                    help="decode work shares (0 = the library's choice)")
    ap.add_argument("--graph", action="store_true",
                    help="replay each step as a captured HIP graph instead of launching its kernels one by one")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic_counters.json from two rocprofv3 --pmc runs (no GPU needed)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (scale for HBM byte counters)")
    return ap.parse_args()


def recorded_traffic(path: str):
    """HBM bytes per call of the decode call and of the prefill kernel, from the
    committed rocprofv3 FETCH_SIZE / WRITE_SIZE record (profiles/), each counter
    scaled by what it reads for a plain copy of known size.  None for a path whose
    sources have changed since the counters were taken."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return {"decode": None, "prefill": None}
    cal = rec["copy_calibration"]
    out = {}
    for part in ("decode", "prefill"):
        r = rec.get(part)
        if r is None:
            out[part] = None
            continue
        h = hashlib.sha256()
        for f in r["sources"]:
            with open(os.path.join(here, f), "rb") as fh:
                h.update(fh.read())
        if h.hexdigest()[:16] != r["sha256_16"]:
            out[part] = None
            continue
        out[part] = int(sum(k["fetch_kib"] * 1024 * cal["fetch_factor"] + k["write_kib"] * 1024 * cal["write_factor"]
                            for k in r["kernels"].values()))
    return out


TRAFFIC_PARTS = {
    # part -> (kernels whose FETCH_SIZE / WRITE_SIZE add up to one call, sources they are built from)
    "decode": (["decode_split_kernel<2,128,4,1,2>", "decode_merge_kernel<2,128,4>"],
               ["paged_gqa_kv_02_amd/csrc/decode.hip", "paged_gqa_kv_02_amd/csrc/device_common.hpp",
                "paged_gqa_kv_02_amd/csrc/launch.hpp"]),
    "prefill": (["prefill_kernel<128,4,false>"],
                ["paged_gqa_kv_02_amd/csrc/prefill.hip", "paged_gqa_kv_02_amd/csrc/device_common.hpp",
                 "paged_gqa_kv_02_amd/csrc/launch.hpp"]),
}


def _kernel_short(name: str) -> str:
    n = name.replace("void ", "").replace("pgqa::", "").replace("(anonymous namespace)::", "")
    return n.split("(")[0].replace(" ", "")


def record_traffic(fetch_dir: str, write_dir: str, path: str) -> dict:
    """Write the per-dispatch FETCH_SIZE / WRITE_SIZE means (KiB) of the decode and
    prefill kernels from two rocprofv3 --pmc runs of this script into `path`, with
    the hash of the sources they belong to (the copy calibration already there is
    kept).  Run on the output of
      rocprofv3 --pmc FETCH_SIZE -d FETCH_DIR -o pmc -- python3 bench.py --steps 20 --warmup 4
          --no-cpu-baseline --no-extend --no-shared --no-window
    and the same with WRITE_SIZE."""
    import csv
    import hashlib
    from collections import defaultdict
    here = os.path.dirname(os.path.abspath(__file__))

    def means(d, counter):
        per = defaultdict(float)
        with open(os.path.join(d, "pmc_counter_collection.csv")) as f:
            for x in csv.DictReader(f):
                if x["Counter_Name"] == counter:
                    per[(_kernel_short(x["Kernel_Name"]), int(x["Dispatch_Id"]))] += float(x["Counter_Value"])
        agg = defaultdict(list)
        for (k, _), v in per.items():
            agg[k].append(v)
        return {k: sum(v) / len(v) for k, v in agg.items()}

    fetch, write = means(fetch_dir, "FETCH_SIZE"), means(write_dir, "WRITE_SIZE")
    with open(path) as f:
        rec = json.load(f)
    for part, (kernels, sources) in TRAFFIC_PARTS.items():
        h = hashlib.sha256()
        for src in sources:
            with open(os.path.join(here, src), "rb") as fh:
                h.update(fh.read())
        rec[part] = {"workload": rec.get(part, {}).get("workload", ""), "sources": sources,
                     "sha256_16": h.hexdigest()[:16],
                     "kernels": {k: {"fetch_kib": round(fetch[k], 2), "write_kib": round(write[k], 2)}
                                 for k in kernels}}
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return rec


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def decode_leg(args, torch, pg, W, T):
    case = W.make_workload(args.decode_workload)
    B, hq, hkv, d, bs = case.batch, case.num_q_heads, case.num_kv_heads, case.head_dim, case.block_size
    kv_bytes = case.kv_bytes()
    log(f"decode workload: B={B} ctx sum={int(case.context_lens.sum())} KV bytes={kv_bytes}")

    table = T.to_dev(case.block_table)
    ctx = T.to_dev(case.context_lens)
    k_all, v_all = T.to_dev(case.k), T.to_dev(case.v)
    cu_all, sp0 = T.to_dev(case.cu_ctx), T.to_dev(case.start_pos)
    # newest token of every sequence (its K/V is written by each step)
    last = case.cu_ctx[1:] - 1
    k_new, v_new = T.to_dev(np.ascontiguousarray(case.k[last])), T.to_dev(np.ascontiguousarray(case.v[last]))
    cu_new = T.to_dev(np.arange(B + 1, dtype=np.int32))
    sp_new = T.to_dev((case.context_lens - 1).astype(np.int32))
    q = T.to_dev(case.q)
    pools = []
    for _ in range(COPIES):
        kc = T.nan_pool_dev(case.num_blocks, hkv, bs, d, case.dtype)
        vc = T.nan_pool_dev(case.num_blocks, hkv, bs, d, case.dtype)
        pg.paged_kv_write(k_all, v_all, cu_all, sp0, table, kc, vc)
        pools.append((kc, vc))
    del k_all, v_all
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
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    dec_ms = np.array([a.elapsed_time(b) for a, b in evs])
    return {
        "case": case, "kv_bytes": kv_bytes, "ms_per_step": ms_per_step,
        "decode_ms_mean": float(dec_ms.mean()), "decode_ms_median": float(np.median(dec_ms)),
        "decode_ms_p10": float(np.percentile(dec_ms, 10)), "decode_ms_p90": float(np.percentile(dec_ms, 90)),
        "out": out, "pools": pools,
    }


def prefill_leg(args, torch, pg, W, T):
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

    for _ in range(max(3, args.warmup // 4)):
        step()
    torch.cuda.synchronize()
    n = max(10, args.steps // 4)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    t0 = time.perf_counter()
    for i in range(n):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_ms = np.array([a.elapsed_time(b) for a, b in evs])
    flops = p.flops()
    tf = flops / (pre_ms.mean() * 1e-3) / 1e12
    return {
        "workload": "varlen_prefill", "tokens": p.total_tokens, "flops_per_call": flops,
        "prefill_ms_mean": float(pre_ms.mean()), "ms_per_step": wall * 1e3 / n,
        "tflops": tf, "tokens_per_s": p.total_tokens / (pre_ms.mean() * 1e-3),
        "roofline": {"bound": "mfma", "achieved": tf, "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / BF16_MFMA_PEAK_TFLOPS, "traffic": None},
    }


def extend_leg(key, args, torch, pg, W, T):
    """One multi-token step on a named workload: write the new tokens' K/V into
    their pages, then gqa_paged_extend over prefix + new tokens.  HIP events
    bracket the extend call; two pool copies alternate between steps."""
    c = W.make_workload(key)
    q, cu_q = T.to_dev(c.q), T.to_dev(c.cu_q)
    table, ctx = T.to_dev(c.block_table), T.to_dev(c.context_lens)
    pools = []
    for _ in range(2):
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
        kc, vc = pools[i % 2]
        pg.paged_kv_write(k_new, v_new, cu_q, sp_new, table, kc, vc)
        if ev is not None:
            ev[0].record()
        pg.gqa_paged_extend(q, cu_q, kc, vc, table, ctx, c.max_q_len, c.max_context_len, scale=scale, out=out)
        if ev is not None:
            ev[1].record()

    for i in range(max(4, args.warmup // 4)):
        step(i)
    torch.cuda.synchronize()
    n = max(10, args.steps // 4)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    t0 = time.perf_counter()
    for i in range(n):
        step(i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    flops, kv = c.flops(), c.kv_bytes()
    tf = flops / (ms.mean() * 1e-3) / 1e12
    gbs = kv / (ms.mean() * 1e-3) / 1e9
    # Bound by arithmetic intensity against the ridge point (peak FLOP/s / peak B/s).
    mfma = flops / kv > BF16_MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    roof = ({"bound": "mfma", "achieved": tf, "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
             "frac": tf / BF16_MFMA_PEAK_TFLOPS, "traffic": None} if mfma else
            {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
             "traffic": None})
    return {
        "workload": key, "batch": c.batch, "query_tokens": c.total_q, "flops_per_call": flops,
        "kv_bytes_per_call": kv, "extend_us_mean": float(ms.mean() * 1e3), "extend_us_median": float(np.median(ms) * 1e3),
        "ms_per_step": wall * 1e3 / n, "tflops": tf, "kv_gbs": gbs,
        "query_tokens_per_s": c.total_q / (ms.mean() * 1e-3), "roofline": roof,
    }


def shared_prefix_leg(args, torch, pg, W, T):
    """Decode over pages shared by samples of one prompt.  The library's block
    manager builds the tables (prompt stored once, its partly filled last block
    copied on write by each sample), then each step rewrites every sample's newest
    token and decodes, as in the headline step.  The same samples laid out with no
    sharing are decoded too, for the comparison and a bitwise check."""
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
    cu_cont = c.cu_cont
    pg.paged_kv_write(T.to_dev(c.k_cont), T.to_dev(c.v_cont), T.to_dev(cu_cont), T.to_dev(np.full(B, P, np.int32)),
                      table, kc, vc)
    bm.free(root)
    blocks_used = pool - bm.num_free_blocks()
    ctx_np = c.context_lens
    ctx = T.to_dev(ctx_np)
    last = cu_cont[1:] - 1
    k_new, v_new = T.to_dev(np.ascontiguousarray(c.k_cont[last])), T.to_dev(np.ascontiguousarray(c.v_cont[last]))
    cu_new = T.to_dev(np.arange(B + 1, dtype=np.int32))
    sp_new = T.to_dev((ctx_np - 1).astype(np.int32))
    q = T.to_dev(c.q)
    scale, maxctx = float(c.scale), int(ctx_np.max())
    ws = pg.decode_workspace(B, hq, hkv, d, 0, q.device)

    def timed(kc_, vc_, table_, out):
        def step(ev=None):
            pg.paged_kv_write(k_new, v_new, cu_new, sp_new, table_, kc_, vc_)
            if ev is not None:
                ev[0].record()
            pg.gqa_paged_decode(q, kc_, vc_, table_, ctx, maxctx, scale=scale, out=out, workspace=ws)
            if ev is not None:
                ev[1].record()
        for _ in range(max(5, args.warmup // 2)):
            step()
        torch.cuda.synchronize()
        n = max(20, args.steps // 2)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        t0 = time.perf_counter()
        for i in range(n):
            step(evs[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return np.array([a.elapsed_time(b) for a, b in evs]), wall * 1e3 / n

    out_sh = torch.empty_like(q)
    ms_sh, step_sh = timed(kc, vc, table, out_sh)
    u = c.logical(np.random.default_rng(c.seed))
    ukc = T.nan_pool_dev(u.num_blocks, hkv, bs, d, c.dtype)
    uvc = T.nan_pool_dev(u.num_blocks, hkv, bs, d, c.dtype)
    utable = T.to_dev(u.block_table)
    pg.paged_kv_write(T.to_dev(u.k), T.to_dev(u.v), T.to_dev(u.cu_ctx), T.to_dev(u.start_pos), utable, ukc, uvc)
    out_un = torch.empty_like(q)
    ms_un, _ = timed(ukc, uvc, utable, out_un)
    same = bool(torch.equal(out_sh.view(torch.int16), out_un.view(torch.int16)))
    logical, unique = c.logical_kv_bytes(), c.unique_kv_bytes()
    us = float(ms_sh.mean() * 1e3)
    hbm = unique / (us * 1e-6) / 1e9
    return {
        "workload": "shared_prefix_decode", "batch": B, "prompt_len": P, "logical_kv_bytes": logical,
        "unique_kv_bytes": unique, "blocks_used": blocks_used, "blocks_unshared": int((u.block_table >= 0).sum()), "cow_copies": len(cps),
        "decode_us_mean": us, "unshared_decode_us_mean": float(ms_un.mean() * 1e3), "ms_per_step": step_sh,
        "logical_kv_gbs": logical / (us * 1e-6) / 1e9, "speedup_vs_unshared": float(ms_un.mean() / ms_sh.mean()),
        "bit_identical_to_unshared": same,
        "roofline": {"bound": "hbm", "achieved": hbm, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": hbm / HBM_PEAK_GBS, "traffic": None,
                     "bytes": "unique K/V bytes (prompt once + continuations), the HBM floor"},
    }


def window_leg(args, torch, pg, W, T, window=4096):
    """Local-attention decode on the long-context workload (B = 8, ctx 32768,
    Hq 64, Hkv 8): each sequence attends to its newest `window` positions only,
    so the pages before the window are never read.  Bytes = the K/V inside the
    windows; the full-attention call on the same pools is timed for comparison."""
    case = W.make_workload("long_ctx_decode")
    B, hq, hkv, d, bs = case.batch, case.num_q_heads, case.num_kv_heads, case.head_dim, case.block_size
    table, ctx = T.to_dev(case.block_table), T.to_dev(case.context_lens)
    kc = T.nan_pool_dev(case.num_blocks, hkv, bs, d, case.dtype)
    vc = T.nan_pool_dev(case.num_blocks, hkv, bs, d, case.dtype)
    pg.paged_kv_write(T.to_dev(case.k), T.to_dev(case.v), T.to_dev(case.cu_ctx), T.to_dev(case.start_pos), table,
                      kc, vc)
    q, out = T.to_dev(case.q), None
    out = torch.empty_like(q)
    ws = pg.decode_workspace(B, hq, hkv, d, 0, q.device)
    scale, maxctx = float(case.scale), case.max_context_len

    def run(win):
        f = lambda: pg.gqa_paged_decode(q, kc, vc, table, ctx, maxctx, scale=scale, out=out, workspace=ws,
                                        window=win)
        for _ in range(5):
            f()
        torch.cuda.synchronize()
        n = max(20, args.steps // 2)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i in range(n):
            evs[i][0].record()
            f()
            evs[i][1].record()
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs]) * 1e3)

    us_w, us_full = run(window), run(0)
    row = hkv * d * 2 * 2
    kv_w = int(np.minimum(case.context_lens, window).astype(np.int64).sum()) * row
    gbs = kv_w / (us_w * 1e-6) / 1e9
    return {
        "workload": "long_ctx_decode", "window": window, "kv_bytes_in_window": kv_w, "decode_us_mean": us_w,
        "full_attention_us_mean": us_full, "full_attention_kv_gbs": case.kv_bytes() / (us_full * 1e-6) / 1e9,
        "kv_gbs": gbs,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": None},
    }


def fp8_leg(args, torch, pg, W, T):
    """Decode of the headline workload over FP8 pages (codes + one fp32 scale per
    token and KV head), written by the quantising paged write.  Step = quantising
    write of the 64 newest tokens + FP8 decode; the decode call is event-timed.
    Bytes = codes + row scales actually stored (264 B per token and KV head for
    d 128, against 512 B in bf16); tokens/s is compared with the bf16 decode."""
    case = W.make_workload(args.decode_workload)
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

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in evs]) * 1e3)
    tokens = int(case.context_lens.astype(np.int64).sum())
    stored = tokens * hkv * 2 * (d + 4)
    gbs = stored / (us * 1e-6) / 1e9
    return {
        "workload": args.decode_workload, "kv_format": "fp8 e4m3 + fp32 row scale", "bytes_per_call": stored,
        "bf16_equivalent_bytes": case.kv_bytes(), "decode_us_mean": us, "ms_per_step": ms_step, "kv_gbs": gbs,
        "bf16_equivalent_gbs": case.kv_bytes() / (us * 1e-6) / 1e9,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": None},
    }


def mqa_leg(args, torch, pg, W, T):
    """MQA decode (B = 256, lognormal contexts, 32 query heads on one KV head,
    bs 32).  With one KV head and a group of 32 the library routes the call to
    the matrix-core multi-token kernel (the query heads form the rows of the
    32-row MFMA tile, contexts cut into key chunks merged afterwards); the VALU
    split kernel on the same pools (forced by an explicit 1,024-share split) is
    timed beside it.  Calls rotate over COPIES pools so that the K/V (~180 MB per
    copy) is not served from the last call's cache.  Bytes = the K/V read."""
    case = W.make_workload("mqa_decode")
    B, hq, hkv, d, bs = case.batch, case.num_q_heads, case.num_kv_heads, case.head_dim, case.block_size
    table, ctx = T.to_dev(case.block_table), T.to_dev(case.context_lens)
    k_all, v_all = T.to_dev(case.k), T.to_dev(case.v)
    cu_all, sp0 = T.to_dev(case.cu_ctx), T.to_dev(case.start_pos)
    pools = []
    for _ in range(COPIES):
        kc = T.nan_pool_dev(case.num_blocks, hkv, bs, d, case.dtype)
        vc = T.nan_pool_dev(case.num_blocks, hkv, bs, d, case.dtype)
        pg.paged_kv_write(k_all, v_all, cu_all, sp0, table, kc, vc)
        pools.append((kc, vc))
    del k_all, v_all
    q = T.to_dev(case.q)
    out = torch.empty_like(q)
    ws = pg.decode_workspace(B, hq, hkv, d, 0, q.device)
    scale, maxctx = float(case.scale), case.max_context_len

    def run(splits):
        def f(i):
            kc, vc = pools[i % COPIES]
            pg.gqa_paged_decode(q, kc, vc, table, ctx, maxctx, scale=scale, out=out, workspace=ws,
                                num_splits=splits)
        for i in range(5):
            f(i)
        torch.cuda.synchronize()
        n = max(20, args.steps // 2)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i in range(n):
            evs[i][0].record()
            f(i)
            evs[i][1].record()
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs]) * 1e3)

    us, us_split = run(0), run(1024)
    kvb = case.kv_bytes()
    gbs = kvb / (us * 1e-6) / 1e9
    return {
        "workload": "mqa_decode", "batch": B, "num_q_heads": hq, "num_kv_heads": hkv, "block_size": bs,
        "kv_bytes_per_call": kvb, "route": "matrix-core multi-token kernel (query heads as MFMA tile rows)",
        "decode_us_mean": us, "kv_gbs": gbs, "split_kernel_us_mean": us_split,
        "speedup_vs_split_kernel": round(us_split / us, 3),
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": None},
    }


def cpu_baseline(args, case, W):
    """The fp64 oracle, as it stands, on the same decode step (write + decode),
    repeated until at least --cpu-seconds of host time have been spent."""
    import oracle
    orc = oracle.default()
    kc = W.nan_pool(case.num_blocks, case.num_kv_heads, case.block_size, case.head_dim, case.dtype)
    vc = W.nan_pool(case.num_blocks, case.num_kv_heads, case.block_size, case.head_dim, case.dtype)
    orc.paged_kv_write(case.k, case.v, case.cu_ctx, case.start_pos, case.block_table, kc, vc)
    last = case.cu_ctx[1:] - 1
    cu_new = np.arange(case.batch + 1, dtype=np.int32)
    sp_new = (case.context_lens - 1).astype(np.int32)
    k_new, v_new = np.ascontiguousarray(case.k[last]), np.ascontiguousarray(case.v[last])
    reps, t0 = 0, time.perf_counter()
    ref = None
    while True:
        orc.paged_kv_write(k_new, v_new, cu_new, sp_new, case.block_table, kc, vc)
        ref = orc.gqa_paged_decode(case.q, kc, vc, case.block_table, case.context_lens, case.scale)
        reps += 1
        el = time.perf_counter() - t0
        if el >= args.cpu_seconds or reps >= 1000:
            break
    per_step = el / reps
    return ref, {"value": case.kv_bytes() / per_step / 1e9, "unit": "GB/s", "cores": orc.max_threads(),
                 "kind": "oracle", "seconds_per_step": per_step,
                 "sample": f"the full decode step of the same workload (paged write of the 64 newest tokens + "
                           f"fp64 decode of all 64 sequences), repeated {reps}x over {el:.1f} s"}


def main():
    args = _args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        return 2
    here = os.path.dirname(os.path.abspath(__file__))
    if args.record_traffic:
        rec = record_traffic(args.record_traffic[0], args.record_traffic[1],
                             os.path.join(here, "profiles", "traffic_counters.json"))
        print(json.dumps({k: rec[k] for k in TRAFFIC_PARTS}), flush=True)
        return 0
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
        # the counter-to-bytes scale used for the decode kernel's HBM traffic.
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "dispatches": 5}), flush=True)
        return 0

    traffic = recorded_traffic(os.path.join(here, "profiles", "traffic_counters.json"))
    dec = decode_leg(args, torch, pg, W, T)
    kv = dec["kv_bytes"]
    value = kv / (dec["ms_per_step"] * 1e-3) / 1e9
    achieved = kv / (dec["decode_ms_mean"] * 1e-3) / 1e9
    case = dec["case"]
    line = {
        "metric": ("decode KV-read GB/s (Llama-3-8B-shaped GQA decode, B=64)" if args.decode_workload == "llama3_8b_decode"
                   else f"decode KV-read GB/s ({args.decode_workload})"),
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1), bf16-rounded)",
        "config": {"workload": args.decode_workload, "batch": case.batch, "num_q_heads": case.num_q_heads,
                   "num_kv_heads": case.num_kv_heads, "head_dim": case.head_dim, "block_size": case.block_size,
                   "context_lens": W.WORKLOADS[args.decode_workload].description, "kv_bytes_per_step": kv,
                   "tokens_per_step": case.batch, "launch": "hip_graph" if args.graph else "eager"},
        "tokens_per_s": round(case.batch / (dec["ms_per_step"] * 1e-3), 1),
        "decode_call_us": {"mean": round(dec["decode_ms_mean"] * 1e3, 2),
                           "median": round(dec["decode_ms_median"] * 1e3, 2),
                           "p10": round(dec["decode_ms_p10"] * 1e3, 2), "p90": round(dec["decode_ms_p90"] * 1e3, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic["decode"],
                     "kernel": "gqa_paged_decode (split + merge kernels, one call)"},
    }
    if not args.no_prefill:
        log("prefill leg")
        line["prefill"] = prefill_leg(args, torch, pg, W, T)
        line["prefill"]["roofline"]["traffic"] = traffic["prefill"]
    if not args.no_extend:
        line["extend"] = {}
        for key in ("chunked_prefill", "spec_verify"):
            log(f"extend leg {key}")
            line["extend"][key] = extend_leg(key, args, torch, pg, W, T)
    if not args.no_fp8:
        log("fp8 pages leg")
        line["fp8"] = fp8_leg(args, torch, pg, W, T)
        line["fp8"]["speedup_vs_bf16_call"] = round(line["decode_call_us"]["mean"] / line["fp8"]["decode_us_mean"], 3)
    if not args.no_window:
        log("sliding window leg")
        line["window"] = window_leg(args, torch, pg, W, T)
    if not args.no_shared:
        log("shared prefix leg")
        line["shared_prefix"] = shared_prefix_leg(args, torch, pg, W, T)
    if not args.no_mqa:
        log("mqa decode leg")
        line["mqa"] = mqa_leg(args, torch, pg, W, T)
    if not args.no_cpu_baseline:
        log("cpu baseline leg (oracle)")
        ref, cb = cpu_baseline(args, case, W)
        line["cpu_baseline"] = cb
        got = T.to_f64(dec["out"])
        e = T.errors(got, ref)
        line["parity_vs_oracle"] = {k: float(f"{v:.3e}") for k, v in e.items()}
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
