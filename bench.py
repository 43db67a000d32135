#!/usr/bin/env python3
"""Benchmark of the MSA hot path on one MI355X.

One step = one pass of the whole decode hot path over one batch: the segment
plan (msa_plan_segments) followed by decode attention with its split-K merge
(msa_decode), on the headline decode workload (bf16, batch 32, 32 q / 8 KV
heads, head_dim 128, 4096-token contexts, block size 16, 20% of blocks evicted
in geometric runs).  Inputs are resident in HBM before the timed region.

Printed: ONE JSON line with the decode KV GB/s (value), tokens/s, % of HBM
peak, a roofline object for the dominant call (measured live with HIP events
on the launch stream), the fp64 oracle timed on the host cores
(cpu_baseline), cold-cache timing, and the chunked-prefill TFLOP/s / % of bf16
MFMA peak on the prefill workload (bf16, batch 4, chunk 512 over 8192 cached
tokens, 15% evicted).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MSA decode KV GB/s (% HBM peak) + tokens/s; prefill-chunk TFLOP/s (% MFMA)"
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA, published
COUNTERS = os.path.join(ROOT, "profiles", "decode_cfg2_counters.json")
DECODE_SOURCES = ["decode.hip", "merge.hip", "msa_internal.h"]
PF_COUNTERS = os.path.join(ROOT, "profiles", "prefill_cfg3_counters.json")
PREFILL_SOURCES = ["prefill.hip", "msa_internal.h"]


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--split-blocks", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cold", action="store_true")
    ap.add_argument("--no-gather", action="store_true",
                    help="skip the gather-then-attend baseline leg")
    ap.add_argument("--no-recompute", action="store_true",
                    help="skip the recompute (middle chunk) prefill leg")
    ap.add_argument("--latency-model", action="store_true",
                    help="fit the decode latency model used by the eviction scorer")
    ap.add_argument("--chunk-sweep", action="store_true",
                    help="also time the prefill workload at chunk sizes 128..2048")
    ap.add_argument("--more-decode", action="store_true",
                    help="also time msa_decode on the lognormal shared-prefix batch and the "
                         "131k-token fragmented batch")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (for counter calibration)")
    ap.add_argument("--no-layout", action="store_true",
                    help="skip the head-major pool layout decode leg")
    ap.add_argument("--kv-layout", choices=["nhd", "hnd"], default="nhd",
                    help="pool block layout of the headline decode leg: token-major "
                         "[P, 16, Hkv, D] (default) or head-major [P, Hkv, 16, D]")
    ap.add_argument("--only", choices=["decode", "prefill"], default=None,
                    help="time only one call (for profiler runs)")
    return ap.parse_args()


def sources_sha(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "kv_cache_attention_msa_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def alive_tokens_per_seq(w):
    """Number of alive tokens per sequence (input bookkeeping for byte counts)."""
    import numpy as np
    out = []
    for b in range(w.B):
        n = int(w.ctx_len[b])
        nb = -(-n // w.block_size)
        tok = np.minimum(w.block_size, n - w.block_size * np.arange(nb))
        out.append(int((tok * (w.alive[b, :nb] != 0)).sum()))
    return out


def unique_alive_bytes(w):
    """K+V bytes of the distinct alive pool blocks (a block shared by several
    sequences, such as a common prefix, counted once)."""
    import numpy as np
    tok = {}
    for b in range(w.B):
        n = int(w.ctx_len[b])
        nb = -(-n // w.block_size)
        for l in np.nonzero(w.alive[b, :nb])[0]:
            t = min(w.block_size, n - w.block_size * int(l))
            ph = int(w.block_table[b, l])
            tok[ph] = max(tok.get(ph, 0), t)
    return sum(tok.values()) * w.Hkv * w.D * (2 if w.dtype == "bf16" else 4) * 2


def visible_pairs(w, rows=None):
    """(query row, key) pairs with key position <= row position, over alive
    keys (all chunk rows, or only the given row indices)."""
    import numpy as np
    rows = np.arange(w.C) if rows is None else np.asarray(rows)
    tot = 0
    for b in range(w.B):
        n = int(w.ctx_len[b])
        pos = np.arange(n)
        keep = w.alive[b, pos // w.block_size] != 0
        kpos = pos[keep]
        qpos = int(w.q_pos0[b]) + rows
        tot += int(np.searchsorted(kpos, qpos, side="right").sum())
    return tot


class Prepared:
    """Device buffers and pre-marshalled C-ABI arguments for one workload, so
    the timed loops make the library calls with no allocation and no
    per-call argument building."""

    def __init__(self, w, split_blocks=0, kv_layout=0):
        import ctypes
        import torch
        from kv_cache_attention_msa_amd import _lib
        from workloads.device import to_device
        self.lib = _lib.load()
        self.w = w
        d = to_device(w, "cuda")
        if kv_layout == _lib.MSA_LAYOUT_HND:
            # the same values in head-major blocks [P, Hkv, 16, D]
            d["k_pool"] = d["k_pool"].permute(0, 2, 1, 3).contiguous()
            d["v_pool"] = d["v_pool"].permute(0, 2, 1, 3).contiguous()
        self.d = d
        dev = d["q"].device
        B, mb = w.block_table.shape
        self.cap = B * mb
        self.segs = torch.empty((self.cap, 6), dtype=torch.int32, device=dev)
        self.indptr = torch.empty(B + 1, dtype=torch.int32, device=dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        self.pws = torch.empty(max(1, int(self.lib.msa_plan_workspace_size(B))), dtype=torch.uint8, device=dev)
        self.out = torch.empty_like(d["q"])
        lse_shape = (B, w.Hq) if w.kind == "decode" else (B, w.C, w.Hq)
        self.lse = torch.empty(lse_shape, dtype=torch.float32, device=dev)
        self.max_ctx = int(w.ctx_len.max())
        if w.kind == "decode":
            wsb = int(self.lib.msa_decode_workspace_size(B, w.Hq, w.Hkv, w.D, self.max_ctx, 16, split_blocks))
        else:
            wsb = int(self.lib.msa_prefill_workspace_size(B, w.C, w.Hq, w.Hkv, w.D, self.max_ctx, 16, split_blocks))
        self.ws = torch.empty(max(1, wsb), dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.current_stream()
        P = ctypes.c_void_p
        s = P(self.stream.cuda_stream)
        dt = _lib.MSA_BF16 if w.dtype == "bf16" else _lib.MSA_F32
        self.plan_args = (P(d["block_table"].data_ptr()), P(d["alive"].data_ptr()), P(d["ctx_len"].data_ptr()),
                          B, mb, w.block_size, w.num_phys_blocks, P(self.segs.data_ptr()), self.cap,
                          P(self.indptr.data_ptr()), P(self.err.data_ptr()), P(self.pws.data_ptr()),
                          self.pws.numel(), s)
        # the default token-major layout goes through msa_decode /
        # msa_prefill_chunk, any other through their *_ex forms
        lay = () if kv_layout == _lib.MSA_LAYOUT_NHD else (kv_layout,)
        if w.kind == "decode":
            self.attn = self.lib.msa_decode_ex if lay else self.lib.msa_decode
            self.attn_args = (P(d["q"].data_ptr()), P(d["k_pool"].data_ptr()), P(d["v_pool"].data_ptr()),
                              w.num_phys_blocks, w.block_size, P(self.segs.data_ptr()), P(self.indptr.data_ptr()),
                              B, w.Hq, w.Hkv, w.D, self.max_ctx, dt, float(w.scale), split_blocks,
                              P(self.out.data_ptr()), P(self.lse.data_ptr()), P(self.ws.data_ptr()),
                              self.ws.numel()) + lay + (s,)
        else:
            self.attn = self.lib.msa_prefill_chunk_ex if lay else self.lib.msa_prefill_chunk
            self.attn_args = (P(d["q"].data_ptr()), w.C, P(d["q_pos0"].data_ptr()), P(d["k_pool"].data_ptr()),
                              P(d["v_pool"].data_ptr()), w.num_phys_blocks, w.block_size,
                              P(self.segs.data_ptr()), P(self.indptr.data_ptr()), B, w.Hq, w.Hkv, w.D,
                              self.max_ctx, dt, float(w.scale), split_blocks, P(self.out.data_ptr()),
                              P(self.lse.data_ptr()), P(self.ws.data_ptr()), self.ws.numel()) + lay + (s,)

    def plan(self):
        st = self.lib.msa_plan_segments(*self.plan_args)
        if st != 0:
            raise RuntimeError(f"msa_plan_segments failed: {st}")

    def attention(self):
        st = self.attn(*self.attn_args)
        if st != 0:
            raise RuntimeError(f"attention call failed: {st}")

    def step(self):
        self.plan()
        self.attention()


class GatherBaseline:
    """The detour MSA avoids: gather the alive blocks into dense pools
    (msa_gather_alive), then the same decode kernel over one segment per
    sequence.  Pre-marshalled like Prepared; uses its plan and buffers."""

    def __init__(self, prep):
        import ctypes
        import torch
        w, d, lib = prep.w, prep.d, prep.lib
        self.lib = lib
        P = ctypes.c_void_p
        s = P(prep.stream.cuda_stream)
        bps = -(-prep.max_ctx // w.block_size)
        dev = d["q"].device
        shape = (w.B * bps, w.block_size, w.Hkv, w.D)
        self.dk = torch.empty(shape, dtype=d["k_pool"].dtype, device=dev)
        self.dv = torch.empty_like(self.dk)
        self.dsegs = torch.empty((w.B, 6), dtype=torch.int32, device=dev)
        self.dind = torch.empty(w.B + 1, dtype=torch.int32, device=dev)
        dt = 1 if w.dtype == "bf16" else 0
        self.gather_args = (P(d["k_pool"].data_ptr()), P(d["v_pool"].data_ptr()), w.num_phys_blocks,
                            w.block_size, P(prep.segs.data_ptr()), P(prep.indptr.data_ptr()), w.B,
                            w.Hkv, w.D, dt, bps, P(self.dk.data_ptr()), P(self.dv.data_ptr()),
                            P(self.dsegs.data_ptr()), P(self.dind.data_ptr()), s)
        a = list(prep.attn_args)
        a[1], a[2], a[3] = P(self.dk.data_ptr()), P(self.dv.data_ptr()), w.B * bps
        a[5], a[6] = P(self.dsegs.data_ptr()), P(self.dind.data_ptr())
        self.attn_args = tuple(a)
        self.attn = prep.attn  # msa_decode, or msa_decode_ex with the layout argument

    def gather(self):
        st = self.lib.msa_gather_alive(*self.gather_args)
        if st != 0:
            raise RuntimeError(f"msa_gather_alive failed: {st}")

    def attention(self):
        st = self.attn(*self.attn_args)
        if st != 0:
            raise RuntimeError(f"msa_decode (dense) failed: {st}")

    def step(self):
        self.gather()
        self.attention()


def time_calls(fn, n, stream):
    """Average duration of fn() over n back-to-back calls, from HIP events
    recorded on the launch stream."""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n):
        fn()
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / n * 1e-3  # seconds


def call_percentiles(fn, n, stream):
    """p10 / median / p90 of single-call durations (us), each call between
    its own pair of HIP events on the launch stream, calls back to back."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    ev[-1][1].synchronize()
    us = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
    q = lambda f: us[min(n - 1, int(round(f * (n - 1))))]
    return {"p10": round(q(0.1), 3), "p50": round(q(0.5), 3), "p90": round(q(0.9), 3), "calls": n}


def time_cold(fn, n, stream, flush):
    """Median duration of fn() when a 1 GiB read evicts L2 and the Infinity
    Cache before every call (the read is outside the events; a read leaves
    clean lines, so the call pays no write-back of the flush)."""
    import torch
    ts = []
    sink = torch.empty((), dtype=torch.float32, device=flush.device)
    for _ in range(n):
        torch.sum(flush, dim=0, out=sink)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        e1.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    return statistics.median(ts)


def realised(w, prep):
    """What the seeded draw actually produced: eviction fraction, segment
    count (from the device plan) and context lengths."""
    import numpy as np
    ctx = np.asarray(w.ctx_len)
    return {"evicted_fraction": round(float(w.meta["evicted_fraction"]), 4),
            "segments": int(prep.indptr[-1].item()),
            "ctx_len": {"min": int(ctx.min()), "median": int(np.median(ctx)), "max": int(ctx.max())}}


def warm_for(fn, seconds=0.25):
    """Run fn in bursts for a while: the first milliseconds of a burst run at
    a lower clock."""
    import torch
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()


def prefill_leg(w, n, warm):
    """Time msa_prefill_chunk (plus its merge when split) on workload w."""
    import torch
    prep = Prepared(w)
    flops = 4.0 * w.D * w.Hq * visible_pairs(w)
    prep.plan()
    for _ in range(warm):
        prep.attention()
    torch.cuda.synchronize()
    # keep the matrix cores busy for a quarter second before timing: the
    # first milliseconds of a burst run at a lower clock (about 10% slower)
    warm_for(prep.attention)
    t = time_calls(prep.attention, n, prep.stream)
    dist = call_percentiles(prep.attention, n, prep.stream)
    tfs = flops / t / 1e12
    stats = realised(w, prep)
    del prep
    G = w.Hq // w.Hkv
    # (256 query rows, KV head, sequence) work items: one workgroup each; the
    # library splits the key stream too when these do not cover the 256 CUs
    items = -(-w.C * G // 256) * w.Hkv * w.B
    return {"us_per_call": round(t * 1e6, 3), "TFLOP/s": round(tfs, 2),
            "pct_mfma_bf16_peak": round(100 * tfs / MFMA_BF16_PEAK_TFS, 2), "calls": n,
            "call_us": dist, **stats,
            "row_tile_items": items, "flops": flops}


def latency_model_leg(args):
    """Fit msa_decode time = c0 + c_tok * alive tokens + c_seg * segments over
    decode batches that vary the context length (alive tokens) and the mean
    alive-run length (segments at a given token count), then use the fitted
    model in the kernel-aware eviction scorer on the headline batch and
    check its prediction against the measured time after eviction."""
    import numpy as np
    import torch
    from workloads import make_workload
    from kv_cache_attention_msa_amd.evict import (DecodeLatencyModel, choose_evictions,
                                                  recompute_cost_us)
    pts = []
    for ctx in (2048, 4096, 8192):
        for run in (1.0, 4.0, 32.0):
            w = make_workload(2, seed=args.seed, ctx=ctx, mean_alive=run, mean_dead=max(1.0, run / 4),
                              pool_factor=2.5)
            prep = Prepared(w)
            prep.plan()
            for _ in range(5):
                prep.attention()
            torch.cuda.synchronize()
            t = time_calls(prep.attention, 30, prep.stream)
            pts.append({"ctx": ctx, "mean_alive_run": run, "alive_tokens": int(sum(alive_tokens_per_seq(w))),
                        "segments": int(prep.indptr[-1].item()), "us": round(t * 1e6, 3)})
            del prep, w
    m = DecodeLatencyModel.fit([p["alive_tokens"] for p in pts], [p["segments"] for p in pts],
                               [p["us"] for p in pts])
    pred = m.predict([p["alive_tokens"] for p in pts], [p["segments"] for p in pts])
    meas = np.array([p["us"] for p in pts])
    r2 = 1.0 - float(((meas - pred) ** 2).sum() / ((meas - meas.mean()) ** 2).sum())
    # the scorer on the headline batch: evict a further 10% of the blocks
    w = make_workload(2, seed=args.seed)
    rng = np.random.default_rng(args.seed + 7)
    hit = rng.random(w.alive.shape)
    rec = [recompute_cost_us(w.alive[b], w.ctx_len[b], 16, w.D, w.Hq, 800.0) for b in range(w.B)]
    n_ev = int(0.1 * w.alive.sum())
    al, _ = choose_evictions(w.block_table, w.alive, w.ctx_len, 16, n_ev, hit, rec, m,
                             alpha=float(np.mean([r.mean() for r in rec])), beta=1.0, gamma=1000.0,
                             batch_seqs=w.B)
    w.alive = al
    prep = Prepared(w)
    prep.plan()
    for _ in range(5):
        prep.attention()
    torch.cuda.synchronize()
    t_after = time_calls(prep.attention, 30, prep.stream)
    segs_after = int(prep.indptr[-1].item())
    tok_after = int(sum(alive_tokens_per_seq(w)))
    del prep
    return {"c0_us": round(m.c0, 3), "c_tok_us": m.c_tok, "c_seg_us": m.c_seg, "r2": round(r2, 4),
            "points": pts,
            "eviction_check": {"evicted_blocks": n_ev, "alive_tokens": tok_after, "segments": segs_after,
                               "predicted_us": round(float(m.predict(tok_after, segs_after)), 3),
                               "measured_us": round(t_after * 1e6, 3)}}


def cpu_baseline(w, bytes_per_pass, budget_s=10.0, max_reps=20):
    """The fp64 oracle, as it stands, on the same decode workload."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    reps, t0 = 0, time.perf_counter()
    while reps < max_reps:
        oracle.decode_ref(w.q, w.k_pool, w.v_pool, w.block_table, w.alive, w.ctx_len,
                          w.block_size, w.scale)
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(bytes_per_pass * reps / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"fp64 numpy oracle (decode_ref) over the full headline decode batch "
                      f"({w.B} sequences x {w.Hq} heads), {reps} passes in {dt:.1f} s; "
                      f"BLAS threads {threads}, gathering single-threaded",
            "seconds_per_pass": round(dt / reps, 4)}


def prefill_cpu_baseline(w, row_step=16, budget_s=10.0, max_reps=5):
    """The fp64 oracle, as it stands, on a row sample of the prefill workload:
    every row_step-th chunk row of every sequence and head, over all the keys
    each row sees."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    rows = np.arange(0, w.C, row_step)
    flops = 4.0 * w.D * w.Hq * visible_pairs(w, rows)
    reps, t0 = 0, time.perf_counter()
    while reps < max_reps:
        oracle.prefill_ref(w.q, w.q_pos0, w.k_pool, w.v_pool, w.block_table, w.alive, w.ctx_len,
                           w.block_size, w.scale, rows=rows)
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(flops * reps / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"fp64 numpy oracle (prefill_ref) on every {row_step}th chunk row "
                      f"({len(rows)} of {w.C}) of all {w.B} sequences x {w.Hq} heads, visible keys "
                      f"only; {reps} passes in {dt:.1f} s; BLAS threads {threads}",
            "seconds_per_pass": round(dt / reps, 4)}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs on exactly one GPU; multi-GPU runs are not supported "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from workloads import make_workload, NAMES

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)

    result = {}
    # ---------------------------------------------------------------- decode
    if args.only in (None, "decode"):
        from kv_cache_attention_msa_amd import _lib as _l
        w = make_workload(2, seed=args.seed)
        head_major = args.kv_layout == "hnd"
        prep = Prepared(w, args.split_blocks,
                        kv_layout=_l.MSA_LAYOUT_HND if head_major else _l.MSA_LAYOUT_NHD)
        esz = 2 if w.dtype == "bf16" else 4
        alive = alive_tokens_per_seq(w)
        kv_bytes = sum(alive) * w.Hkv * w.D * 2 * esz
        qo_bytes = 2 * w.B * w.Hq * w.D * esz + w.B * w.Hq * 4
        alg_bytes = kv_bytes + qo_bytes
        stream = prep.stream
        for _ in range(args.warmup):
            prep.step()
        torch.cuda.synchronize()
        err = int(prep.err.item())
        nseg = int(prep.indptr[-1].item())
        if err != 0:
            raise RuntimeError(f"plan reported device error {err}")
        # contract timing: K whole steps bracketed by synchronize
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            prep.step()
        torch.cuda.synchronize()
        step_s = (time.perf_counter() - t0) / args.steps
        # dominant call: msa_decode (decode kernel + its split merge), HIP events
        dec_s = time_calls(prep.attention, args.steps, stream)
        dec_dist = call_percentiles(prep.attention, args.steps, stream)
        out_nhd = prep.out.clone()
        plan_s = time_calls(prep.plan, args.steps, stream)
        value = alg_bytes / step_s / 1e9
        achieved = alg_bytes / dec_s / 1e9
        traffic = None
        if os.path.exists(COUNTERS):
            c = json.load(open(COUNTERS))
            if (c.get("sources_sha") == sources_sha(DECODE_SOURCES) and c.get("split_blocks", 0) == args.split_blocks
                    and c.get("kv_layout", "nhd") == args.kv_layout):
                traffic = c.get("bytes_per_call")
        result.update({
            "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": NAMES[2], "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
                       "head_dim": w.D, "ctx_len": int(w.ctx_len[0]), "block_size": w.block_size,
                       "evicted_fraction": round(w.meta["evicted_fraction"], 4),
                       "alive_tokens": int(sum(alive)), "segments": nseg,
                       "kv_layout": "[P, Hkv, 16, D]" if head_major else "[P, 16, Hkv, D]",
                       "step": "msa_plan_segments + msa_decode (decode kernel + split-K merge)",
                       "seed": args.seed, "parallelism": "single GPU"},
            "tokens_per_s": round(w.B / step_s, 1),
            "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
            "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": traffic, "traffic_unit": "bytes per call",
                         "kernel": "msa_decode (decode kernel, plus the split merge when a sequence has several splits)",
                         "algorithmic_bytes_per_call": int(alg_bytes),
                         "us_per_call": round(dec_s * 1e6, 3)},
            "plan_us_per_call": round(plan_s * 1e6, 3),
            "decode_tokens_per_s": round(w.B / dec_s, 1),
            "decode_call_us": dec_dist,
        })
        if not args.no_cold:
            flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
            cold_s = time_cold(prep.attention, 30, stream, flush)
            del flush
            result["cold"] = {"us_per_call": round(cold_s * 1e6, 3),
                              "GB/s": round(alg_bytes / cold_s / 1e9, 2),
                              "pct_hbm_peak": round(100 * alg_bytes / cold_s / 1e9 / HBM_PEAK_GBS, 2),
                              "note": "msa_decode alone, a 1 GiB read evicts L2 and Infinity Cache before each call"}
        if not args.no_gather:
            # the gather-then-attend detour on the same inputs, same kernel
            gb = GatherBaseline(prep)
            for _ in range(3):
                gb.step()
            torch.cuda.synchronize()
            g_step = time_calls(gb.step, max(20, args.steps // 4), stream)
            g_copy = time_calls(gb.gather, max(20, args.steps // 4), stream)
            g_attn = time_calls(gb.attention, max(20, args.steps // 4), stream)
            result["gather_baseline"] = {
                "us_per_call": round(g_step * 1e6, 3), "gather_us": round(g_copy * 1e6, 3),
                "dense_decode_us": round(g_attn * 1e6, 3), "msa_decode_us": round(dec_s * 1e6, 3),
                "msa_speedup": round(g_step / dec_s, 3),
                "note": "gather alive K/V blocks into dense pools (msa_gather_alive) + msa_decode "
                        "over one segment per sequence, vs msa_decode over the segments"}
            del gb
            torch.cuda.empty_cache()
        if not args.no_cpu_baseline:
            result["cpu_baseline"] = cpu_baseline(w, alg_bytes)
        del prep
        torch.cuda.empty_cache()
        if not args.no_layout and not head_major:
            # the same batch with head-major pool blocks (msa_decode_ex)
            hp = Prepared(w, args.split_blocks, kv_layout=_l.MSA_LAYOUT_HND)
            hp.plan()
            warm_for(hp.attention, 0.1)
            torch.cuda.synchronize()
            same = bool(torch.equal(hp.out, out_nhd))
            hnd_s = time_calls(hp.attention, args.steps, stream)
            result["decode_hnd"] = {
                "us_per_call": round(hnd_s * 1e6, 3), "GB/s": round(alg_bytes / hnd_s / 1e9, 2),
                "pct_hbm_peak": round(100 * alg_bytes / hnd_s / 1e9 / HBM_PEAK_GBS, 2),
                "bitwise_equal_to_nhd": same,
                "note": "msa_decode_ex on the same batch with head-major pool blocks [P, Hkv, 16, D] "
                        "(each KV head's 16 rows of a block contiguous)"}
            del hp
            torch.cuda.empty_cache()

    # ------------------------------------------- decode latency model (next)
    if args.latency_model:
        result["latency_model"] = latency_model_leg(args)

    # ------------------------- decode on the other two decode families
    if args.more_decode and args.only in (None, "decode"):
        legs = []
        for fam in (4, 5):
            from kv_cache_attention_msa_amd import _lib as _l
            wf = make_workload(fam, seed=args.seed)
            prep = Prepared(wf, args.split_blocks, kv_layout=_l.MSA_LAYOUT_HND if args.kv_layout == "hnd"
                            else _l.MSA_LAYOUT_NHD)
            prep.plan()
            warm_for(prep.attention)
            t = time_calls(prep.attention, max(10, args.steps // 10), prep.stream)
            logical = sum(alive_tokens_per_seq(wf)) * wf.Hkv * wf.D * (2 if wf.dtype == "bf16" else 4) * 2
            unique = unique_alive_bytes(wf)
            legs.append({"workload": NAMES[fam], "us_per_call": round(t * 1e6, 3),
                         "logical_bytes": logical, "unique_bytes": unique,
                         "GB/s_logical": round(logical / t / 1e9, 1),
                         "GB/s_unique": round(unique / t / 1e9, 1),
                         "pct_hbm_peak_unique": round(100 * unique / t / 1e9 / HBM_PEAK_GBS, 2),
                         "tokens_per_s": round(wf.B / t, 1), "kv_layout": args.kv_layout,
                         **realised(wf, prep)})
            del prep, wf
            torch.cuda.empty_cache()
        result["more_decode"] = legs

    # --------------------------------------------------------------- prefill
    import kv_cache_attention_msa_amd as msa
    if args.only in (None, "prefill") and not args.no_prefill and msa.prefill_available():
        n = max(10, args.steps // 4)
        wp = make_workload(3, seed=args.seed)
        leg = prefill_leg(wp, n, max(3, args.warmup // 4))
        tfs = leg["TFLOP/s"]
        pf_traffic = None
        if os.path.exists(PF_COUNTERS):
            c = json.load(open(PF_COUNTERS))
            if c.get("sources_sha") == sources_sha(PREFILL_SOURCES):
                pf_traffic = c.get("bytes_per_call")
        leg["roofline"] = {"bound": "mfma", "achieved": tfs, "peak": MFMA_BF16_PEAK_TFS,
                           "unit": "TFLOP/s", "frac": round(tfs / MFMA_BF16_PEAK_TFS, 4),
                           "traffic": pf_traffic, "traffic_unit": "bytes per call",
                           "kernel": "msa_prefill_chunk",
                           "algorithmic_flops_per_call": leg.pop("flops")}
        if not args.no_cpu_baseline:
            leg["cpu_baseline"] = prefill_cpu_baseline(wp)
        result["prefill"] = {"workload": NAMES[3], **leg}
        del wp
        # recompute of an evicted middle range (chunk rows in the middle of the
        # context, later alive blocks hidden by the causal mask)
        if not args.no_recompute:
            wr = make_workload(6, seed=args.seed)
            leg = prefill_leg(wr, n, 3)
            leg.pop("flops")
            result["recompute"] = {"workload": NAMES[6], **leg}
            del wr
        if args.chunk_sweep:
            sweep = []
            for C in (128, 256, 512, 1024, 2048):
                wc = make_workload(3, seed=args.seed, C=C)
                leg = prefill_leg(wc, n, 3)
                leg.pop("flops")
                sweep.append({"C": C, **leg})
                del wc
            result["chunk_sweep"] = {"workload": NAMES[3] + " with chunk C varied", "points": sweep}
    if args.copy_calibration:
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        bb = torch.empty_like(a)
        for _ in range(5):
            bb.copy_(a)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = 256 << 20
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
