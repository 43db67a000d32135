#!/usr/bin/env python3
"""Benchmark of the MSA hot path on one MI355X.

One step = one pass of the whole decode hot path over one batch: the segment
plan (msa_plan_segments) followed by decode attention with its split-K merge
(msa_decode), on the headline decode workload (bf16, batch 32, 32 q / 8 KV
heads, head_dim 128, 4096-token contexts, block size 16, 20% of blocks evicted
in geometric runs).  Inputs are resident in HBM before the timed region.

Timing is cold by default: before every timed step or call a 512 MiB read
evicts L2 and the 256 MB Infinity Cache, so each call streams its K/V from
HBM, as it does in a model where other layers run between two attention
calls; the flush's own time is taken off (see cold_times).  Back-to-back
(warm) figures are reported beside the cold ones.  GPU times come from HIP
events (created without the system-scope fence) on the launch stream.

Printed: ONE JSON line with the decode KV GB/s (value, cold), tokens/s, % of
HBM peak, a roofline object for the dominant call, the fp64 oracle timed on
the host cores (cpu_baseline), and legs for the other workloads: the small
fp32 decode batch, the lognormal shared-prefix batch and the 131k-token
fragmented batch (each with roofline and oracle baseline), the chunked
prefill (TFLOP/s, % of the bf16 MFMA peak) and the recompute chunk, the
gather-then-attend detour, head-major pool blocks, the vector against the
matrix-core decode kernel, kernel-aware against hit-only eviction, and the
chunk-size curve with the adaptive chooser's pick.

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
COUNTERS4 = os.path.join(ROOT, "profiles", "decode_lognormal_counters.json")
COUNTERS5 = os.path.join(ROOT, "profiles", "decode_131k_counters.json")
PREFILL_SOURCES = ["prefill.hip", "msa_internal.h"]
FLUSH_BYTES = 512 << 20  # twice the Infinity Cache (256 MB), far above L2

ONLY = ("decode", "decode-warm", "decode4", "decode5", "prefill", "kernels", "choice", "peaks")
# (batch, context tokens) of the kernel-choice sweep: 128k tokens in all from
# batch 4 up, 32k and 64k below
CHOICE_POINTS = ((1, 32768), (2, 32768), (4, 32768), (8, 16384), (16, 8192), (32, 4096), (64, 2048),
                 (128, 1024), (256, 512), (512, 256))


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--split-blocks", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-gather", action="store_true",
                    help="skip the gather-then-attend baseline leg")
    ap.add_argument("--no-recompute", action="store_true",
                    help="skip the recompute (middle chunk) prefill leg")
    ap.add_argument("--no-more-decode", action="store_true",
                    help="skip the small fp32, lognormal and 131k-token decode legs")
    ap.add_argument("--no-kernels", action="store_true",
                    help="skip the vector against matrix-core decode kernel leg")
    ap.add_argument("--no-eviction", action="store_true",
                    help="skip the kernel-aware against hit-only eviction leg")
    ap.add_argument("--no-box-peaks", action="store_true",
                    help="skip re-measuring the HBM and bf16 matrix-core ceilings on the box")
    ap.add_argument("--no-chunk-sweep", action="store_true",
                    help="skip the prefill chunk-size curve")
    ap.add_argument("--no-layout", action="store_true",
                    help="skip the head-major pool layout decode leg")
    ap.add_argument("--latency-model", action="store_true",
                    help="also fit the decode latency model over new batches of varied context "
                         "length and alive-run length")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (for counter calibration)")
    ap.add_argument("--kv-layout", choices=["nhd", "hnd"], default="nhd",
                    help="pool block layout of the headline decode leg: token-major "
                         "[P, 16, Hkv, D] (default) or head-major [P, Hkv, 16, D]")
    ap.add_argument("--choice-points", default=None,
                    help="with --only choice: comma-separated BxCTX points (default: the built-in sweep)")
    ap.add_argument("--only", choices=ONLY, default=None,
                    help="time only one call, cold (decode, decode4, decode5, prefill, kernels) "
                         "or back to back (decode-warm), for profiler runs; choice: the automatic "
                         "decode-kernel choice against each kernel over batch sizes; peaks: the "
                         "re-measured HBM and matrix-core denominators")
    return ap.parse_args(argv)


def sources_sha(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "kv_cache_attention_msa_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# --------------------------------------------------------------------------
# algorithmic work (host bookkeeping over the generated inputs)
# --------------------------------------------------------------------------

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


def esize(w):
    return 2 if w.dtype == "bf16" else 4


def decode_bytes(w, seqs=None):
    """Algorithmic bytes of one decode call: the alive K and V rows of every
    sequence (a shared block counted once per sequence that reads it) plus Q,
    O and LSE.  seqs restricts the count to a subset of sequences."""
    per = alive_tokens_per_seq(w)
    sel = range(w.B) if seqs is None else seqs
    kv = sum(per[b] for b in sel) * w.Hkv * w.D * 2 * esize(w)
    qo = len(list(sel)) * w.Hq * (2 * w.D * esize(w) + 4)
    return kv + qo


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
    return sum(tok.values()) * w.Hkv * w.D * esize(w) * 2


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


# --------------------------------------------------------------------------
# pre-marshalled library calls
# --------------------------------------------------------------------------

class Prepared:
    """Device buffers and pre-marshalled C-ABI arguments for one workload, so
    the timed loops make the library calls with no allocation and no
    per-call argument building.  The attention call ORs its truncation bit
    into the plan's error word."""

    def __init__(self, w, split_blocks=0, kv_layout=0, kernel=0, d=None):
        import ctypes
        import torch
        from kv_cache_attention_msa_amd import _lib
        from workloads.device import to_device
        self.lib = _lib.load()
        self.w = w
        if d is None:
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
        errp = P(self.err.data_ptr())
        if w.kind == "decode":
            self.attn = self.lib.msa_decode_ex
            self.attn_args = (P(d["q"].data_ptr()), P(d["k_pool"].data_ptr()), P(d["v_pool"].data_ptr()),
                              w.num_phys_blocks, w.block_size, P(self.segs.data_ptr()), P(self.indptr.data_ptr()),
                              B, w.Hq, w.Hkv, w.D, self.max_ctx, dt, float(w.scale), split_blocks,
                              P(self.out.data_ptr()), P(self.lse.data_ptr()), P(self.ws.data_ptr()),
                              self.ws.numel(), kv_layout, kernel, errp, s)
        else:
            self.attn = self.lib.msa_prefill_chunk_ex
            self.attn_args = (P(d["q"].data_ptr()), w.C, P(d["q_pos0"].data_ptr()), P(d["k_pool"].data_ptr()),
                              P(d["v_pool"].data_ptr()), w.num_phys_blocks, w.block_size,
                              P(self.segs.data_ptr()), P(self.indptr.data_ptr()), B, w.Hq, w.Hkv, w.D,
                              self.max_ctx, dt, float(w.scale), split_blocks, P(self.out.data_ptr()),
                              P(self.lse.data_ptr()), P(self.ws.data_ptr()), self.ws.numel(), kv_layout,
                              errp, s)

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

    def check_error(self):
        import torch
        torch.cuda.synchronize()
        e = int(self.err.item())
        if e != 0:
            raise RuntimeError(f"device error word {e}")


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
        shape = (w.B * bps,) + tuple(d["k_pool"].shape[1:])
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
        self.attn = prep.attn

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


# --------------------------------------------------------------------------
# timing
# --------------------------------------------------------------------------

HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence (hip_runtime_api.h)


class HipEvent:
    """A HIP timing event created with hipEventDisableSystemFence.  A default
    event record performs a system-scope fence (cache write-back and
    invalidation) that leaves the GPU idle for about 6 us before the next
    dispatch, which a single-kernel interval would include; timing events
    need no such fence (elapsed times are read after a stream
    synchronize)."""
    _hip = None

    def __init__(self):
        import ctypes
        if HipEvent._hip is None:
            hip = ctypes.CDLL("libamdhip64.so")
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            HipEvent._hip = hip
        self.ev = ctypes.c_void_p()
        st = HipEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.ev), HIP_EVENT_DISABLE_SYSTEM_FENCE)
        if st != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {st}")

    def record(self, stream):
        import ctypes
        st = HipEvent._hip.hipEventRecord(self.ev, ctypes.c_void_p(stream.cuda_stream))
        if st != 0:
            raise RuntimeError(f"hipEventRecord failed: {st}")

    def elapsed_s(self, end):
        """Seconds from this event to `end`; the stream must have been
        synchronized after both were recorded."""
        import ctypes
        ms = ctypes.c_float()
        st = HipEvent._hip.hipEventElapsedTime(ctypes.byref(ms), self.ev, end.ev)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {st}")
        return ms.value * 1e-3

    def __del__(self):
        if HipEvent._hip is not None and self.ev:
            HipEvent._hip.hipEventDestroy(self.ev)


def time_calls(fn, n, stream):
    """Average duration (s) of fn() over n back-to-back (warm) calls, from HIP
    events recorded on the launch stream."""
    e0, e1 = HipEvent(), HipEvent()
    e0.record(stream)
    for _ in range(n):
        fn()
    e1.record(stream)
    stream.synchronize()
    return e0.elapsed_s(e1) / n


class Flush:
    """A 512 MiB read that evicts L2 and the Infinity Cache (a 1 GiB read gives
    the same cold times).  A read leaves clean lines, so the timed call
    after it pays no write-back."""

    def __init__(self):
        import torch
        self.buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        self.sink = torch.empty((), dtype=torch.float32, device="cuda")

    def __call__(self):
        import torch
        torch.sum(self.buf, dim=0, out=self.sink)


def cold_times(fn, n, stream, flush):
    """Durations (s) of n cold calls of fn(): the HIP events bracket [flush,
    fn()] and, interleaved with it (order alternating), [flush] alone, and the
    mean flush time is taken off each bracketed pair.  An event record
    directly before a dispatch leaves the GPU idle for about 4.5 us (against
    about 1 us between back-to-back kernels), so a bracket around fn() alone
    would overstate a short call; here that cost sits in both brackets and
    cancels, while the ordinary kernel-to-kernel transition after the flush
    stays in, as it would after any kernel of a model."""
    ts = []
    ev = [HipEvent() for _ in range(4)]
    for i in range(n):
        for first in ((True, False) if i % 2 == 0 else (False, True)):
            a, b = (ev[0], ev[1]) if first else (ev[2], ev[3])
            a.record(stream)
            flush()
            if first:
                fn()
            b.record(stream)
        stream.synchronize()
        # the two brackets of one pair ran back to back: their difference
        ts.append(ev[0].elapsed_s(ev[1]) - ev[2].elapsed_s(ev[3]))
    return ts


def tmean(ts, cut=0.1):
    """Mean of ts without its lowest and highest `cut` fraction (a stray
    host or clock hiccup in one pair of brackets does not move it)."""
    s = sorted(ts)
    k = int(len(s) * cut)
    return statistics.fmean(s[k:len(s) - k] if len(s) > 2 * k else s)


def cold_times_direct(fn, n, stream, flush):
    """Durations (s) of n calls of fn(), each after a flush, each timed by a
    pair of HIP events directly around it (includes the event-to-dispatch
    idle gap; reported beside cold_times for reference)."""
    ts = []
    e0, e1 = HipEvent(), HipEvent()
    for _ in range(n):
        flush()
        e0.record(stream)
        fn()
        e1.record(stream)
        stream.synchronize()
        ts.append(e0.elapsed_s(e1))
    return ts


def dist_us(ts):
    s = sorted(ts)
    n = len(s)
    q = lambda f: s[min(n - 1, int(round(f * (n - 1))))] * 1e6
    return {"mean": round(tmean(s) * 1e6, 3), "p10": round(q(0.1), 3),
            "p50": round(q(0.5), 3), "p90": round(q(0.9), 3), "calls": n}


def warm_for(fn, seconds=0.25):
    """Run fn in bursts for a while: the first milliseconds of a burst run at
    a lower clock."""
    import torch
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()


def realised(w, prep):
    """What the seeded draw actually produced: eviction fraction, segment
    count (from the device plan) and context lengths."""
    import numpy as np
    ctx = np.asarray(w.ctx_len)
    return {"evicted_fraction": round(float(w.meta.get("evicted_fraction", 0.0)), 4),
            "segments": int(prep.indptr[-1].item()),
            "ctx_len": {"min": int(ctx.min()), "median": int(np.median(ctx)), "max": int(ctx.max())}}


def counter_traffic(path, names, **want):
    """HBM bytes per call from a committed counter summary, if it was taken on
    the current kernel sources and the same launch configuration."""
    if not os.path.exists(path):
        return None
    c = json.load(open(path))
    if c.get("sources_sha") != sources_sha(names):
        return None
    for k, v in want.items():
        if c.get(k, {"split_blocks": 0, "kv_layout": "nhd"}.get(k)) != v:
            return None
    return c.get("bytes_per_call")


# --------------------------------------------------------------------------
# the oracle on the host cores (CPU baseline)
# --------------------------------------------------------------------------

def host_cores():
    return len(os.sched_getaffinity(0))


def _oracle_rate(fn, work, budget_s, max_reps, threads):
    """Run fn() (one oracle pass over `work` units) repeatedly for about
    budget_s with the BLAS pool limited to `threads`; returns (units/s,
    passes, seconds, threads the BLAS pool reported)."""
    from threadpoolctl import threadpool_info, threadpool_limits
    with threadpool_limits(limits=threads):
        used = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        reps, t0 = 0, time.perf_counter()
        while reps < max_reps:
            fn()
            reps += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = time.perf_counter() - t0
    return work * reps / dt, reps, dt, used


def oracle_baseline(fn, work, unit, scale, sample, budget_s=6.0, max_reps=20, single=True,
                    single_budget_s=3.0):
    """CPU-baseline record: the fp64 oracle as it stands, on every core of
    this process's affinity mask, and (single=True) on one thread."""
    cores = host_cores()
    rate, reps, dt, used = _oracle_rate(fn, work, budget_s, max_reps, cores)
    rec = {"value": round(rate / scale, 6), "unit": unit, "cores": used, "kind": "oracle",
           "sample": f"{sample}; {reps} passes in {dt:.1f} s, BLAS threads {used} of {cores} host "
                     f"cores (the gather loops are single-threaded)",
           "seconds_per_pass": round(dt / reps, 4), "host_cores": cores}
    if single:
        r1, reps1, dt1, _ = _oracle_rate(fn, work, single_budget_s, max_reps, 1)
        rec["single_thread"] = {"value": round(r1 / scale, 6), "unit": unit, "cores": 1,
                                "seconds_per_pass": round(dt1 / reps1, 4), "passes": reps1}
    return rec


def decode_cpu_baseline(w, seqs=None, budget_s=6.0, single=True, label="", max_reps=20):
    """The oracle's decode (decode_ref) on the whole batch or on the given
    sequences (all heads), as GB/s of algorithmic bytes."""
    import oracle
    work = decode_bytes(w, seqs)
    which = "all sequences" if seqs is None else f"sequences {list(seqs)}"
    fn = lambda: oracle.decode_ref(w.q, w.k_pool, w.v_pool, w.block_table, w.alive, w.ctx_len,
                                   w.block_size, w.scale, seqs=seqs)
    return oracle_baseline(fn, work, "GB/s", 1e9,
                           f"fp64 numpy oracle (decode_ref) on {label} {which} x {w.Hq} heads "
                           f"({work / 1e6:.1f} MB of alive K/V + Q/O)", budget_s=budget_s,
                           max_reps=max_reps, single=single)


def prefill_cpu_baseline(w, row_step=16, budget_s=6.0, max_reps=5, single=True):
    """The oracle's prefill (prefill_ref) on a row sample of the chunk: every
    row_step-th chunk row of every sequence and head, over all the keys each
    row sees."""
    import numpy as np
    import oracle
    rows = np.arange(0, w.C, row_step)
    flops = 4.0 * w.D * w.Hq * visible_pairs(w, rows)
    fn = lambda: oracle.prefill_ref(w.q, w.q_pos0, w.k_pool, w.v_pool, w.block_table, w.alive,
                                    w.ctx_len, w.block_size, w.scale, rows=rows)
    return oracle_baseline(fn, flops, "TFLOP/s", 1e12,
                           f"fp64 numpy oracle (prefill_ref) on every {row_step}th chunk row "
                           f"({len(rows)} of {w.C}) of all {w.B} sequences x {w.Hq} heads, visible "
                           f"keys only", budget_s=budget_s, max_reps=max_reps, single=single)


# --------------------------------------------------------------------------
# legs
# --------------------------------------------------------------------------

def decode_roofline(alg_bytes, cold_mean_s, warm_s, traffic=None, kernel="msa_decode"):
    a = alg_bytes / cold_mean_s / 1e9
    return {"bound": "hbm", "achieved": round(a, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(a / HBM_PEAK_GBS, 4), "traffic": traffic, "traffic_unit": "bytes per call",
            "kernel": kernel,
            "timing": "cold: HIP events (no system fence) around [512 MiB read flush + call] minus the "
                      "same around [flush] alone, pairs interleaved; 10%-trimmed mean over the calls",
            "algorithmic_bytes_per_call": int(alg_bytes), "us_per_call": round(cold_mean_s * 1e6, 3),
            "warm": {"achieved": round(alg_bytes / warm_s / 1e9, 2),
                     "frac": round(alg_bytes / warm_s / 1e9 / HBM_PEAK_GBS, 4),
                     "us_per_call": round(warm_s * 1e6, 3)}}


def decode_leg(w, n, flush, split_blocks=0, kv_layout=0, kernel=0, unique=False, d=None):
    """Cold and warm msa_decode on workload w, with its roofline (on the
    distinct alive bytes too when unique=True)."""
    import torch
    prep = Prepared(w, split_blocks, kv_layout=kv_layout, kernel=kernel, d=d)
    prep.plan()
    prep.attention()
    prep.check_error()
    warm_for(prep.attention, 0.1)
    cold = cold_times(prep.attention, n, prep.stream, flush)
    warm_s = time_calls(prep.attention, n, prep.stream)
    alg = decode_bytes(w)
    cold_mean = tmean(cold)
    leg = {"us_per_call": round(cold_mean * 1e6, 3), "cold_us": dist_us(cold),
           "warm_us_per_call": round(warm_s * 1e6, 3),
           "GB/s": round(alg / cold_mean / 1e9, 2), "pct_hbm_peak": round(100 * alg / cold_mean / 8e12, 2),
           "tokens_per_s": round(w.B / cold_mean, 1),
           "roofline": decode_roofline(alg, cold_mean, warm_s), **realised(w, prep)}
    if unique:
        ub = unique_alive_bytes(w) + w.B * w.Hq * (2 * w.D * esize(w) + 4)
        leg["roofline"]["logical_bytes_per_call"] = leg["roofline"].pop("algorithmic_bytes_per_call")
        leg["roofline"]["logical_GB/s"] = leg["roofline"]["achieved"]
        leg["roofline"]["algorithmic_bytes_per_call"] = int(ub)
        leg["roofline"]["achieved"] = round(ub / cold_mean / 1e9, 2)
        leg["roofline"]["frac"] = round(ub / cold_mean / 1e9 / HBM_PEAK_GBS, 4)
        leg["roofline"]["note"] = ("algorithmic bytes = distinct alive blocks (a shared prefix counted "
                                   "once) + Q/O/LSE; logical = per sequence")
        leg["roofline"]["warm"]["frac"] = round(ub / warm_s / 1e9 / HBM_PEAK_GBS, 4)
    out = prep.out.clone()
    del prep
    torch.cuda.empty_cache()
    return leg, out


def prefill_leg(w, n, warm, flush=None):
    """Time msa_prefill_chunk (plus its merge when split) on workload w: the
    mean of back-to-back calls after a quarter second of warm-up (the rate
    of a stream of chunks), and cold single calls when flush is given."""
    import torch
    prep = Prepared(w)
    flops = 4.0 * w.D * w.Hq * visible_pairs(w)
    prep.plan()
    for _ in range(warm):
        prep.attention()
    prep.check_error()
    # keep the matrix cores busy for a quarter second before timing: the
    # first milliseconds of a burst run at a lower clock (about 10% slower)
    warm_for(prep.attention)
    t = time_calls(prep.attention, n, prep.stream)
    tfs = flops / t / 1e12
    stats = realised(w, prep)
    rec = {"us_per_call": round(t * 1e6, 3), "TFLOP/s": round(tfs, 2),
           "pct_mfma_bf16_peak": round(100 * tfs / MFMA_BF16_PEAK_TFS, 2), "calls": n, **stats}
    if flush is not None:
        cold = cold_times(prep.attention, max(5, n // 2), prep.stream, flush)
        rec["cold_us"] = dist_us(cold)
    del prep
    torch.cuda.empty_cache()
    G = w.Hq // w.Hkv
    # (256/G query positions, KV head, sequence) work items: one workgroup
    # each; the library splits the key stream too when these do not cover
    # the 256 CUs
    rec["row_tile_items"] = -(-w.C * G // 256) * w.Hkv * w.B
    rec["flops"] = flops
    return rec


def kernel_cases(args, w2, w5, w4=None):
    """Batches for the decode-kernel comparison: the headline batch as drawn
    (G 4) and with 64 query heads (G 8: 32 more rows drawn N(0,1)); the
    131k-token batch as drawn (G 8) and with its first 32 query heads (G 4);
    the lognormal shared-prefix batch (G 4) when given."""
    import copy
    import numpy as np
    from workloads import f32_to_bf16_bits
    rng = np.random.default_rng(args.seed + 30)
    w2g8 = copy.copy(w2)
    extra = f32_to_bf16_bits(rng.standard_normal((w2.B, w2.Hq, w2.D)).astype(np.float32))
    w2g8.q = np.concatenate([w2.q, extra], axis=1)
    w2g8.Hq = 2 * w2.Hq
    w5g4 = copy.copy(w5)
    w5g4.q = np.ascontiguousarray(w5.q[:, :w5.Hq // 2])
    w5g4.Hq = w5.Hq // 2
    cases = (("headline batch, G 4", w2), ("headline batch, G 8", w2g8),
             ("131k-token batch, G 8", w5), ("131k-token batch, G 4", w5g4))
    if w4 is not None:
        cases += (("lognormal shared-prefix batch, G 4", w4),)
    return cases


def kernels_leg(args, flush, w2, w5, w4=None):
    """The three decode kernels -- vector-ALU, per-KV-head matrix-core, and
    the block kernel (whole KV blocks of all heads per workgroup, shared
    prefixes streamed once per sub-group) -- on the same batches (4 and 8
    query heads per KV head): cold time and max error against the oracle on
    sampled (sequence, head) pairs."""
    import numpy as np
    import torch
    import oracle
    from kv_cache_attention_msa_amd import _lib
    from workloads.device import from_device
    rng = np.random.default_rng(args.seed + 31)
    cases = []
    for name, w in kernel_cases(args, w2, w5, w4):
        seqs = sorted(rng.choice(w.B, size=min(2, w.B), replace=False).tolist())
        heads = sorted(rng.choice(w.Hq, size=3, replace=False).tolist())
        Or, Lr = oracle.decode_ref(w.q, w.k_pool, w.v_pool, w.block_table, w.alive, w.ctx_len,
                                   w.block_size, w.scale, seqs=seqs, heads=heads)
        row = {"batch": name, "G": w.Hq // w.Hkv}
        for kname, k in (("vector", _lib.MSA_DECODE_VECTOR), ("matrix", _lib.MSA_DECODE_MATRIX),
                         ("block", _lib.MSA_DECODE_BLOCK)):
            leg, out = decode_leg(w, max(10, args.steps // 2), flush, kernel=k)
            O = from_device(out)
            sel = np.ix_(seqs, heads)
            err = float(np.max(np.abs(O[sel] - Or[sel])))
            row[kname] = {"us_per_call": leg["us_per_call"], "warm_us_per_call": leg["warm_us_per_call"],
                          "pct_hbm_peak": leg["pct_hbm_peak"], "max_abs_err_vs_oracle": err,
                          "checked": f"sequences {seqs} x heads {heads}"}
            del out
        cases.append(row)
        torch.cuda.empty_cache()
    return cases


def eviction_leg(args, flush, w):
    """Kernel-aware eviction (keep-score = hit probability + recompute cost +
    the decode time a block costs, from a latency model of msa_decode fitted
    here over alive tokens, segments and the longest sequence's alive tokens)
    against hit-only eviction, at the same number of evicted blocks, on the
    headline batch.  Only the alive mask changes, so the same device pools
    serve every point; each point re-plans and times msa_decode cold."""
    import numpy as np
    import torch
    from kv_cache_attention_msa_amd.evict import (DecodeLatencyModel, choose_evictions,
                                                  recompute_cost_us)
    from workloads.device import to_device
    base = to_device(w, "cuda")
    rng = np.random.default_rng(args.seed + 7)
    B = w.B
    nb = -(-w.ctx_len.astype(np.int64) // w.block_size)
    evictable = [(b, l) for b in range(B) for l in range(int(nb[b]) - 1) if w.alive[b, l]]

    def measure(alive):
        import copy
        wv = copy.copy(w)
        wv.alive = alive
        d = dict(base)
        d["alive"] = torch.from_numpy(np.ascontiguousarray(alive)).to("cuda")
        prep = Prepared(wv, d=d)
        prep.plan()
        prep.attention()
        prep.check_error()
        ts = cold_times(prep.attention, max(30, args.steps), prep.stream, flush)
        segs = int(prep.indptr[-1].item())
        del prep
        per = alive_tokens_per_seq(wv)
        return {"alive_tokens": int(sum(per)), "max_seq_tokens": int(max(per)), "segments": segs,
                "us": round(tmean(ts) * 1e6, 3)}

    def level(al, n, longest):
        # n more evictions, each from the sequence with the most (longest) or
        # fewest alive tokens, a random evictable block of it
        al = al.copy()
        for _ in range(n):
            per = [int(al[b, :nb[b] - 1].sum()) for b in range(B)]
            cand = [b for b in range(B) if per[b] > 0]
            b = max(cand, key=lambda x: per[x]) if longest else min(cand, key=lambda x: per[x])
            ls = np.nonzero(al[b, :nb[b] - 1])[0]
            al[b, int(rng.choice(ls))] = 0
        return al

    # fit points: extra evictions of single random blocks (more segments) and
    # of whole alive runs (fewer segments) at three fractions each
    pts = [dict(kind="as drawn", **measure(w.alive))]
    for frac in (0.1, 0.2, 0.3):
        al = w.alive.copy()
        pick = rng.choice(len(evictable), size=int(frac * len(evictable)), replace=False)
        for i in pick:
            al[evictable[i]] = 0
        pts.append(dict(kind=f"random blocks {frac:.0%}", **measure(al)))
        al = w.alive.copy()
        runs = []
        for b in range(B):
            l = 0
            while l < nb[b] - 1:
                if al[b, l]:
                    s = l
                    while l < nb[b] - 1 and al[b, l]:
                        l += 1
                    runs.append((b, s, l))
                else:
                    l += 1
        order = rng.permutation(len(runs))
        target, done = int(frac * len(evictable)), 0
        for i in order:
            b, s, e = runs[i]
            if done >= target:
                break
            al[b, s:e] = 0
            done += e - s
        pts.append(dict(kind=f"whole runs {frac:.0%}", **measure(al)))
    # the longest sequence apart from the total: blocks from the longest
    # sequences only, or from the shortest only
    for frac in (0.05, 0.1):
        k = int(frac * len(evictable))
        pts.append(dict(kind=f"longest first {frac:.0%}", **measure(level(w.alive, k, True))))
        pts.append(dict(kind=f"shortest first {frac:.0%}", **measure(level(w.alive, k, False))))
    cols = lambda key: [p[key] for p in pts]
    m = DecodeLatencyModel.fit(cols("alive_tokens"), cols("segments"), cols("us"),
                               max_seq_tokens=cols("max_seq_tokens"))
    meas = np.array([p["us"] for p in pts])
    pred = m.predict(cols("alive_tokens"), cols("segments"), cols("max_seq_tokens"))
    r2 = 1.0 - float(((meas - pred) ** 2).sum() / max(((meas - meas.mean()) ** 2).sum(), 1e-30))
    hit = rng.random(w.alive.shape)
    rec = [recompute_cost_us(w.alive[b], w.ctx_len[b], w.block_size, w.D, w.Hq, 1000.0)
           for b in range(B)]
    n_ev = int(0.1 * len(evictable))
    policies = {}
    # kernel_aware: the pages' full score (hit probability, recompute cost,
    # decode cost over 1000 steps); latency_aware: hit probability and the
    # decode cost only (1 us of decode time per step weighs as much as a hit
    # probability of 10); hit_only: hit probability alone
    rec_mean = float(np.mean([r.mean() for r in rec]))
    import copy
    preps = {}
    for name, kw in (("kernel_aware", dict(alpha=rec_mean, beta=1.0, gamma=1000.0)),
                     ("latency_aware", dict(alpha=1.0, beta=0.0, gamma=10.0 * B)),
                     ("hit_only", dict(alpha=1.0, beta=0.0, gamma=0.0))):
        al, ev = choose_evictions(w.block_table, w.alive, w.ctx_len, w.block_size, n_ev, hit, rec, m,
                                  batch_seqs=B, **kw)
        wv = copy.copy(w)
        wv.alive = al
        d = dict(base)
        d["alive"] = torch.from_numpy(np.ascontiguousarray(al)).to("cuda")
        prep = Prepared(wv, d=d)
        prep.plan()
        prep.attention()
        prep.check_error()
        per = alive_tokens_per_seq(wv)
        r = {"alive_tokens": int(sum(per)), "max_seq_tokens": int(max(per)),
             "segments": int(prep.indptr[-1].item())}
        r["predicted_us"] = round(float(m.predict(r["alive_tokens"], r["segments"],
                                                  r["max_seq_tokens"])), 3)
        r["evicted_blocks"] = len(ev)
        r["mean_hit_prob_evicted"] = round(float(np.mean([hit[b, l] for b, l in ev])), 4)
        r["recompute_us_evicted"] = round(float(sum(rec[b][l] for b, l in ev)), 1)
        policies[name] = r
        preps[name] = prep
    # the three masks timed in interleaved rounds (the order rotating), so
    # drift of the box's clock or memory state between policies cancels;
    # a policy's time is the median of its round means, a saving the median
    # of the per-round differences
    names = list(preps)
    rounds = {n: [] for n in names}
    for rd in range(8):
        for k in range(len(names)):
            n = names[(rd + k) % len(names)]
            rounds[n].append(tmean(cold_times(preps[n].attention, 15, preps[n].stream, flush)) * 1e6)
    for n in names:
        policies[n]["us"] = round(float(np.median(rounds[n])), 3)
        policies[n]["us_rounds"] = [round(x, 2) for x in rounds[n]]
    saved = lambda n: round(float(np.median(np.array(rounds["hit_only"]) - np.array(rounds[n]))), 3)
    del preps, base
    torch.cuda.empty_cache()
    return {"model": {"c0_us": round(m.c0, 3), "c_tok_us": m.c_tok, "c_seg_us": m.c_seg,
                      "c_max_us": m.c_max, "r2": round(r2, 4), "points": pts},
            "evicted_blocks": n_ev, "policies": policies,
            "decode_us_saved_by_kernel_aware": saved("kernel_aware"),
            "decode_us_saved_by_latency_aware": saved("latency_aware"),
            "timing": "each policy's mask timed cold in 8 interleaved rounds of 15 calls (10%-trimmed "
                      "mean per round); us = median over rounds; saved = median of per-round "
                      "differences against hit_only"}


def mfma_rate(st):
    """bf16 matrix-core rate with register operands only (libmsa_peaks.so):
    8192 workgroups of four wavefronts, each issuing 256 x 8 independent
    v_mfma_f32_32x32x16_bf16 -- about 1.1 ms of matrix work on 256 CUs."""
    import ctypes
    import torch
    from kv_cache_attention_msa_amd import build as _build
    lib = ctypes.CDLL(_build.PEAKS_LIB)
    fn = lib.msa_peaks_mfma_bf16
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    wgs, iters = 8192, 256
    sink = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")

    def call():
        rc = fn(wgs, iters, ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(st.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"msa_peaks_mfma_bf16 returned {rc}")

    for _ in range(3):
        call()
    best = min(time_calls(call, 5, st) for _ in range(4))
    flops = wgs * 4 * iters * 8 * 32768
    return round(flops / best / 1e12, 1)


def box_peaks_leg():
    """The roofline denominators re-measured on this GPU, for context beside
    the published peaks: a 1 GiB streaming read (torch row sums over 4096
    rows) and a 1 GiB device-to-device copy (HBM bytes per second), the
    matrix cores' bf16 rate with register operands (the instrument kernel in
    libmsa_peaks.so), and a large bf16 GEMM (torch matmul through the vendor
    BLAS) as the practical matrix-core ceiling with memory traffic.  Each is
    the best of several back-to-back runs after warm-up."""
    import torch
    st = torch.cuda.current_stream()
    n = 1 << 30
    a = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    rows = a.view(4096, -1)
    sink = torch.empty(4096, dtype=torch.float32, device="cuda")
    rd = lambda: torch.sum(rows, dim=1, out=sink)
    cp = lambda: b.copy_(a)
    res = {}
    for name, fn, nbytes in (("hbm_read_GB/s", rd, n), ("hbm_copy_GB/s", cp, 2 * n)):
        for _ in range(3):
            fn()
        best = min(time_calls(fn, 5, st) for _ in range(4))
        res[name] = round(nbytes / best / 1e9, 1)
    del a, b
    m = 8192
    x = torch.randn(m, m, dtype=torch.bfloat16, device="cuda")
    y = torch.randn(m, m, dtype=torch.bfloat16, device="cuda")
    z = torch.empty(m, m, dtype=torch.bfloat16, device="cuda")
    mm = lambda: torch.matmul(x, y, out=z)
    warm_for(mm, 0.25)
    best = min(time_calls(mm, 10, st) for _ in range(4))
    res["bf16_gemm_TFLOP/s"] = round(2 * m ** 3 / best / 1e12, 1)
    try:
        res["mfma_bf16_TFLOP/s"] = mfma_rate(st)
        res["mfma"] = "v_mfma_f32_32x32x16_bf16, register operands, every CU (libmsa_peaks.so)"
    except (OSError, RuntimeError) as e:
        res["mfma_bf16_TFLOP/s"] = None
        res["mfma"] = f"not measured: {e}"
    res["gemm"] = f"bf16 {m} x {m} x {m}, torch.matmul"
    res["published"] = {"hbm_GB/s": HBM_PEAK_GBS, "bf16_dense_TFLOP/s": MFMA_BF16_PEAK_TFS}
    del x, y, z
    torch.cuda.empty_cache()
    return res


def chunk_sweep_leg(args, flush):
    """The prefill workload with the chunk length varied (8192 cached tokens,
    batch 4, 32 / 8 heads): the chunk-size curve, and the chunk length the
    adaptive chooser (msa_prefill_chunk_rows) picks for this batch."""
    import kv_cache_attention_msa_amd as msa
    from workloads import make_workload
    n = max(10, args.steps // 2)
    pts = []
    for C in (128, 256, 512, 1024, 2048):
        wc = make_workload(3, seed=args.seed, C=C)
        leg = prefill_leg(wc, n, 3)
        leg.pop("flops")
        pts.append({"C": C, "us_per_call": leg["us_per_call"], "TFLOP/s": leg["TFLOP/s"],
                    "pct_mfma_bf16_peak": leg["pct_mfma_bf16_peak"],
                    "row_tile_items": leg["row_tile_items"],
                    "us_per_chunk_row": round(leg["us_per_call"] / C, 4)})
        del wc
    pick = msa.msa_prefill_chunk_rows(4, 32, 8, 1 << 20)
    best = max(p["TFLOP/s"] for p in pts)
    at = [p for p in pts if p["C"] == pick]
    return {"workload": "prefill workload with the chunk length C varied", "points": pts,
            "chooser": {"call": "msa_prefill_chunk_rows(B=4, Hq=32, Hkv=8, remaining=2^20)",
                        "chunk_rows": pick,
                        "TFLOP/s_at_pick": at[0]["TFLOP/s"] if at else None,
                        "fraction_of_best_point": round(at[0]["TFLOP/s"] / best, 4) if at else None}}


# --------------------------------------------------------------------------

def main(argv=None):
    args = parse(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs on exactly one GPU; multi-GPU runs are not supported "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import kv_cache_attention_msa_amd as msa
    from kv_cache_attention_msa_amd import _lib
    from workloads import make_workload, NAMES

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    flush = Flush()
    cpu = not args.no_cpu_baseline and args.only is None
    result = {}
    layout = _lib.MSA_LAYOUT_HND if args.kv_layout == "hnd" else _lib.MSA_LAYOUT_NHD

    # ------------------------------------------------------------ profiler modes
    if args.only is not None:
        n = args.steps
        if args.only in ("decode", "decode-warm"):
            w = make_workload(2, seed=args.seed)
            prep = Prepared(w, args.split_blocks, kv_layout=layout)
            for _ in range(args.warmup):
                prep.step()
            prep.check_error()
            if args.only == "decode-warm":
                result["us_per_call_warm"] = round(time_calls(prep.attention, n, prep.stream) * 1e6, 3)
            else:
                result["cold_us"] = dist_us(cold_times(prep.attention, n, prep.stream, flush))
        elif args.only == "kernels":
            # each batch with the vector kernel, the per-KV-head matrix-core
            # kernel and the block kernel
            cases = kernel_cases(args, make_workload(2, seed=args.seed), make_workload(5, seed=args.seed),
                                 make_workload(4, seed=args.seed))
            for name, w in cases:
                for kname, k in (("vector", _lib.MSA_DECODE_VECTOR), ("matrix", _lib.MSA_DECODE_MATRIX),
                                 ("block", _lib.MSA_DECODE_BLOCK)):
                    prep = Prepared(w, kernel=k)
                    for _ in range(args.warmup):
                        prep.step()
                    prep.check_error()
                    result[f"{name}, {kname}"] = dist_us(cold_times(prep.attention, n, prep.stream, flush))
                    del prep
                    torch.cuda.empty_cache()
        elif args.only == "choice":
            # the automatic decode-kernel choice against each kernel forced,
            # over batch sizes at a fixed total context (the headline recipe)
            pts = []
            points = CHOICE_POINTS if not args.choice_points else tuple(
                (int(a), int(c)) for a, c in (x.split("x") for x in args.choice_points.split(",")))
            for B, ctx in points:
                w = make_workload(2, seed=args.seed, B=B, ctx=ctx)
                d = None
                row = {"B": B, "ctx": ctx}
                for kname, k in (("auto", _lib.MSA_DECODE_AUTO), ("vector", _lib.MSA_DECODE_VECTOR),
                                 ("matrix", _lib.MSA_DECODE_MATRIX), ("block", _lib.MSA_DECODE_BLOCK)):
                    prep = Prepared(w, kernel=k, d=d)
                    d = prep.d
                    for _ in range(args.warmup):
                        prep.step()
                    prep.check_error()
                    row[kname] = round(tmean(cold_times(prep.attention, n, prep.stream, flush)) * 1e6, 2)
                    del prep
                row["auto_vs_best"] = round(row["auto"] / min(row["vector"], row["matrix"], row["block"]), 3)
                pts.append(row)
                del d
                torch.cuda.empty_cache()
            result["points"] = pts
        elif args.only in ("decode4", "decode5"):
            w = make_workload(4 if args.only == "decode4" else 5, seed=args.seed)
            prep = Prepared(w, args.split_blocks, kv_layout=layout)
            for _ in range(args.warmup):
                prep.step()
            prep.check_error()
            result["cold_us"] = dist_us(cold_times(prep.attention, n, prep.stream, flush))
        elif args.only == "prefill":
            w = make_workload(3, seed=args.seed)
            prep = Prepared(w)
            prep.plan()
            for _ in range(args.warmup):
                prep.attention()
            prep.check_error()
            warm_for(prep.attention)
            result["us_per_call"] = round(time_calls(prep.attention, n, prep.stream) * 1e6, 3)
        elif args.only == "peaks":
            result["box_peaks"] = box_peaks_leg()
        if args.copy_calibration:
            a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
            bb = torch.empty_like(a)
            for _ in range(5):
                bb.copy_(a)
            torch.cuda.synchronize()
            result["copy_calibration_bytes"] = 256 << 20
        result["only"] = args.only
        print(json.dumps(result), flush=True)
        return

    # ------------------------------------------------------ headline decode step
    w2 = make_workload(2, seed=args.seed)
    head_major = layout == _lib.MSA_LAYOUT_HND
    prep = Prepared(w2, args.split_blocks, kv_layout=layout)
    alg_bytes = decode_bytes(w2)
    stream = prep.stream
    for _ in range(args.warmup):
        prep.step()
    prep.check_error()
    nseg = int(prep.indptr[-1].item())
    # contract region: exactly K steps, each after an untimed cache flush and
    # timed by its own HIP events; bracketed by synchronize on both sides
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step_ts = cold_times(prep.step, args.steps, stream, flush)
    torch.cuda.synchronize()
    bracket_s = time.perf_counter() - t0
    step_s = tmean(step_ts)
    # the same K steps back to back (warm)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        prep.step()
    torch.cuda.synchronize()
    warm_step_s = (time.perf_counter() - t0) / args.steps
    prep.check_error()
    # dominant call: msa_decode (decode kernel + split merge), cold and warm
    # (at least 60 pairs: each pair difference carries the flush's jitter)
    dec_cold = cold_times(prep.attention, max(args.steps, 60), stream, flush)
    dec_warm_s = time_calls(prep.attention, args.steps, stream)
    plan_s = time_calls(prep.plan, args.steps, stream)
    dec_mean = tmean(dec_cold)
    out_headline = prep.out.clone()
    traffic = counter_traffic(COUNTERS, DECODE_SOURCES, split_blocks=args.split_blocks,
                              kv_layout=args.kv_layout)
    value = alg_bytes / step_s / 1e9
    result.update({
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": NAMES[2], "batch": w2.B, "q_heads": w2.Hq, "kv_heads": w2.Hkv,
                   "head_dim": w2.D, "ctx_len": int(w2.ctx_len[0]), "block_size": w2.block_size,
                   "evicted_fraction": round(w2.meta["evicted_fraction"], 4),
                   "alive_tokens": int(sum(alive_tokens_per_seq(w2))), "segments": nseg,
                   "kv_layout": "[P, Hkv, 16, D]" if head_major else "[P, 16, Hkv, D]",
                   "step": "msa_plan_segments + msa_decode (decode kernel + split-K merge)",
                   "timing": "cold: a 512 MiB read evicts L2 and the Infinity Cache before each step; "
                             "each step's time is the HIP-event interval of [flush + step] minus that "
                             "of [flush] alone (pairs interleaved); value and ms_per_step use the "
                             "10%-trimmed mean over the K steps",
                   "seed": args.seed, "parallelism": "single GPU"},
        "tokens_per_s": round(w2.B / step_s, 1),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "step_us": dist_us(step_ts),
        "contract_bracket_s": round(bracket_s, 4),
        "warm_step": {"ms_per_step": round(warm_step_s * 1e3, 4),
                      "GB/s": round(alg_bytes / warm_step_s / 1e9, 2),
                      "tokens_per_s": round(w2.B / warm_step_s, 1),
                      "note": "the same K steps back to back (caches warm), bracketed by synchronize"},
        "roofline": decode_roofline(alg_bytes, dec_mean, dec_warm_s, traffic,
                                    kernel="msa_decode (decode kernel, plus the split merge when a "
                                           "sequence has several splits)"),
        "decode_call_us": dist_us(dec_cold),
        "plan_us_per_call": round(plan_s * 1e6, 3),
        "decode_tokens_per_s": round(w2.B / dec_mean, 1),
    })
    if not args.no_gather:
        # the gather-then-attend detour on the same inputs, same kernel
        gb = GatherBaseline(prep)
        for _ in range(3):
            gb.step()
        torch.cuda.synchronize()
        n = max(10, args.steps // 2)
        g_step = tmean(cold_times(gb.step, n, stream, flush))
        g_copy = tmean(cold_times(gb.gather, n, stream, flush))
        g_attn = time_calls(gb.attention, n, stream)
        result["gather_baseline"] = {
            "us_per_call": round(g_step * 1e6, 3), "gather_us": round(g_copy * 1e6, 3),
            "dense_decode_us_warm": round(g_attn * 1e6, 3), "msa_decode_us": round(dec_mean * 1e6, 3),
            "msa_speedup": round(g_step / dec_mean, 3),
            "note": "cold (flush-subtracted): gather alive K/V blocks into dense pools (msa_gather_alive) + msa_decode "
                    "over one segment per sequence, vs msa_decode over the segments"}
        del gb
        torch.cuda.empty_cache()
    d2 = prep.d
    del prep
    torch.cuda.empty_cache()
    if cpu:
        result["cpu_baseline"] = decode_cpu_baseline(w2, budget_s=12.0, max_reps=60,
                                                     label="the headline batch,")
    if not args.no_layout and not head_major:
        # the same batch with head-major pool blocks (msa_decode_ex)
        dh = dict(d2)
        dh["k_pool"] = d2["k_pool"].permute(0, 2, 1, 3).contiguous()
        dh["v_pool"] = d2["v_pool"].permute(0, 2, 1, 3).contiguous()
        leg, out = decode_leg(w2, args.steps, flush, kv_layout=_lib.MSA_LAYOUT_HND, d=dh)
        leg["bitwise_equal_to_token_major"] = bool(torch.equal(out, out_headline))
        leg["note"] = ("msa_decode_ex on the same batch with head-major pool blocks [P, Hkv, 16, D] "
                       "(each KV head's 16 rows of a block contiguous)")
        result["decode_hnd"] = leg
        del dh, out
        torch.cuda.empty_cache()
    del d2
    torch.cuda.empty_cache()

    # --------------------------------------- the other decode workloads
    w5 = None
    if not args.no_more_decode:
        w1 = make_workload(1, seed=args.seed)
        leg, _ = decode_leg(w1, args.steps, flush)
        leg["note"] = "correctness configuration: 0.79 MB of K/V per call, launch-latency bound"
        if cpu:
            leg["cpu_baseline"] = decode_cpu_baseline(w1, budget_s=2.0, label="the fp32 batch,")
        result["decode_small_fp32"] = {"workload": NAMES[1], **leg}
        n = max(10, args.steps // 2)
        w4 = make_workload(4, seed=args.seed)
        leg, _ = decode_leg(w4, n, flush, kv_layout=layout, unique=True)
        leg["roofline"]["traffic"] = counter_traffic(COUNTERS4, DECODE_SOURCES, split_blocks=0,
                                                     kv_layout=args.kv_layout)
        if cpu:
            pick = sorted(np.random.default_rng(args.seed + 4).choice(w4.B, 4, replace=False).tolist())
            leg["cpu_baseline"] = decode_cpu_baseline(w4, seqs=pick, budget_s=4.0, single=False,
                                                      label="the lognormal batch,")
        result["decode_lognormal"] = {"workload": NAMES[4], **leg}
        del w4
        w5 = make_workload(5, seed=args.seed)
        leg, _ = decode_leg(w5, n, flush, kv_layout=layout)
        leg["roofline"]["traffic"] = counter_traffic(COUNTERS5, DECODE_SOURCES, split_blocks=0,
                                                     kv_layout=args.kv_layout)
        if cpu:
            leg["cpu_baseline"] = decode_cpu_baseline(w5, seqs=[0], budget_s=4.0, single=False,
                                                      label="the 131k-token batch,")
        result["decode_long"] = {"workload": NAMES[5], **leg}
        torch.cuda.empty_cache()

    # --------------------------- vector against matrix-core decode kernel
    if not args.no_kernels:
        if w5 is None:
            w5 = make_workload(5, seed=args.seed)
        result["decode_kernels"] = kernels_leg(args, flush, w2, w5)
    del w5
    torch.cuda.empty_cache()

    # -------------------------- kernel-aware against hit-only eviction
    if not args.no_eviction:
        result["eviction"] = eviction_leg(args, flush, w2)

    if args.latency_model:
        result["latency_model"] = latency_model_leg(args, flush)

    # --------------------------------------------------------------- prefill
    if not args.no_prefill and msa.prefill_available():
        n = max(10, args.steps // 2)
        wp = make_workload(3, seed=args.seed)
        leg = prefill_leg(wp, n, max(3, args.warmup // 4), flush)
        tfs = leg["TFLOP/s"]
        pf_traffic = counter_traffic(PF_COUNTERS, PREFILL_SOURCES, split_blocks=0)
        leg["roofline"] = {"bound": "mfma", "achieved": tfs, "peak": MFMA_BF16_PEAK_TFS,
                           "unit": "TFLOP/s", "frac": round(tfs / MFMA_BF16_PEAK_TFS, 4),
                           "traffic": pf_traffic, "traffic_unit": "bytes per call",
                           "kernel": "msa_prefill_chunk",
                           "timing": "mean of back-to-back calls after a quarter second of warm-up",
                           "algorithmic_flops_per_call": leg.pop("flops")}
        if cpu:
            leg["cpu_baseline"] = prefill_cpu_baseline(wp, budget_s=10.0, max_reps=40)
        result["prefill"] = {"workload": NAMES[3], **leg}
        del wp
        if not args.no_recompute:
            # recompute of an evicted middle range (chunk rows in the middle of
            # the context, later alive blocks hidden by the causal mask)
            wr = make_workload(6, seed=args.seed)
            leg = prefill_leg(wr, n, 3)
            leg.pop("flops")
            result["recompute"] = {"workload": NAMES[6], **leg}
            del wr
        if not args.no_chunk_sweep:
            result["chunk_sweep"] = chunk_sweep_leg(args, flush)
    if not args.no_box_peaks:
        result["box_peaks"] = box_peaks_leg()
    if args.copy_calibration:
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        bb = torch.empty_like(a)
        for _ in range(5):
            bb.copy_(a)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = 256 << 20
    print(json.dumps(result), flush=True)


def latency_model_leg(args, flush):
    """Fit msa_decode time = c0 + c_tok * alive tokens + c_seg * segments over
    new decode batches that vary the context length (alive tokens) and the
    mean alive-run length (segments at a given token count)."""
    import numpy as np
    import torch
    from kv_cache_attention_msa_amd.evict import DecodeLatencyModel
    from workloads import make_workload
    pts = []
    for ctx in (2048, 4096, 8192):
        for run in (1.0, 4.0, 32.0):
            w = make_workload(2, seed=args.seed, ctx=ctx, mean_alive=run, mean_dead=max(1.0, run / 4),
                              pool_factor=2.5)
            prep = Prepared(w)
            prep.plan()
            prep.attention()
            prep.check_error()
            t = tmean(cold_times(prep.attention, 20, prep.stream, flush))
            pts.append({"ctx": ctx, "mean_alive_run": run, "alive_tokens": int(sum(alive_tokens_per_seq(w))),
                        "segments": int(prep.indptr[-1].item()), "us": round(t * 1e6, 3)})
            del prep, w
            torch.cuda.empty_cache()
    m = DecodeLatencyModel.fit([p["alive_tokens"] for p in pts], [p["segments"] for p in pts],
                               [p["us"] for p in pts])
    pred = m.predict([p["alive_tokens"] for p in pts], [p["segments"] for p in pts])
    meas = np.array([p["us"] for p in pts])
    r2 = 1.0 - float(((meas - pred) ** 2).sum() / ((meas - meas.mean()) ** 2).sum())
    return {"c0_us": round(m.c0, 3), "c_tok_us": m.c_tok, "c_seg_us": m.c_seg, "r2": round(r2, 4),
            "points": pts}


if __name__ == "__main__":
    main()
