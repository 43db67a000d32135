"""Seeded synthetic inputs for Multi-Segment Attention (MSA).

This module only *draws* inputs: context lengths, which KV blocks survive
eviction, where the surviving blocks sit in the physical pool, and the Q/K/V
values.  It holds none of the method's arithmetic (no segment plan, no
attention), so both the fp64 oracle and the HIP path can consume what it
produces without sharing any computation.

The five workload families stand in for the pages' "multi-session, multi-turn
dialogue" and "long-context" serving workloads (P2, Methodology / Key Results;
P1, "关键实验与数据"), which name no dataset.  Draw order per instance is fixed:
lengths -> eviction pattern -> placement -> Q -> K pool -> V pool, all from one
``numpy.random.default_rng(seed)``.

Layout of what is returned (see ``Workload``):
  block_table int32 [B, max_blocks]   logical block -> physical block id
                                      (-1, or a stale id, where not alive)
  alive       uint8 [B, max_blocks]   1 = block resident (survived eviction)
  ctx_len     int32 [B]               tokens in the sequence (all positions)
  k_pool/v_pool [P, block_size, Hkv, D]  float32 (fp32 workloads) or uint16
                                      bf16 bit patterns (bf16 workloads)
  q           [B, Hq, D] (decode) or [B, C, Hq, D] (prefill), same dtype rule
Every pool slot that does not hold an alive token (free slots, evicted
blocks, padding past ctx_len in a last block) is NaN.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BF16_NAN_BITS = np.uint16(0x7FC0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest even) and return the bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    out = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    out[np.isnan(x)] = BF16_NAN_BITS
    return out


@dataclass
class Workload:
    name: str
    kind: str  # "decode" | "prefill"
    dtype: str  # "f32" | "bf16"
    B: int
    Hq: int
    Hkv: int
    D: int
    block_size: int
    block_table: np.ndarray
    alive: np.ndarray
    ctx_len: np.ndarray
    q: np.ndarray
    k_pool: np.ndarray
    v_pool: np.ndarray
    scale: float
    C: int = 1
    q_pos0: np.ndarray | None = None
    meta: dict = field(default_factory=dict)

    @property
    def num_phys_blocks(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def max_ctx_len(self) -> int:
        return int(self.ctx_len.max()) if self.B else 0


# ----------------------------------------------------------------------------
# eviction patterns
# ----------------------------------------------------------------------------

def _alternating_runs(rng, nb, draw_alive, draw_dead):
    """Alive mask of length nb made of alternating alive/evicted runs, alive first."""
    mask = np.zeros(nb, dtype=np.uint8)
    pos, alive = 0, True
    while pos < nb:
        n = int(draw_alive() if alive else draw_dead())
        n = max(1, n)
        if alive:
            mask[pos:pos + n] = 1
        pos += n
        alive = not alive
    return mask


def _runs_of(mask, lo=0, hi=None):
    """Maximal logical runs of alive blocks in mask[lo:hi] as (start, length)."""
    hi = len(mask) if hi is None else hi
    runs, l = [], lo
    while l < hi:
        if mask[l]:
            s = l
            while l < hi and mask[l]:
                l += 1
            runs.append((s, l - s))
        else:
            l += 1
    return runs


def _place_runs_with_gaps(rng, run_sizes, pool_blocks):
    """Shuffle runs and lay them into a pool of pool_blocks slots, each run
    contiguous, at least one free slot between neighbouring runs.
    Returns (order, starts) with starts[i] the slot of run i's first block."""
    n = len(run_sizes)
    used = int(sum(run_sizes))
    free = pool_blocks - used
    assert free >= max(0, n - 1), "pool too small for gaps"
    order = rng.permutation(n)
    # n+1 gaps: before, between (>=1), after
    extra = free - max(0, n - 1)
    extra_split = rng.multinomial(extra, np.full(n + 1, 1.0 / (n + 1)))
    starts = np.zeros(n, dtype=np.int64)
    cur = int(extra_split[0])
    for j, i in enumerate(order):
        starts[i] = cur
        cur += int(run_sizes[i])
        if j + 1 < n:
            cur += 1 + int(extra_split[j + 1])
    assert cur <= pool_blocks
    return starts


# ----------------------------------------------------------------------------
# value fill
# ----------------------------------------------------------------------------

_VALUES = {"on": True}


def _fill_pools_and_q(rng, dtype, q_shape, P, bs, Hkv, D, live_slots):
    """Draw Q, then the K pool, then the V pool, N(0,1); poison dead slots.

    live_slots: bool [P, bs], True where an alive token lives.
    """
    if not _VALUES["on"]:
        shape = (P, bs, Hkv, D)
        return None, np.empty((shape[0], 0), np.float32), None
    q = rng.standard_normal(q_shape, dtype=np.float32)
    pools = []
    dead = ~live_slots
    for _ in range(2):
        pool = rng.standard_normal((P, bs, Hkv, D), dtype=np.float32)
        pool[dead] = np.nan
        pools.append(pool)
    if dtype == "bf16":
        q = f32_to_bf16_bits(q)
        pools = [f32_to_bf16_bits(p) for p in pools]
    return q, pools[0], pools[1]


def _live_slots(P, bs, block_table, alive, ctx_len):
    live = np.zeros((P, bs), dtype=bool)
    if not _VALUES["on"]:
        return live
    B = block_table.shape[0]
    for b in range(B):
        nb = -(-int(ctx_len[b]) // bs)
        for l in range(nb):
            if alive[b, l]:
                ntok = min(bs, int(ctx_len[b]) - l * bs)
                live[block_table[b, l], :ntok] = True
    return live


# ----------------------------------------------------------------------------
# the five workload families
# ----------------------------------------------------------------------------

def _decode_fp32_permuted(rng, B=1, Hq=8, Hkv=2, D=64, nb=64, pool=256, n_evict=16, dtype="f32"):
    """Decode, fp32: table = first nb entries of a random permutation of the pool;
    exactly n_evict of the first nb-1 blocks evicted uniformly."""
    bs = 16
    ctx_len = np.full(B, nb * bs, dtype=np.int32)
    alive = np.ones((B, nb), dtype=np.uint8)
    for b in range(B):
        ev = rng.choice(nb - 1, size=n_evict, replace=False)
        alive[b, ev] = 0
    table = np.full((B, nb), -1, dtype=np.int32)
    perm = rng.permutation(pool)
    # sequences take disjoint slices of one permutation of the pool
    assert B * nb <= pool
    for b in range(B):
        table[b] = perm[b * nb:(b + 1) * nb]
    table[alive == 0] = -1
    q_shape = (B, Hq, D)
    live = _live_slots(pool, bs, table, alive, ctx_len)
    q, kp, vp = _fill_pools_and_q(rng, dtype, q_shape, pool, bs, Hkv, D, live)
    return dict(kind="decode", dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, block_size=bs,
                block_table=table, alive=alive, ctx_len=ctx_len, q=q, k_pool=kp, v_pool=vp)


def _geom_runs_layout(rng, B, nb_cached, mean_alive, mean_dead, chunk_blocks, pool_factor):
    """Alive runs of geometric length, evicted runs of geometric length; each
    alive run (and the prefill chunk, if any) is physically contiguous, and
    all runs of all sequences are shuffled into the pool with gaps >= 1."""
    nb = nb_cached + chunk_blocks
    alive = np.zeros((B, nb), dtype=np.uint8)
    for b in range(B):
        m = _alternating_runs(rng, nb_cached,
                              lambda: rng.geometric(1.0 / mean_alive),
                              lambda: rng.geometric(1.0 / mean_dead))
        if chunk_blocks == 0:
            m[-1] = 1  # the block holding the newest token is never evicted
        alive[b, :nb_cached] = m
        alive[b, nb_cached:] = 1
    runs = []  # (b, logical start, length)
    for b in range(B):
        for s, n in _runs_of(alive[b], 0, nb_cached):
            runs.append((b, s, n))
        if chunk_blocks:
            # the chunk is its own run even if the last cached block is alive
            runs.append((b, nb_cached, chunk_blocks))
    sizes = [n for (_, _, n) in runs]
    used = int(sum(sizes))
    P = int(math.ceil(pool_factor * used))
    starts = _place_runs_with_gaps(rng, sizes, P)
    table = np.full((B, nb), -1, dtype=np.int32)
    for (b, s, n), st in zip(runs, starts):
        table[b, s:s + n] = np.arange(st, st + n, dtype=np.int32)
    return alive, table, P


def _decode_geometric_runs(rng, B=32, Hq=32, Hkv=8, D=128, ctx=4096, mean_alive=8.0, mean_dead=2.0,
          dtype="bf16", pool_factor=1.25):
    """Decode, bf16: alternating alive ~ Geom(mean 8) / evicted ~ Geom(mean 2) runs."""
    bs = 16
    nb = -(-ctx // bs)
    alive, table, P = _geom_runs_layout(rng, B, nb, mean_alive, mean_dead, 0, pool_factor)
    ctx_len = np.full(B, ctx, dtype=np.int32)
    live = _live_slots(P, bs, table, alive, ctx_len)
    q, kp, vp = _fill_pools_and_q(rng, dtype, (B, Hq, D), P, bs, Hkv, D, live)
    return dict(kind="decode", dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, block_size=bs,
                block_table=table, alive=alive, ctx_len=ctx_len, q=q, k_pool=kp, v_pool=vp)


def _prefill_chunk(rng, B=4, Hq=32, Hkv=8, D=128, cached=8192, C=512, mean_alive=16.0,
          evict_frac=0.15, dtype="bf16"):
    """Chunked prefill, bf16: C query rows at positions [cached, cached+C) over
    the alive cached blocks plus the chunk's own blocks (causal)."""
    bs = 16
    assert cached % bs == 0
    nb_c = cached // bs
    cb = -(-C // bs)
    mean_dead = mean_alive * evict_frac / (1.0 - evict_frac)
    alive, table, P = _geom_runs_layout(rng, B, nb_c, mean_alive, mean_dead, cb, 1.25)
    ctx_len = np.full(B, cached + C, dtype=np.int32)
    live = _live_slots(P, bs, table, alive, ctx_len)
    q, kp, vp = _fill_pools_and_q(rng, dtype, (B, C, Hq, D), P, bs, Hkv, D, live)
    q_pos0 = np.full(B, cached, dtype=np.int32)
    return dict(kind="prefill", dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, block_size=bs,
                block_table=table, alive=alive, ctx_len=ctx_len, q=q, k_pool=kp, v_pool=vp,
                C=C, q_pos0=q_pos0)


def _prefill_recompute_middle(rng, B=4, Hq=32, Hkv=8, D=128, ctx=8704, q_pos0=4096, C=512, mean_alive=16.0,
          evict_frac=0.15, dtype="bf16"):
    """Recompute (lossless reconstruction), bf16: an evicted range of C tokens
    in the middle of the context, [q_pos0, q_pos0+C), is recomputed as a
    prefill chunk.  Its K/V go into fresh pool slots (one contiguous run, like
    a chunk) and the sequence is re-planned; the alive blocks after the chunk
    stay in the plan and are hidden from the chunk rows by the causal mask
    alone.  Elsewhere blocks are evicted in geometric runs as in the prefill
    family."""
    bs = 16
    assert q_pos0 % bs == 0 and ctx % bs == 0 and q_pos0 + C <= ctx
    nb = ctx // bs
    c0, cb = q_pos0 // bs, -(-C // bs)
    mean_dead = mean_alive * evict_frac / (1.0 - evict_frac)
    alive = np.zeros((B, nb), dtype=np.uint8)
    for b in range(B):
        alive[b] = _alternating_runs(rng, nb, lambda: rng.geometric(1.0 / mean_alive),
                                     lambda: rng.geometric(1.0 / mean_dead))
        alive[b, c0:c0 + cb] = 1
        alive[b, nb - 1] = 1
    runs = []
    for b in range(B):
        for st, n in _runs_of(alive[b], 0, c0):
            runs.append((b, st, n))
        runs.append((b, c0, cb))  # the recomputed range: fresh slots, its own run
        for st, n in _runs_of(alive[b], c0 + cb, nb):
            runs.append((b, st, n))
    sizes = [n for (_, _, n) in runs]
    P = int(math.ceil(1.25 * sum(sizes)))
    starts = _place_runs_with_gaps(rng, sizes, P)
    table = np.full((B, nb), -1, dtype=np.int32)
    for (b, st, n), ps in zip(runs, starts):
        table[b, st:st + n] = np.arange(ps, ps + n, dtype=np.int32)
    ctx_len = np.full(B, ctx, dtype=np.int32)
    live = _live_slots(P, bs, table, alive, ctx_len)
    q, kp, vp = _fill_pools_and_q(rng, dtype, (B, C, Hq, D), P, bs, Hkv, D, live)
    return dict(kind="prefill", dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, block_size=bs,
                block_table=table, alive=alive, ctx_len=ctx_len, q=q, k_pool=kp, v_pool=vp,
                C=C, q_pos0=np.full(B, q_pos0, dtype=np.int32))


def _decode_lognormal_shared_prefix(rng, B=64, Hq=32, Hkv=8, D=128, median=6144, sigma=0.75, lo=2064, hi=32768,
          shared_tokens=2048, group=16, evict_frac=0.3, dtype="bf16"):
    """Multi-session decode mix: lognormal contexts, a shared prefix per group of
    sequences (one contiguous run, never evicted), a fraction of each sequence's
    private blocks evicted (their slots become NaN holes, the table keeps the
    stale id)."""
    bs = 16
    ctx_len = np.clip(np.round(rng.lognormal(math.log(median), sigma, size=B)), lo, hi)
    ctx_len = ctx_len.astype(np.int32)
    nsh = shared_tokens // bs
    max_blocks = hi // bs
    alive = np.zeros((B, max_blocks), dtype=np.uint8)
    for b in range(B):
        nb = -(-int(ctx_len[b]) // bs)
        alive[b, :nb] = 1
        npriv = nb - nsh
        k = int(round(evict_frac * (npriv - 1)))
        if k > 0:
            ev = rng.choice(npriv - 1, size=k, replace=False)
            alive[b, nsh + ev] = 0
    ngroups = -(-B // group)
    # runs: shared prefixes, then each sequence's private range (holes included)
    sizes = [nsh] * ngroups
    for b in range(B):
        nb = -(-int(ctx_len[b]) // bs)
        sizes.append(nb - nsh)
    used = int(sum(sizes))
    P = int(math.ceil(1.25 * used))
    starts = _place_runs_with_gaps(rng, sizes, P)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    for b in range(B):
        nb = -(-int(ctx_len[b]) // bs)
        gs = int(starts[b // group])
        table[b, :nsh] = np.arange(gs, gs + nsh, dtype=np.int32)
        ps = int(starts[ngroups + b])
        table[b, nsh:nb] = np.arange(ps, ps + nb - nsh, dtype=np.int32)
    live = _live_slots(P, bs, table, alive, ctx_len)
    q, kp, vp = _fill_pools_and_q(rng, dtype, (B, Hq, D), P, bs, Hkv, D, live)
    return dict(kind="decode", dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, block_size=bs,
                block_table=table, alive=alive, ctx_len=ctx_len, q=q, k_pool=kp, v_pool=vp)


def _decode_long_fragmented(rng, B=4, Hq=64, Hkv=8, D=128, ctx=131072, dtype="bf16"):
    """Long-context fragmented decode: alive/evicted runs of 1-2 blocks each;
    every alive block at its own random pool slot."""
    bs = 16
    nb = -(-ctx // bs)
    alive = np.zeros((B, nb), dtype=np.uint8)
    for b in range(B):
        m = _alternating_runs(rng, nb, lambda: rng.integers(1, 3), lambda: rng.integers(1, 3))
        m[-1] = 1
        alive[b] = m
    used = int(alive.sum())
    P = int(math.ceil(1.25 * used))
    slots = rng.permutation(P)[:used]
    table = np.full((B, nb), -1, dtype=np.int32)
    table[alive == 1] = slots.astype(np.int32)
    ctx_len = np.full(B, ctx, dtype=np.int32)
    live = _live_slots(P, bs, table, alive, ctx_len)
    q, kp, vp = _fill_pools_and_q(rng, dtype, (B, Hq, D), P, bs, Hkv, D, live)
    return dict(kind="decode", dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, block_size=bs,
                block_table=table, alive=alive, ctx_len=ctx_len, q=q, k_pool=kp, v_pool=vp)


_FAMILIES = {1: _decode_fp32_permuted, 2: _decode_geometric_runs, 3: _prefill_chunk, 4: _decode_lognormal_shared_prefix, 5: _decode_long_fragmented, 6: _prefill_recompute_middle}

NAMES = {
    1: "decode_f32_b1_h8kv2_d64_ctx1k_evict25_randperm",
    2: "decode_bf16_b32_h32kv8_d128_ctx4k_evict20_geomruns8",
    3: "prefill_bf16_b4_h32kv8_d128_chunk512_cached8k_evict15",
    4: "decode_bf16_b64_h32kv8_d128_lognormal6k_shared2k_evict30",
    5: "decode_bf16_b4_h64kv8_d128_ctx128k_evict50_runs1to2",
    6: "recompute_bf16_b4_h32kv8_d128_chunk512_at4k_ctx8704_evict15",
}

# Reduced sizes with the same recipe: several tiles and ragged tails, but small
# enough for the fp64 oracle to finish in seconds.
SMALL = {
    1: {},
    2: dict(B=6, ctx=1024 + 512),
    3: dict(B=2, cached=1024, C=96),
    4: dict(B=8, median=2600, lo=2064, hi=4000, group=4),
    5: dict(B=2, ctx=4096),
    6: dict(B=2, ctx=1536, q_pos0=512, C=96),
}


def make_workload(family: int, seed: int = 0, size: str = "full", values: bool = True,
                  **overrides) -> Workload:
    """Draw workload family ``family`` (1..6) with ``seed``.

    size="full" uses the family's defining sizes, "small" the reduced ones;
    keyword overrides change individual shape parameters.  values=False skips
    the Q/K/V draw (they come last, so the tables are the same either way):
    q and v_pool are then None and k_pool is an empty [P, 0] placeholder.
    """
    fn = _FAMILIES[family]
    kw = {}
    if size == "small":
        kw.update(SMALL[family])
    elif size != "full":
        raise ValueError(size)
    kw.update(overrides)
    rng = np.random.default_rng(seed)
    _VALUES["on"] = values
    try:
        d = fn(rng, **kw)
    finally:
        _VALUES["on"] = True
    D = d["D"]
    w = Workload(name=NAMES[family] if size == "full" and not overrides else f"{NAMES[family]}[{size}]",
                 scale=1.0 / math.sqrt(D), **d)
    bs = w.block_size
    nb = -(-w.ctx_len.astype(np.int64) // bs)
    tot = int(nb.sum())
    alive_blocks = int(sum(int(w.alive[b, :nb[b]].sum()) for b in range(w.B)))
    w.meta = dict(seed=seed, family=family, size=size, pool_blocks=w.num_phys_blocks,
                  logical_blocks=tot, alive_blocks=alive_blocks,
                  evicted_fraction=1.0 - alive_blocks / max(tot, 1))
    return w


def random_small_case(rng, B=None, bs=None, max_nb=8, pool=None, allow_stale=True):
    """A tiny random (table, alive, ctx_len) triple with a valid layout, for
    fuzzing the segment plan: distinct physical ids within a sequence, some
    forced physical adjacency and descending ids."""
    B = int(rng.integers(1, 4)) if B is None else B
    bs = int(rng.choice([1, 2, 4, 16])) if bs is None else bs
    nb_max = max_nb
    pool = pool if pool is not None else 2 * nb_max + 4
    table = np.full((B, nb_max), -1, dtype=np.int32)
    alive = np.zeros((B, nb_max), dtype=np.uint8)
    ctx_len = np.zeros(B, dtype=np.int32)
    for b in range(B):
        nb = int(rng.integers(0, nb_max + 1))
        ctx_len[b] = 0 if nb == 0 else (nb - 1) * bs + int(rng.integers(1, bs + 1))
        mode = int(rng.integers(0, 3))
        if mode == 0:
            ids = rng.permutation(pool)[:nb]
        elif mode == 1:
            st = int(rng.integers(0, pool - nb + 1)) if nb else 0
            ids = np.arange(st, st + nb)
        else:
            st = int(rng.integers(nb, pool)) if nb else 0
            ids = np.arange(st, st - nb, -1)
        table[b, :nb] = ids
        alive[b, :nb] = rng.integers(0, 2, size=nb)
        dead = alive[b] == 0
        if not allow_stale or rng.random() < 0.5:
            table[b, dead] = -1
    return table, alive, ctx_len, bs, pool
