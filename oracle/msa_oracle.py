"""fp64 CPU oracle for Multi-Segment Attention (MSA).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, links or runs
this module: only the tests, the smoke check and the CPU-baseline leg of the
benchmark do.  It shares no code, constant or helper with the HIP library.

Sources (web pages, cited by title and section):
  P1  "AsymCache：把 KV Cache 决策摆到 GPU 注意力内核的同一张桌子上"
      (papers.ananclaw.com explainer of arXiv 2606.02964), section
      "核心方法 / 1. Multi-Segment Attention (MSA)" with its pseudocode.
  P2  "Multi-Segment Attention: Enabling Efficient KV-Cache Management for
      Faster Large Language Model Serving" (gptget.net), Abstract and
      Methodology.

What it computes, and why this is the plain definition:
  * The pages call eviction *lossless*: outputs equal those of the model that
    never evicted, for the tokens that are kept (P2 Abstract; P1 "它在解决什么
    真问题", item 2).  MSA only changes how attention over the surviving
    tokens is evaluated (split into segments, per-segment attention, stitched
    by a normaliser; P1 MSA pseudocode).  So the oracle for attention is dense
    softmax attention over every alive token, taken in logical order, with a
    key visible to a query iff its logical position is not after the query's
    (causal masking by logical position).  It does NOT use the segment plan:
    it reads the alive tokens straight from the block table.
  * The segment plan is the pages' `split_into_contiguous_segments`: the
    alive blocks of a sequence cut into maximal runs that are contiguous in
    physical memory (P1 MSA pseudocode comment and the paragraph after it:
    the split follows the physical layout, and a hole left by an evicted
    block breaks a run).  Reading used here: a run continues from logical
    block l to l+1 iff both are alive and phys(l+1) == phys(l)+1.
  * `normalizer(seg)` is not defined on the pages; the reading used is the
    log-sum-exp weight, which makes the stitched result equal dense
    attention.  `merge_ref` states it for partials (m, l, o).

Every function is parity-pinned by the `-m "not gpu"` tests in tests/
(brute force, closed forms, a library reduction to torch's SDPA, invariants).
"""
from __future__ import annotations

import math

import numpy as np

# Plan record fields, in order (int32 each).
SEG_FIELDS = ("seq", "logical_block", "phys_block", "num_blocks", "num_tokens",
              "alive_token_start")


# ----------------------------------------------------------------------------
# a1: segment plan  (P1, MSA pseudocode: split_into_contiguous_segments)
# ----------------------------------------------------------------------------

def plan_ref(block_table, alive, ctx_len, block_size):
    """Cut each sequence's alive blocks into maximal physically-contiguous runs.

    Walk logical blocks l = 0 .. ceil(ctx_len/bs)-1 of sequence b, skipping
    dead ones.  An alive block extends the current record iff the record ends
    at logical l-1 and at physical table[b,l]-1; otherwise it opens a new
    record.  Records are listed by (seq, logical_block).

    Returns (segs int32 [N, 6], seg_indptr int32 [B+1]) with the fields
    SEG_FIELDS.  num_tokens counts positions < ctx_len only;
    alive_token_start is the number of alive tokens of the sequence before
    the record.
    """
    table = np.asarray(block_table)
    alive = np.asarray(alive)
    ctx_len = np.asarray(ctx_len)
    B = table.shape[0]
    bs = int(block_size)
    recs = []
    indptr = [0]
    for b in range(B):
        n_tok = int(ctx_len[b])
        nb = (n_tok + bs - 1) // bs
        cur = None  # [seq, lb, pb, nblk, ntok, start]
        running = 0
        for l in range(nb):
            if not alive[b, l]:
                continue
            p = int(table[b, l])
            tokens_here = min(bs, n_tok - l * bs)
            if cur is not None and cur[1] + cur[3] == l and cur[2] + cur[3] == p:
                cur[3] += 1
                cur[4] += tokens_here
            else:
                if cur is not None:
                    recs.append(cur)
                    running += cur[4]
                cur = [b, l, p, 1, tokens_here, running]
        if cur is not None:
            recs.append(cur)
        indptr.append(len(recs))
    segs = np.array(recs, dtype=np.int32).reshape(-1, 6)
    return segs, np.array(indptr, dtype=np.int32)


# ----------------------------------------------------------------------------
# reading the pool
# ----------------------------------------------------------------------------

def to_f64(x):
    """Stored values -> float64, exactly.  uint16 arrays are bf16 bit patterns
    (the upper half of an IEEE float32); float arrays are taken as they are."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def alive_tokens_ref(block_table, alive, ctx_len, b, block_size):
    """Alive tokens of sequence b in logical order, straight from the table.

    Returns (phys_block, slot, position) int64 arrays: the token at logical
    position p lives in block table[b, p//bs] at slot p%bs; it is kept iff
    its block is alive and p < ctx_len.  (Positions are the original logical
    positions; eviction does not renumber them.)
    """
    bs = int(block_size)
    n_tok = int(ctx_len[b])
    pos = np.arange(n_tok, dtype=np.int64)
    lblk = pos // bs
    keep = np.asarray(alive)[b, lblk].astype(bool) if n_tok else np.zeros(0, bool)
    pos = pos[keep]
    lblk = lblk[keep]
    phys = np.asarray(block_table)[b, lblk].astype(np.int64)
    return phys, pos % bs, pos


# ----------------------------------------------------------------------------
# a3/a4: attention over the alive tokens
# ----------------------------------------------------------------------------

def attention_ref(q_rows, q_pos, keys, values, k_pos, scale):
    """Dense softmax attention of query rows over keys, fp64.

    q_rows [R, D], q_pos [R], keys/values [N, D], k_pos [N].  Key j is
    visible to row i iff k_pos[j] <= q_pos[i].  Returns (O [R, D], LSE [R])
    with LSE = ln(sum_j visible exp(s_ij)), s = scale * q.k.  A row with no
    visible key gets O = 0 and LSE = -inf.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    R, D = q_rows.shape
    out = np.zeros((R, values.shape[1] if values.ndim == 2 else D), dtype=np.float64)
    lse = np.full(R, -np.inf, dtype=np.float64)
    if keys.shape[0] == 0 or R == 0:
        return out, lse
    s = scale * (q_rows @ keys.T)                        # [R, N]
    vis = np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None]
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1)
    has = np.isfinite(m)
    w = np.zeros_like(s)
    w[has] = np.exp(s[has] - m[has, None])
    w[~vis] = 0.0
    den = w.sum(axis=1)
    out[has] = (w[has] @ values) / den[has, None]
    lse[has] = m[has] + np.log(den[has])
    return out, lse


def _gather(pool, phys, slot, g):
    return to_f64(np.asarray(pool)[phys, slot, g, :])


def decode_ref(q, k_pool, v_pool, block_table, alive, ctx_len, block_size, scale,
               seqs=None, heads=None):
    """MSA decode: one query per sequence at position ctx_len-1, over the
    sequence's alive tokens (all of which are at or before it).

    q [B, Hq, D]; pools [P, bs, Hkv, D]; GQA: query head h reads KV head
    h // (Hq // Hkv).  Returns (O [B, Hq, D], LSE [B, Hq]) in fp64; entries of
    sequences/heads not in `seqs`/`heads` are left NaN.
    """
    q = to_f64(q)
    B, Hq, D = q.shape
    Hkv = np.asarray(k_pool).shape[2]
    G = Hq // Hkv
    O = np.full((B, Hq, D), np.nan)
    L = np.full((B, Hq), np.nan)
    seqs = range(B) if seqs is None else seqs
    heads = range(Hq) if heads is None else heads
    for b in seqs:
        phys, slot, pos = alive_tokens_ref(block_table, alive, ctx_len, b, block_size)
        qpos = np.array([int(ctx_len[b]) - 1])
        by_kv = {}
        for h in heads:
            by_kv.setdefault(h // G, []).append(h)
        for g, hs in by_kv.items():
            K = _gather(k_pool, phys, slot, g)
            V = _gather(v_pool, phys, slot, g)
            for h in hs:
                o, l = attention_ref(q[b, h][None, :], qpos, K, V, pos, scale)
                O[b, h] = o[0]
                L[b, h] = l[0]
    return O, L


def prefill_ref(q, q_pos0, k_pool, v_pool, block_table, alive, ctx_len, block_size,
                scale, seqs=None, heads=None, rows=None):
    """MSA chunked prefill: C query rows of sequence b at logical positions
    q_pos0[b] + i.  The chunk's own K/V are already alive blocks of the pool;
    key visible iff its position <= the row's position.

    q [B, C, Hq, D].  Returns (O [B, C, Hq, D], LSE [B, C, Hq]) fp64; entries
    not requested stay NaN.
    """
    q = to_f64(q)
    B, C, Hq, D = q.shape
    Hkv = np.asarray(k_pool).shape[2]
    G = Hq // Hkv
    O = np.full((B, C, Hq, D), np.nan)
    L = np.full((B, C, Hq), np.nan)
    seqs = range(B) if seqs is None else seqs
    heads = range(Hq) if heads is None else heads
    rows = np.arange(C) if rows is None else np.asarray(rows)
    for b in seqs:
        phys, slot, pos = alive_tokens_ref(block_table, alive, ctx_len, b, block_size)
        qpos = int(q_pos0[b]) + rows
        by_kv = {}
        for h in heads:
            by_kv.setdefault(h // G, []).append(h)
        for g, hs in by_kv.items():
            K = _gather(k_pool, phys, slot, g)
            V = _gather(v_pool, phys, slot, g)
            for h in hs:
                o, l = attention_ref(q[b, rows, h], qpos, K, V, pos, scale)
                O[b, rows, h] = o
                L[b, rows, h] = l
    return O, L


# ----------------------------------------------------------------------------
# a5: partials and their log-sum-exp merge  (P1 MSA pseudocode: the
# per-segment result times normalizer(seg), accumulated into `out`)
# ----------------------------------------------------------------------------

def partial_ref(q_rows, q_pos, keys, values, k_pos, scale):
    """One partial over a subset of keys: m = max visible score, l = sum of
    exp(s - m), o = sum of exp(s - m) * v (unnormalised).  With no visible
    key: m = -inf, l = 0, o = 0."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    R = q_rows.shape[0]
    Dv = values.shape[1]
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    o = np.zeros((R, Dv))
    if keys.shape[0] == 0:
        return m, l, o
    s = scale * (q_rows @ keys.T)
    vis = np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None]
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1)
    has = np.isfinite(m)
    w = np.zeros_like(s)
    w[has] = np.exp(s[has] - m[has, None])
    w[~vis] = 0.0
    l = w.sum(axis=1)
    o = w @ values
    return m, l, o


def merge_ref(o_part, m_part, l_part, part_indptr):
    """Merge partials by log-sum-exp, per sequence, in logical order.

    o_part [N, R, H, D], m_part/l_part [N, R, H] (any float dtype); the
    partials of sequence b are rows [part_indptr[b], part_indptr[b+1]).
    M = max_i m_i; w_i = exp(m_i - M) (0 where m_i = -inf);
    L = sum_i w_i l_i; O = sum_i w_i o_i / L; LSE = M + ln L.
    A sequence whose partials are all empty gets O = 0, LSE = -inf.
    Returns (O [B, R, H, D], LSE [B, R, H]) fp64.
    """
    o_part = np.asarray(o_part, dtype=np.float64)
    m_part = np.asarray(m_part, dtype=np.float64)
    l_part = np.asarray(l_part, dtype=np.float64)
    indptr = np.asarray(part_indptr)
    B = len(indptr) - 1
    _, R, H, D = o_part.shape
    O = np.zeros((B, R, H, D))
    LSE = np.full((B, R, H), -np.inf)
    for b in range(B):
        lo, hi = int(indptr[b]), int(indptr[b + 1])
        if hi <= lo:
            continue
        m = m_part[lo:hi]                   # [n, R, H]
        M = m.max(axis=0)                   # [R, H]
        ok = np.isfinite(M)
        w = np.zeros_like(m)
        fin = np.isfinite(m)
        Mb = np.broadcast_to(M, m.shape)
        w[fin] = np.exp(m[fin] - Mb[fin])
        L = (w * l_part[lo:hi]).sum(axis=0)
        num = np.zeros((R, H, D))
        for i in range(hi - lo):
            wi = w[i]
            sel = wi > 0
            num[sel] += wi[sel, None] * o_part[lo + i][sel]
        O[b][ok] = num[ok] / L[ok][:, None]
        LSE[b][ok] = M[ok] + np.log(L[ok])
    return O, LSE


__all__ = ["SEG_FIELDS", "plan_ref", "to_f64", "alive_tokens_ref", "attention_ref",
           "decode_ref", "prefill_ref", "partial_ref", "merge_ref"]
