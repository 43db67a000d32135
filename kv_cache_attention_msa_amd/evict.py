"""Kernel-aware eviction scoring for an MSA-served KV cache (host side).

The pages' eviction policy (P1, "Core method 2: position-aware + hit-rate
joint eviction") scores every resident block by how likely it is to be hit
again and by what it would cost to recompute it if it were evicted and then
needed, with coefficients tuned to the batch and the hardware profile, and
evicts the lowest-scoring blocks first.  This module builds that policy
around the kernels of this library:

* hit probability: supplied by the caller (this library sees no traces);
* position-aware recompute cost: the time our chunked-prefill kernel would
  need to rebuild the block, from its measured throughput;
* kernel cost: what keeping the block costs every decode step, from a
  latency model of our decode kernel fitted to measurements
  (time = c0 + c_tok * alive tokens + c_seg * segments).  Evicting a block
  removes its tokens and changes the segment count by -1, 0 or +1 depending
  on whether its logical neighbours are alive and physically adjacent.

Readings of the pages (they state the formula with a minus sign on the cost
term and, in the same passage, say that costly positions are kept; the
cost's dependence on position is described both as "re-prefill up to the
position" and as "cheap near the end"):

* the score is alpha*hit + beta*recompute_cost + gamma*decode_saving_loss,
  lowest evicted first, so that costly-to-recompute blocks are kept;
* recompute cost "suffix" (default): rebuilding block l means prefilling the
  positions from its first token to the end of the sequence over their
  visible keys, so blocks near the end are cheap and early/middle blocks are
  expensive; "block" is the alternative reading (prefilling only the block's
  own tokens over the keys before it).

Nothing here runs on the GPU; it reads block tables and alive masks (numpy)
and returns eviction masks.  The fitted latency model comes from timings of
msa_decode taken by the caller (bench.py --latency-model does this).
"""
from __future__ import annotations

import heapq
from dataclasses import dataclass

import numpy as np


@dataclass
class DecodeLatencyModel:
    """Predicted msa_decode time (microseconds) of one batch:
    c0 + c_tok * alive_tokens + c_seg * segments."""
    c0: float
    c_tok: float
    c_seg: float

    def predict(self, alive_tokens, segments):
        return self.c0 + self.c_tok * np.asarray(alive_tokens, dtype=np.float64) + \
            self.c_seg * np.asarray(segments, dtype=np.float64)

    @staticmethod
    def fit(alive_tokens, segments, times_us) -> "DecodeLatencyModel":
        """Least-squares fit to measured (alive tokens, segments, time) triples."""
        a = np.asarray(alive_tokens, dtype=np.float64)
        s = np.asarray(segments, dtype=np.float64)
        t = np.asarray(times_us, dtype=np.float64)
        X = np.stack([np.ones_like(a), a, s], axis=1)
        coef, *_ = np.linalg.lstsq(X, t, rcond=None)
        return DecodeLatencyModel(float(coef[0]), float(coef[1]), float(coef[2]))


def _block_tokens(ctx_len, nb, bs):
    tok = np.full(nb, bs, dtype=np.int64)
    if nb:
        tok[-1] = int(ctx_len) - (nb - 1) * bs
    return tok


def segment_delta(table_row, alive_row, l):
    """Change in the sequence's segment count if alive block l is evicted:
    +1 when both logical neighbours continue it physically (the segment
    splits), -1 when neither does (a one-block segment vanishes), else 0."""
    nb = len(alive_row)
    left = l > 0 and alive_row[l - 1] and table_row[l - 1] + 1 == table_row[l]
    right = l + 1 < nb and alive_row[l + 1] and table_row[l] + 1 == table_row[l + 1]
    return int(left) + int(right) - 1


def recompute_cost_us(alive_row, ctx_len, bs, D, Hq, prefill_tflops, mode="suffix"):
    """Per-block time (us) to rebuild an evicted block with the chunked-prefill
    kernel running at prefill_tflops: 4*D*Hq flops per visible (row, key).

    mode "suffix": rows from the block's first position to the end of the
    sequence; "block": only the block's own rows.  Visible keys of a row are
    the alive tokens at or before it (the block itself counted as alive)."""
    nb = len(alive_row)
    tok = _block_tokens(ctx_len, nb, bs)
    alive_tok = np.where(alive_row[:nb] != 0, tok, 0)
    before = np.concatenate([[0], np.cumsum(alive_tok)[:-1]])  # alive tokens before block l
    # rows of block l see `before[l]` earlier keys plus a causal triangle of their own
    own = tok * before + tok * (tok + 1) // 2
    if mode == "block":
        pairs = own
    elif mode == "suffix":
        # every row after block l must be rebuilt as well: its pairs are its
        # full visible-key count, which the block's eviction does not change
        full_rows = alive_tok * before + alive_tok * (alive_tok + 1) // 2  # alive blocks' own pairs
        after = np.concatenate([np.cumsum(full_rows[::-1])[::-1][1:], [0]])
        pairs = own + after
    else:
        raise ValueError(mode)
    return pairs.astype(np.float64) * 4.0 * D * Hq / (prefill_tflops * 1e12) * 1e6


def eviction_scores(block_table, alive, ctx_len, block_size, hit_prob, recompute_us,
                    model: DecodeLatencyModel, alpha=1.0, beta=1.0, gamma=1.0, batch_seqs=1):
    """Keep-scores of every block (higher = keep); +inf where a block cannot be
    evicted (not alive, past the context, or the sequence's last block, which
    holds the newest token).

    score = alpha * hit_prob + beta * recompute_us - gamma * saving_us, where
    saving_us is the decode time one step saves when the block is gone,
    predicted by the latency model (tokens removed, segments changed) and
    shared over batch_seqs sequences per decode batch."""
    table = np.asarray(block_table)
    al = np.asarray(alive)
    B, mb = table.shape
    bs = int(block_size)
    scores = np.full((B, mb), np.inf)
    for b in range(B):
        nb = -(-int(ctx_len[b]) // bs)
        tok = _block_tokens(ctx_len[b], nb, bs)
        for l in range(nb - 1):
            if not al[b, l]:
                continue
            ds = segment_delta(table[b], al[b], l)
            saving = model.c_tok * tok[l] - model.c_seg * ds
            scores[b, l] = alpha * hit_prob[b, l] + beta * recompute_us[b][l] - gamma * saving / batch_seqs
    return scores


def choose_evictions(block_table, alive, ctx_len, block_size, n_evict, hit_prob, recompute_us,
                     model: DecodeLatencyModel, alpha=1.0, beta=1.0, gamma=1.0, batch_seqs=1):
    """Evict n_evict blocks, lowest score first.  After each eviction the
    neighbours' segment deltas (and so their scores) are recomputed, since
    whether they split or end a segment has changed.  Returns the new alive
    mask (uint8, same shape) and the list of evicted (b, l) in order."""
    table = np.asarray(block_table)
    al = np.array(alive, dtype=np.uint8, copy=True)
    bs = int(block_size)
    sc = eviction_scores(table, al, ctx_len, bs, hit_prob, recompute_us, model, alpha, beta,
                         gamma, batch_seqs)
    heap = [(sc[b, l], b, l) for b, l in zip(*np.nonzero(np.isfinite(sc)))]
    heapq.heapify(heap)
    evicted = []
    while heap and len(evicted) < n_evict:
        s, b, l = heapq.heappop(heap)
        if not al[b, l] or s != sc[b, l]:
            continue  # stale entry
        al[b, l] = 0
        sc[b, l] = np.inf
        evicted.append((int(b), int(l)))
        nb = -(-int(ctx_len[b]) // bs)
        tok = _block_tokens(ctx_len[b], nb, bs)
        for nl in (l - 1, l + 1):
            if 0 <= nl < nb - 1 and al[b, nl]:
                ds = segment_delta(table[b], al[b], nl)
                saving = model.c_tok * tok[nl] - model.c_seg * ds
                sc[b, nl] = alpha * hit_prob[b, nl] + beta * recompute_us[b][nl] - gamma * saving / batch_seqs
                heapq.heappush(heap, (sc[b, nl], b, nl))
    return al, evicted
