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
  (time = c0 + c_tok * alive tokens + c_seg * segments + c_max * the longest
  sequence's alive tokens).  Evicting a block removes its tokens, changes
  the segment count by -1, 0 or +1 depending on whether its logical
  neighbours are alive and physically adjacent, and shortens the longest
  sequence if it is taken from it: when every (sequence, KV head) pair is
  one workgroup and the pairs fill the chip, the call lasts as long as the
  longest sequence's workgroups, so tokens of shorter sequences cost the
  step almost nothing.

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
    c0 + c_tok * alive_tokens + c_seg * segments + c_max * max_seq_tokens
    (alive tokens of the batch's longest sequence)."""
    c0: float
    c_tok: float
    c_seg: float
    c_max: float = 0.0

    def predict(self, alive_tokens, segments, max_seq_tokens=0):
        return self.c0 + self.c_tok * np.asarray(alive_tokens, dtype=np.float64) + \
            self.c_seg * np.asarray(segments, dtype=np.float64) + \
            self.c_max * np.asarray(max_seq_tokens, dtype=np.float64)

    @staticmethod
    def fit(alive_tokens, segments, times_us, max_seq_tokens=None) -> "DecodeLatencyModel":
        """Least-squares fit to measured (alive tokens, segments[, longest
        sequence's alive tokens], time) points."""
        a = np.asarray(alive_tokens, dtype=np.float64)
        s = np.asarray(segments, dtype=np.float64)
        t = np.asarray(times_us, dtype=np.float64)
        cols = [np.ones_like(a), a, s]
        if max_seq_tokens is not None:
            cols.append(np.asarray(max_seq_tokens, dtype=np.float64))
        coef, *_ = np.linalg.lstsq(np.stack(cols, axis=1), t, rcond=None)
        return DecodeLatencyModel(float(coef[0]), float(coef[1]), float(coef[2]),
                                  float(coef[3]) if max_seq_tokens is not None else 0.0)


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


def alive_tokens(alive, ctx_len, block_size):
    """Alive tokens of every sequence (the last block holds ctx_len mod bs)."""
    al = np.asarray(alive)
    bs = int(block_size)
    out = np.zeros(al.shape[0], dtype=np.int64)
    for b in range(al.shape[0]):
        nb = -(-int(ctx_len[b]) // bs)
        out[b] = int(np.dot(al[b, :nb] != 0, _block_tokens(ctx_len[b], nb, bs)))
    return out


def max_seq_gain(seq_tokens, b, tokens):
    """How much the batch's longest alive-token count falls when `tokens`
    alive tokens of sequence b go: nothing unless b is the only longest
    sequence, then at most down to the second longest."""
    A = np.asarray(seq_tokens)
    top = A[b]
    if len(A) > 1:
        others = np.delete(A, b)
        second = int(others.max())
    else:
        second = 0
    if top < second or (top == second and len(A) > 1):
        return 0
    return int(min(tokens, top - second))


def _saving(model, tok, ds, max_gain):
    return model.c_tok * tok - model.c_seg * ds + model.c_max * max_gain


def eviction_scores(block_table, alive, ctx_len, block_size, hit_prob, recompute_us,
                    model: DecodeLatencyModel, alpha=1.0, beta=1.0, gamma=1.0, batch_seqs=1):
    """Keep-scores of every block (higher = keep); +inf where a block cannot be
    evicted (not alive, past the context, or the sequence's last block, which
    holds the newest token).

    score = alpha * hit_prob + beta * recompute_us - gamma * saving_us, where
    saving_us is the decode time one step saves when the block is gone,
    predicted by the latency model (tokens removed, segments changed, the
    longest sequence shortened) and shared over batch_seqs sequences per
    decode batch."""
    table = np.asarray(block_table)
    al = np.asarray(alive)
    B, mb = table.shape
    bs = int(block_size)
    seq_tok = alive_tokens(al, ctx_len, bs)
    scores = np.full((B, mb), np.inf)
    for b in range(B):
        nb = -(-int(ctx_len[b]) // bs)
        tok = _block_tokens(ctx_len[b], nb, bs)
        for l in range(nb - 1):
            if not al[b, l]:
                continue
            ds = segment_delta(table[b], al[b], l)
            gain = max_seq_gain(seq_tok, b, tok[l]) if model.c_max else 0
            scores[b, l] = alpha * hit_prob[b, l] + beta * recompute_us[b][l] - \
                gamma * _saving(model, tok[l], ds, gain) / batch_seqs
    return scores


def choose_evictions(block_table, alive, ctx_len, block_size, n_evict, hit_prob, recompute_us,
                     model: DecodeLatencyModel, alpha=1.0, beta=1.0, gamma=1.0, batch_seqs=1):
    """Evict n_evict blocks, lowest score first.  After each eviction the
    scores that changed are recomputed: the neighbours' (whether they split
    or end a segment has changed) and, with a longest-sequence term, every
    block of the sequences that were or now are among the two longest (their
    share of the longest sequence's time has moved).  Returns the new alive
    mask (uint8, same shape) and the list of evicted (b, l) in order."""
    table = np.asarray(block_table)
    al = np.array(alive, dtype=np.uint8, copy=True)
    bs = int(block_size)
    B = table.shape[0]
    seq_tok = alive_tokens(al, ctx_len, bs)
    sc = eviction_scores(table, al, ctx_len, bs, hit_prob, recompute_us, model, alpha, beta,
                         gamma, batch_seqs)
    heap = [(sc[b, l], b, l) for b, l in zip(*np.nonzero(np.isfinite(sc)))]
    heapq.heapify(heap)
    evicted = []

    def rescore(b, l):
        nb = -(-int(ctx_len[b]) // bs)
        tok = _block_tokens(ctx_len[b], nb, bs)
        ds = segment_delta(table[b], al[b], l)
        gain = max_seq_gain(seq_tok, b, tok[l]) if model.c_max else 0
        sc[b, l] = alpha * hit_prob[b, l] + beta * recompute_us[b][l] - \
            gamma * _saving(model, tok[l], ds, gain) / batch_seqs
        heapq.heappush(heap, (sc[b, l], b, l))

    def top2():
        return set(np.argsort(-seq_tok, kind="stable")[:2].tolist()) if B else set()

    while heap and len(evicted) < n_evict:
        s, b, l = heapq.heappop(heap)
        if not al[b, l] or s != sc[b, l]:
            continue  # stale entry
        before = top2() if model.c_max else set()
        al[b, l] = 0
        sc[b, l] = np.inf
        evicted.append((int(b), int(l)))
        nb = -(-int(ctx_len[b]) // bs)
        seq_tok[b] -= int(_block_tokens(ctx_len[b], nb, bs)[l])
        for nl in (l - 1, l + 1):
            if 0 <= nl < nb - 1 and al[b, nl]:
                rescore(b, nl)
        if model.c_max:
            for bb in before | top2() | {b}:
                nbb = -(-int(ctx_len[bb]) // bs)
                for ll in range(nbb - 1):
                    if al[bb, ll]:
                        rescore(bb, ll)
    return al, evicted
