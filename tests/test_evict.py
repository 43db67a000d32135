"""Kernel-aware eviction scoring (host side).

Pins: the segment-count change of evicting a block is checked against the
oracle's segment plan before and after (brute force over random layouts);
the recompute cost against a row-by-row count of visible (row, key) pairs;
the latency-model fit against exact synthetic data; and the selection
against the policy's stated behaviour (lowest score first, never the last
block, costly positions kept under the reading that the cost term adds to
the keep-score).
"""
import numpy as np
import pytest

import oracle
from kv_cache_attention_msa_amd.evict import (DecodeLatencyModel, choose_evictions,
                                              eviction_scores, recompute_cost_us, segment_delta)
from workloads import make_workload
from workloads.gen import random_small_case


def _nseg(table, alive, ctx_len, bs, b):
    segs, indptr = oracle.plan_ref(table, alive, ctx_len, bs)
    return int(indptr[b + 1] - indptr[b])


def test_segment_delta_matches_plan_brute_force():
    rng = np.random.default_rng(11)
    checked = 0
    for _ in range(300):
        table, alive, ctx_len, bs, pool = random_small_case(rng)
        for b in range(table.shape[0]):
            nb = -(-int(ctx_len[b]) // bs)
            for l in range(nb):
                if not alive[b, l]:
                    continue
                before = _nseg(table, alive, ctx_len, bs, b)
                a2 = alive.copy()
                a2[b, l] = 0
                after = _nseg(table, a2, ctx_len, bs, b)
                assert segment_delta(table[b, :nb], alive[b, :nb], l) == after - before
                checked += 1
    assert checked > 200


def _pairs_brute(alive_row, ctx_len, bs, l, mode):
    pos = np.arange(int(ctx_len))
    blk = pos // bs
    al = alive_row[blk] != 0
    al[blk == l] = True  # the block being scored is resident
    rows = pos[(blk == l)] if mode == "block" else pos[(blk >= l) & al]
    keys = pos[al]
    return int(sum(np.searchsorted(keys, r, side="right") for r in rows))


@pytest.mark.parametrize("mode", ["block", "suffix"])
def test_recompute_cost_counts_visible_pairs(mode):
    rng = np.random.default_rng(3)
    D, Hq, tf = 128, 32, 100.0
    for _ in range(20):
        bs = 16
        nb = int(rng.integers(1, 12))
        ctx = (nb - 1) * bs + int(rng.integers(1, bs + 1))
        alive = rng.integers(0, 2, size=nb).astype(np.uint8)
        cost = recompute_cost_us(alive, ctx, bs, D, Hq, tf, mode=mode)
        for l in range(nb):
            if not alive[l]:
                continue
            want = _pairs_brute(alive, ctx, bs, l, mode) * 4.0 * D * Hq / (tf * 1e12) * 1e6
            assert cost[l] == pytest.approx(want, rel=1e-12)


def test_latency_model_fit_recovers_coefficients():
    rng = np.random.default_rng(0)
    a = rng.integers(1000, 200000, size=12)
    s = rng.integers(10, 20000, size=12)
    t = 3.5 + 7.5e-4 * a + 2e-3 * s
    m = DecodeLatencyModel.fit(a, s, t)
    assert m.c0 == pytest.approx(3.5, rel=1e-6)
    assert m.c_tok == pytest.approx(7.5e-4, rel=1e-6)
    assert m.c_seg == pytest.approx(2e-3, rel=1e-5)
    assert m.predict(1000, 10) == pytest.approx(3.5 + 0.75 + 0.02)


def _setup(seed=0):
    w = make_workload(2, seed=seed, size="small", values=False)
    rng = np.random.default_rng(seed)
    hit = rng.random(w.alive.shape)
    rec = [recompute_cost_us(w.alive[b], w.ctx_len[b], 16, w.D, w.Hq, 800.0) for b in range(w.B)]
    return w, hit, rec


def test_hit_only_evicts_lowest_hit_probability_first():
    w, hit, rec = _setup()
    model = DecodeLatencyModel(0.0, 0.0, 0.0)
    n = 25
    al, ev = choose_evictions(w.block_table, w.alive, w.ctx_len, 16, n, hit, rec, model,
                              alpha=1.0, beta=0.0, gamma=0.0)
    assert len(ev) == n
    cand = [(hit[b, l], b, l) for b in range(w.B) for l in range(-(-int(w.ctx_len[b]) // 16) - 1)
            if w.alive[b, l]]
    want = sorted(cand)[:n]
    assert [(b, l) for _, b, l in want] == ev
    for b, l in ev:
        assert w.alive[b, l] == 1 and al[b, l] == 0


def test_never_evicts_dead_or_last_block():
    w, hit, rec = _setup(1)
    model = DecodeLatencyModel(1.0, 1e-3, 1e-2)
    al, ev = choose_evictions(w.block_table, w.alive, w.ctx_len, 16, 10 ** 6, hit, rec, model)
    for b in range(w.B):
        nb = -(-int(w.ctx_len[b]) // 16)
        assert al[b, nb - 1] == 1          # newest block stays
        assert not (al[b] > w.alive[b]).any()
    evictable = 0
    for b in range(w.B):
        nb = -(-int(w.ctx_len[b]) // 16)
        evictable += int(w.alive[b, :nb].astype(np.int64).sum()) - 1
    assert len(ev) == evictable


def test_costly_positions_are_kept():
    """Equal hit probabilities, cost term only: with the suffix cost, blocks
    near the end are cheapest to rebuild and go first."""
    w, _, rec = _setup(2)
    hit = np.zeros(w.alive.shape)
    model = DecodeLatencyModel(0.0, 0.0, 0.0)
    al, ev = choose_evictions(w.block_table, w.alive, w.ctx_len, 16, 12, hit, rec, model,
                              alpha=0.0, beta=1.0, gamma=0.0)
    costs = [rec[b][l] for b, l in ev]
    assert costs == sorted(costs)
    kept = [rec[b][l] for b in range(w.B) for l in range(-(-int(w.ctx_len[b]) // 16) - 1)
            if al[b, l]]
    assert max(costs) <= min(kept)


def test_segment_cost_prefers_ending_segments_to_splitting_them():
    # one sequence, blocks 0..7 physically contiguous except a break after 3
    table = np.array([[10, 11, 12, 13, 30, 31, 32, 33]], dtype=np.int32)
    alive = np.ones((1, 8), dtype=np.uint8)
    ctx = np.array([8 * 16], dtype=np.int32)
    hit = np.zeros((1, 8))
    rec = [np.zeros(8)]
    model = DecodeLatencyModel(0.0, 0.0, 1.0)  # only segments cost decode time
    sc = eviction_scores(table, alive, ctx, 16, hit, rec, model, alpha=0, beta=0, gamma=1)
    # ends of a run (0, 3, 4) keep the count; interior blocks (1, 2, 5, 6) split it
    assert sc[0, 1] > sc[0, 0] and sc[0, 2] > sc[0, 3] and sc[0, 5] > sc[0, 4]
    al, ev = choose_evictions(table, alive, ctx, 16, 2, hit, rec, model, alpha=0, beta=0, gamma=1)
    # the greedy picks run ends; after evicting 0, block 1 becomes a run end
    for b, l in ev:
        assert l in (0, 1, 3, 4, 2)
    segs_after = _nseg(table, al, ctx, 16, 0)
    assert segs_after <= 2


def test_latency_model_fit_recovers_longest_sequence_term():
    rng = np.random.default_rng(1)
    a = rng.integers(1000, 200000, size=16)
    s = rng.integers(10, 20000, size=16)
    mx = rng.integers(100, 8000, size=16)
    t = 2.0 + 1e-4 * a + 5e-4 * s + 1.8e-2 * mx
    m = DecodeLatencyModel.fit(a, s, t, max_seq_tokens=mx)
    for got, want in ((m.c0, 2.0), (m.c_tok, 1e-4), (m.c_seg, 5e-4), (m.c_max, 1.8e-2)):
        assert got == pytest.approx(want, rel=1e-5)
    assert m.predict(a[0], s[0], mx[0]) == pytest.approx(t[0], rel=1e-9)
    # without the column the model has no longest-sequence term
    assert DecodeLatencyModel.fit(a, s, t).c_max == 0.0


def test_max_seq_gain_cases():
    from kv_cache_attention_msa_amd.evict import max_seq_gain
    A = np.array([100, 300, 250, 40])
    assert max_seq_gain(A, 1, 16) == 16        # the longest, far ahead
    assert max_seq_gain(A, 1, 80) == 50        # only down to the second longest
    assert max_seq_gain(A, 2, 16) == 0         # not the longest
    assert max_seq_gain(np.array([300, 300, 10]), 0, 16) == 0   # a tie: the other still lasts
    assert max_seq_gain(np.array([77]), 0, 16) == 16            # a lone sequence


def test_longest_sequence_term_levels_the_batch():
    """With only the longest-sequence term (and a tiny per-token term to order
    ties), the scorer takes blocks from whichever sequence is longest: the
    batch's longest alive-token count after n evictions is within one block
    of the best any choice of n blocks can reach (water-filling)."""
    from kv_cache_attention_msa_amd.evict import alive_tokens
    rng = np.random.default_rng(5)
    B, nb, bs = 6, 40, 16
    table = np.arange(B * nb, dtype=np.int32).reshape(B, nb)
    alive = np.ones((B, nb), np.uint8)
    ctx = rng.integers(10 * bs, nb * bs + 1, size=B).astype(np.int32)
    for b in range(B):
        alive[b, -(-int(ctx[b]) // bs):] = 0
    hit = rng.random((B, nb))
    rec = [np.zeros(nb) for _ in range(B)]
    model = DecodeLatencyModel(0.0, 1e-6, 0.0, c_max=1.0)
    n = 40
    al, ev = choose_evictions(table, alive, ctx, bs, n, hit, rec, model, alpha=0.0, beta=0.0, gamma=1.0)
    assert len(ev) == n
    got = alive_tokens(al, ctx, bs).max()
    # best reachable: lower the longest sequences by whole blocks (never a
    # sequence's last block), n blocks in all
    A = alive_tokens(alive, ctx, bs)
    full = [int(-(-int(ctx[b]) // bs)) - 1 for b in range(B)]  # evictable blocks each
    best = None
    for level in range(0, int(A.max()) + 1, 1):
        need = sum(max(0, -(-(int(A[b]) - level) // bs)) for b in range(B))
        if need <= n and all(-(-(int(A[b]) - level) // bs) <= full[b] for b in range(B) if A[b] > level):
            best = level
            break
    assert best is not None and got <= best + bs
