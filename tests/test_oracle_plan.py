"""Pins for the oracle's segment plan (row a1).

The plan is `split_into_contiguous_segments` of P1 (AsymCache explainer,
section "Core method 1: MSA", pseudocode and the paragraph after it): alive
blocks cut into runs by physical-address contiguity, every eviction hole
breaking a run.  These tests fix the oracle against things other than itself:

* brute force: every partition of a sequence's alive blocks into groups is
  enumerated; exactly one is made of contiguous groups that no neighbouring
  pair could be joined across, and it must equal the oracle's plan;
* a hand-worked example (tests/golden/plan_example_p.json);
* characterising properties (cover, contiguity, maximality, token counts by
  direct counting) on hypothesis-drawn inputs;
* edge cases: empty sequences, all evicted, stale/garbage ids in dead
  entries, partial last blocks, descending ids.
"""
import itertools
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import plan_ref
from workloads import random_small_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tokens_in_block(l, bs, ctx):
    # count positions of logical block l that exist (< ctx), one by one
    return sum(1 for p in range(l * bs, (l + 1) * bs) if p < ctx)


def _continues(a, b):
    (l0, p0), (l1, p1) = a, b
    return l1 == l0 + 1 and p1 == p0 + 1


def brute_force_plan(table, alive, ctx_len, bs):
    """Enumerate all partitions of each sequence's alive blocks; return the
    unique one whose groups are contiguous and pairwise non-joinable."""
    recs, indptr = [], [0]
    for b in range(table.shape[0]):
        ctx = int(ctx_len[b])
        nb = -(-ctx // bs)
        items = [(l, int(table[b, l])) for l in range(nb) if alive[b, l]]
        n = len(items)
        found = []
        for cuts in itertools.product([0, 1], repeat=max(0, n - 1)):
            groups, cur = [], [items[0]] if n else []
            for i in range(1, n):
                if cuts[i - 1]:
                    groups.append(cur)
                    cur = [items[i]]
                else:
                    cur.append(items[i])
            if n:
                groups.append(cur)
            contiguous = all(_continues(g[i], g[i + 1]) for g in groups for i in range(len(g) - 1))
            maximal = all(not _continues(groups[i][-1], groups[i + 1][0]) for i in range(len(groups) - 1))
            if contiguous and maximal:
                found.append(groups)
        assert len(found) == 1, "the plan must be unique"
        start = 0
        for g in found[0]:
            ntok = sum(_tokens_in_block(l, bs, ctx) for l, _ in g)
            recs.append([b, g[0][0], g[0][1], len(g), ntok, start])
            start += ntok
        indptr.append(len(recs))
    return np.array(recs, dtype=np.int32).reshape(-1, 6), np.array(indptr, dtype=np.int32)


def check_plan_properties(table, alive, ctx_len, bs, segs, indptr):
    """Characterisation of the plan, stated without the oracle's algorithm."""
    B = table.shape[0]
    assert indptr[0] == 0 and len(indptr) == B + 1
    assert np.all(np.diff(indptr) >= 0) and indptr[-1] == len(segs)
    for b in range(B):
        ctx = int(ctx_len[b])
        nb = -(-ctx // bs)
        want = {l for l in range(nb) if alive[b, l]}
        rs = segs[indptr[b]:indptr[b + 1]]
        covered = []
        start = 0
        for i, (s, lb, pb, n, ntok, ats) in enumerate(rs):
            assert s == b and n >= 1
            for j in range(n):
                assert alive[b, lb + j]
                assert table[b, lb + j] == pb + j          # physically consecutive
                covered.append(lb + j)
            assert ntok == sum(_tokens_in_block(lb + j, bs, ctx) for j in range(n))
            assert ats == start
            start += ntok
            if i + 1 < len(rs):
                nlb, npb = rs[i + 1][1], rs[i + 1][2]
                assert nlb > lb + n - 1                    # logical order
                # maximal: the next record could not have been appended
                assert not (nlb == lb + n and npb == pb + n)
        assert covered == sorted(want)
        assert start == sum(_tokens_in_block(l, bs, ctx) for l in want)


def test_worked_example_p():
    with open(os.path.join(GOLDEN, "plan_example_p.json")) as f:
        ex = json.load(f)
    table = np.array(ex["block_table"], dtype=np.int32)
    alive = np.array(ex["alive"], dtype=np.uint8)
    ctx = np.array(ex["ctx_len"], dtype=np.int32)
    segs, indptr = plan_ref(table, alive, ctx, ex["block_size"])
    assert segs.tolist() == ex["segs"]
    assert indptr.tolist() == ex["seg_indptr"]


@pytest.mark.parametrize("seed", range(40))
def test_brute_force_random(seed):
    rng = np.random.default_rng(1000 + seed)
    table, alive, ctx, bs, _ = random_small_case(rng, max_nb=9)
    segs, indptr = plan_ref(table, alive, ctx, bs)
    bs_segs, bs_indptr = brute_force_plan(table, alive, ctx, bs)
    assert segs.tolist() == bs_segs.tolist()
    assert indptr.tolist() == bs_indptr.tolist()


LAYOUTS = {
    "ascending": lambda nb: np.arange(3, 3 + nb),
    "descending": lambda nb: np.arange(40, 40 - nb, -1),
    "pairs": lambda nb: np.array([10 + 2 * (l // 2) * 3 + (l % 2) for l in range(nb)]),
    "permuted": lambda nb: np.random.default_rng(nb).permutation(64)[:nb],
    "adjacent_across_hole": lambda nb: np.array([20 + l - (1 if l >= 2 else 0) for l in range(nb)]),
}


@pytest.mark.parametrize("layout", sorted(LAYOUTS))
@pytest.mark.parametrize("bs", [1, 3, 16])
def test_exhaustive_alive_masks(layout, bs):
    """All 2^nb alive masks for nb <= 6, each against brute force."""
    for nb in range(1, 7):
        ids = LAYOUTS[layout](nb).astype(np.int32)
        for ctx in {(nb - 1) * bs + 1, nb * bs}:
            for mask in itertools.product([0, 1], repeat=nb):
                table = ids[None, :].copy()
                alive = np.array(mask, dtype=np.uint8)[None, :]
                ctx_len = np.array([ctx], dtype=np.int32)
                segs, indptr = plan_ref(table, alive, ctx_len, bs)
                bsegs, bindptr = brute_force_plan(table, alive, ctx_len, bs)
                assert segs.tolist() == bsegs.tolist(), (layout, bs, nb, mask)
                assert indptr.tolist() == bindptr.tolist()


def test_hole_breaks_even_if_physically_adjacent():
    # logical 0,1 alive at phys 4,5; logical 2 evicted; logical 3 at phys 6.
    table = np.array([[4, 5, 99, 6]], dtype=np.int32)
    alive = np.array([[1, 1, 0, 1]], dtype=np.uint8)
    segs, indptr = plan_ref(table, alive, np.array([64], np.int32), 16)
    assert segs.tolist() == [[0, 0, 4, 2, 32, 0], [0, 3, 6, 1, 16, 32]]


def test_dead_entries_are_ignored():
    rng = np.random.default_rng(5)
    table, alive, ctx, bs, pool = random_small_case(rng, B=3, max_nb=8)
    a = plan_ref(table, alive, ctx, bs)
    garbage = table.copy()
    garbage[alive == 0] = rng.integers(-(2 ** 31), 2 ** 31 - 1, size=int((alive == 0).sum()))
    b = plan_ref(garbage, alive, ctx, bs)
    assert a[0].tolist() == b[0].tolist() and a[1].tolist() == b[1].tolist()


def test_empty_and_degenerate():
    # zero-length sequence, all evicted, single token
    table = np.array([[0, 1], [2, 3], [4, -1]], dtype=np.int32)
    alive = np.array([[1, 1], [0, 0], [1, 0]], dtype=np.uint8)
    ctx = np.array([0, 32, 1], dtype=np.int32)
    segs, indptr = plan_ref(table, alive, ctx, 16)
    assert indptr.tolist() == [0, 0, 0, 1]
    assert segs.tolist() == [[2, 0, 4, 1, 1, 0]]
    # alive flags beyond ctx_len are ignored
    alive2 = np.array([[1, 1], [0, 0], [1, 1]], dtype=np.uint8)
    segs2, _ = plan_ref(table, alive2, ctx, 16)
    assert segs2.tolist() == segs.tolist()


@settings(max_examples=150, deadline=None)
@given(seed=st.integers(0, 2 ** 31 - 1), nb=st.integers(1, 48), bs=st.sampled_from([1, 2, 16]),
       p_alive=st.floats(0.0, 1.0), p_adjacent=st.floats(0.0, 1.0))
def test_properties_hypothesis(seed, nb, bs, p_alive, p_adjacent):
    rng = np.random.default_rng(seed)
    B = 3
    table = np.full((B, nb), -1, dtype=np.int32)
    for b in range(B):
        cur = int(rng.integers(0, 1000))
        for l in range(nb):
            cur = cur + 1 if rng.random() < p_adjacent else int(rng.integers(0, 100000))
            table[b, l] = cur
    alive = (rng.random((B, nb)) < p_alive).astype(np.uint8)
    ctx = np.array([int(rng.integers(0, nb * bs + 1)) for _ in range(B)], dtype=np.int32)
    segs, indptr = plan_ref(table, alive, ctx, bs)
    check_plan_properties(table, alive, ctx, bs, segs, indptr)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_workload_plans_are_valid(cfg):
    from workloads import make_workload
    w = make_workload(cfg, seed=0, size="small")
    segs, indptr = plan_ref(w.block_table, w.alive, w.ctx_len, w.block_size)
    check_plan_properties(w.block_table, w.alive, w.ctx_len, w.block_size, segs, indptr)
    if cfg == 5:
        # alive blocks at independent random slots: nearly one segment per block
        assert len(segs) >= 0.9 * w.meta["alive_blocks"]
