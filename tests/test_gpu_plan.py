"""GPU parity of the segment plan (row a1): byte-equal to the oracle's plan.

Runs through the C ABI (via the thin binding) on the five workload families
at full size and three seeds, a fuzz over tiny random layouts and block
sizes, the hand-worked example, and the data-error paths (out-of-range
physical ids, too small a capacity, ctx_len out of range).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import kv_cache_attention_msa_amd as msa
from workloads import make_workload, random_small_case
from workloads.device import tensor

pytestmark = pytest.mark.gpu
DEV = "cuda"
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def gpu_plan(table, alive, ctx, bs, P, cap=None):
    t = tensor(np.ascontiguousarray(table, dtype=np.int32), DEV)
    a = tensor(np.ascontiguousarray(alive, dtype=np.uint8), DEV)
    c = tensor(np.ascontiguousarray(ctx, dtype=np.int32), DEV)
    segs, indptr, err = msa.msa_plan_segments(t, a, c, bs, P, seg_capacity=cap)
    torch.cuda.synchronize()
    indptr = indptr.cpu().numpy()
    n = int(indptr[-1])
    return segs[:n].cpu().numpy(), indptr, int(err.cpu().item())


def assert_plan_equal(table, alive, ctx, bs, P):
    segs, indptr, err = gpu_plan(table, alive, ctx, bs, P)
    rs, ri = oracle.plan_ref(table, alive, ctx, bs)
    assert err == 0
    assert indptr.tolist() == ri.tolist()
    assert segs.tobytes() == rs.astype(np.int32).tobytes()


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_plan_workloads_full(cfg, seed):
    w = make_workload(cfg, seed=seed, values=False)
    assert_plan_equal(w.block_table, w.alive, w.ctx_len, w.block_size, w.num_phys_blocks)


@pytest.mark.parametrize("B", [1024, 1025, 3000])
def test_plan_batches_around_the_scan_launch(B):
    # up to 1024 sequences each write workgroup sums the counts before its
    # own; above that a one-workgroup scan launch computes the offsets
    w = make_workload(2, seed=B, B=B, ctx=16 * 24 - 5, values=False)
    assert_plan_equal(w.block_table, w.alive, w.ctx_len, w.block_size, w.num_phys_blocks)


def test_plan_fuzz():
    rng = np.random.default_rng(123)
    for _ in range(150):
        table, alive, ctx, bs, pool = random_small_case(rng, max_nb=int(rng.integers(1, 40)))
        assert_plan_equal(table, alive, ctx, bs, pool)


def test_plan_long_rows_cross_chunks():
    # more than one 1024-block chunk per sequence, runs crossing chunk edges
    rng = np.random.default_rng(7)
    nb = 3000
    B = 3
    table = np.zeros((B, nb), np.int32)
    for b in range(B):
        ids = np.arange(nb) + 5000 * b
        brk = rng.random(nb) < 0.05
        ids = ids + np.cumsum(brk) * 3
        table[b] = ids
    alive = (rng.random((B, nb)) < 0.9).astype(np.uint8)
    alive[:, 1020:1030] = 1
    ctx = np.array([nb * 16, nb * 16 - 7, 1024 * 16 + 1], np.int32)
    assert_plan_equal(table, alive, ctx, 16, 20000)


def test_plan_worked_example():
    ex = json.load(open(os.path.join(GOLDEN, "plan_example_p.json")))
    segs, indptr, err = gpu_plan(np.array(ex["block_table"]), np.array(ex["alive"]),
                                 np.array(ex["ctx_len"]), ex["block_size"], 16)
    assert err == 0
    assert segs.tolist() == ex["segs"] and indptr.tolist() == ex["seg_indptr"]


def test_plan_out_of_range_ids_are_flagged_and_dropped():
    rng = np.random.default_rng(3)
    table, alive, ctx, bs, pool = random_small_case(rng, B=3, max_nb=12, allow_stale=False)
    bad = table.copy()
    live = np.argwhere(alive == 1)
    live = [(b, l) for b, l in live if l * bs < ctx[b]]
    assert len(live) >= 2
    (b0, l0), (b1, l1) = live[0], live[-1]
    bad[b0, l0] = -3
    bad[b1, l1] = pool + 2
    segs, indptr, err = gpu_plan(bad, alive, ctx, bs, pool)
    assert err & msa.MSA_DEVERR_PHYS_RANGE
    a2 = alive.copy()
    a2[b0, l0] = 0
    a2[b1, l1] = 0
    rs, ri = oracle.plan_ref(bad, a2, ctx, bs)
    assert indptr.tolist() == ri.tolist() and segs.tobytes() == rs.tobytes()


def test_plan_capacity_overflow_is_flagged():
    w = make_workload(2, seed=0, size="small", values=False)
    rs, ri = oracle.plan_ref(w.block_table, w.alive, w.ctx_len, w.block_size)
    cap = int(ri[-1]) - 5
    segs, indptr, err = gpu_plan(w.block_table, w.alive, w.ctx_len, w.block_size,
                                 w.num_phys_blocks, cap=cap)
    assert err & msa.MSA_DEVERR_CAPACITY
    assert indptr.tolist() == np.minimum(ri, cap).tolist()
    assert segs[:cap].tobytes() == rs[:cap].tobytes()


def test_plan_ctx_out_of_range_is_flagged_and_clamped():
    table = np.arange(8, dtype=np.int32).reshape(2, 4)
    alive = np.ones((2, 4), np.uint8)
    ctx = np.array([4 * 16 + 9, -5], np.int32)
    segs, indptr, err = gpu_plan(table, alive, ctx, 16, 8)
    assert err & msa.MSA_DEVERR_CTX_RANGE
    rs, ri = oracle.plan_ref(table, alive, np.array([64, 0], np.int32), 16)
    assert indptr.tolist() == ri.tolist() and segs.tobytes() == rs.tobytes()


def test_plan_empty_sequences():
    table = np.array([[1, 2, 3], [4, 5, 6], [7, 8, 9]], np.int32)
    alive = np.array([[0, 0, 0], [1, 1, 1], [1, 0, 1]], np.uint8)
    ctx = np.array([48, 0, 33], np.int32)
    assert_plan_equal(table, alive, ctx, 16, 10)
