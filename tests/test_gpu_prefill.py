"""GPU parity of MSA chunked prefill (rows a2, a4, a5) against the fp64 oracle.

bf16 inputs, bf16 MFMA with fp32 accumulation, softmax weights rounded to
bf16 for PV: max-abs-error <= 2e-2 on O and LSE, element by element.  Covers
several 64-key tiles and ragged tails (partial last block, chunk lengths
that are not a multiple of the 32-row tile), a chunk in the middle of the
context (later alive blocks must be masked by logical position), every GQA
group size, forced key splits merged by log-sum-exp, rows with no visible
key, the full-size prefill workload on sampled rows and heads, and the
recompute workload (an evicted middle range rebuilt as a chunk in fresh pool
slots, with alive blocks after it that only the causal mask hides), the
256-block key-chunk boundary, and the maximum batch the grid takes.
"""
import numpy as np
import pytest
import torch

import oracle
import kv_cache_attention_msa_amd as msa
from workloads import make_workload
from workloads.device import to_device, tensor, from_device

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 2e-2


def run_prefill(w, split_blocks=0, q_pos0=None):
    d = to_device(w, DEV)
    if q_pos0 is not None:
        d["q_pos0"] = tensor(np.asarray(q_pos0, dtype=np.int32), DEV)
    segs, indptr, err = msa.msa_plan_segments(d["block_table"], d["alive"], d["ctx_len"],
                                              w.block_size, w.num_phys_blocks)
    # the plan's error word also collects the prefill's (none expected)
    out, lse = msa.msa_prefill_chunk(d["q"], d["q_pos0"], d["k_pool"], d["v_pool"], segs, indptr,
                                     max_ctx_len=max(1, int(w.ctx_len.max())), scale=w.scale,
                                     split_blocks=split_blocks, dev_error=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    return from_device(out), lse.cpu().numpy().astype(np.float64)


def check(w, O, L, q_pos0=None, seqs=None, heads=None, rows=None):
    qp = w.q_pos0 if q_pos0 is None else np.asarray(q_pos0)
    Or, Lr = oracle.prefill_ref(w.q, qp, w.k_pool, w.v_pool, w.block_table, w.alive, w.ctx_len,
                                w.block_size, w.scale, seqs=seqs, heads=heads, rows=rows)
    sel = ~np.isnan(Lr)
    fin = sel & np.isfinite(Lr)
    e_o = float(np.max(np.abs(O - Or)[~np.isnan(Or)]))
    e_l = float(np.max(np.abs(L[fin] - Lr[fin]))) if fin.any() else 0.0
    empty = sel & np.isneginf(Lr)
    assert np.all(np.isneginf(L[empty]))
    assert e_o <= TOL, f"max |O - ref| = {e_o}"
    assert e_l <= TOL, f"max |LSE - ref| = {e_l}"
    return e_o, e_l


def test_prefill_available():
    assert msa.prefill_available()


@pytest.mark.parametrize("split_blocks", [0, 16, 40])
def test_prefill_small(split_blocks):
    w = make_workload(3, seed=0, size="small")
    O, L = run_prefill(w, split_blocks)
    check(w, O, L)


def test_prefill_ragged_chunk_and_seeds():
    for seed, C in ((1, 70), (2, 33), (3, 1)):
        w = make_workload(3, seed=seed, size="small", C=C)
        O, L = run_prefill(w)
        check(w, O, L)


@pytest.mark.parametrize("G", [1, 2, 8])
def test_prefill_group_sizes(G):
    w = make_workload(3, seed=4, size="small", Hq=2 * G, Hkv=2, C=80, cached=512)
    O, L = run_prefill(w, 0)
    check(w, O, L)
    O, L = run_prefill(w, 16)
    check(w, O, L)


def test_prefill_mid_context_chunk():
    """A chunk whose rows sit in the middle of the context: alive blocks
    after them (and inside the chunk) are hidden by the causal mask."""
    w = make_workload(3, seed=5, size="small", C=96)
    q_pos0 = [300, 517]
    O, L = run_prefill(w, 0, q_pos0=q_pos0)
    check(w, O, L, q_pos0=q_pos0)
    O, L = run_prefill(w, 16, q_pos0=q_pos0)
    check(w, O, L, q_pos0=q_pos0)


def test_prefill_rows_without_visible_keys():
    w = make_workload(3, seed=6, size="small", C=64)
    w.alive[0, :4] = 0                # the first 64 positions are evicted
    q_pos0 = [0, 100]                 # rows 0..63 of sequence 0 see nothing
    O, L = run_prefill(w, 0, q_pos0=q_pos0)
    assert np.all(O[0, :64] == 0) and np.all(np.isneginf(L[0, :64]))
    check(w, O, L, q_pos0=q_pos0)


def test_prefill_determinism():
    w = make_workload(3, seed=7, size="small")
    O1, L1 = run_prefill(w, 16)
    O2, L2 = run_prefill(w, 16)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_prefill_determinism_full():
    """Full-size chunk, three calls: identical bits every time (no tile stage
    may be rewritten by DMA while a wavefront still reads it)."""
    w = make_workload(3, seed=0)
    O1, L1 = run_prefill(w)
    for _ in range(2):
        O2, L2 = run_prefill(w)
        assert np.array_equal(O1, O2) and np.array_equal(L1, L2, equal_nan=True)


def test_prefill_full_sampled():
    w = make_workload(3, seed=0)
    O, L = run_prefill(w)
    rng = np.random.default_rng(3)
    rows = np.sort(np.concatenate([[0, 31, 32, 255, 256, 480, 511], rng.choice(512, 9, replace=False)]))
    heads = sorted(rng.choice(w.Hq, size=5, replace=False).tolist())
    check(w, O, L, seqs=[0, 3], heads=heads, rows=rows)


def test_prefill_full_forced_split_sampled():
    """Full-size chunk with the key stream cut into splits of 128 blocks
    (five per sequence, 1280 workgroups in five waves over the CUs): the
    ping-pong kernel writes partials and the merge stitches them."""
    w = make_workload(3, seed=1)
    O, L = run_prefill(w, split_blocks=128)
    rng = np.random.default_rng(5)
    rows = np.sort(np.concatenate([[0, 63, 64, 300, 511], rng.choice(512, 7, replace=False)]))
    heads = sorted(rng.choice(w.Hq, size=4, replace=False).tolist())
    check(w, O, L, seqs=[1, 2], heads=heads, rows=rows)


@pytest.mark.parametrize("B,cached,C,mean_alive,split_blocks", [
    (1, 3584, 512, 1e9, 4096),   # 256 blocks: exactly one key chunk
    (1, 3600, 512, 1e9, 4096),   # 257 blocks: a second chunk of one block
    (1, 7680, 512, 1e9, 4096),   # 512 blocks: two full chunks
    (2, 20480, 128, 16.0, 4096),  # ~1100 blocks with evictions: five chunks
    (2, 20480, 128, 16.0, 700),   # splits of <= 700 blocks: three chunks per split
])
def test_prefill_key_chunk_boundaries(B, cached, C, mean_alive, split_blocks):
    """The kernel expands a split's alive blocks 256 at a time and restarts
    its tile pipeline for each such key chunk; sequences at and just past
    the boundary, and long ones spanning several chunks (with and without
    splits), against the oracle on sampled rows and heads."""
    w = make_workload(3, seed=2, B=B, cached=cached, C=C, mean_alive=mean_alive)
    O, L = run_prefill(w, split_blocks=split_blocks)
    rng = np.random.default_rng(7)
    rows = np.sort(np.unique(np.concatenate([[0, 1, C // 2, C - 1], rng.choice(C, 6, replace=False)])))
    heads = sorted(rng.choice(w.Hq, size=4, replace=False).tolist())
    check(w, O, L, heads=heads, rows=rows)


@pytest.mark.parametrize("size,split_blocks", [("small", 0), ("small", 16), ("full", 0)])
def test_prefill_head_major_layout(size, split_blocks):
    """Pools in head-major blocks [P, Hkv, 16, D] (msa_prefill_chunk_ex):
    bitwise the same O and LSE as the token-major layout on the same values,
    and the oracle agrees."""
    w = make_workload(3, seed=4, size=size)
    d = to_device(w, DEV)
    segs, indptr, err = msa.msa_plan_segments(d["block_table"], d["alive"], d["ctx_len"],
                                              w.block_size, w.num_phys_blocks)
    outs = []
    for layout in ("NHD", "HND"):
        k, v = d["k_pool"], d["v_pool"]
        if layout == "HND":
            k, v = k.permute(0, 2, 1, 3).contiguous(), v.permute(0, 2, 1, 3).contiguous()
        outs.append(msa.msa_prefill_chunk(d["q"], d["q_pos0"], k, v, segs, indptr,
                                          max_ctx_len=int(w.ctx_len.max()), scale=w.scale,
                                          split_blocks=split_blocks, kv_layout=layout))
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    (o_n, l_n), (o_h, l_h) = outs
    assert torch.equal(o_n, o_h) and torch.equal(l_n, l_h)
    O, L = from_device(o_h), l_h.cpu().numpy().astype(np.float64)
    if size == "small":
        check(w, O, L)
    else:
        check(w, O, L, seqs=[1], heads=[0, 13, 31], rows=np.array([0, 100, 255, 256, 511]))


def test_prefill_max_batch():
    """65535 sequences (the most the grid takes without a key split), each
    a 4-row chunk (a partial block) after two cached blocks; odd sequences
    have their second cached block evicted, so they carry two segments.
    Sequences b and b + 1000 share their physical blocks (as shared prefixes
    do), which keeps the pool small."""
    from workloads.gen import Workload, _fill_pools_and_q, _live_slots
    B, Hq, Hkv, D, bs, C, P = 65535, 4, 1, 128, 16, 4, 3000
    rng = np.random.default_rng(11)
    table = (3 * (np.arange(B, dtype=np.int32) % 1000))[:, None] + np.arange(3, dtype=np.int32)
    alive = np.ones((B, 3), dtype=np.uint8)
    alive[1::2, 1] = 0
    table[alive == 0] = -1
    ctx_len = np.full(B, 2 * bs + C, dtype=np.int32)
    live = _live_slots(P, bs, table, alive, ctx_len)
    q, kp, vp = _fill_pools_and_q(rng, "bf16", (B, C, Hq, D), P, bs, Hkv, D, live)
    w = Workload(name="prefill_max_batch", kind="prefill", dtype="bf16", B=B, Hq=Hq, Hkv=Hkv,
                 D=D, block_size=bs, block_table=table, alive=alive, ctx_len=ctx_len, q=q,
                 k_pool=kp, v_pool=vp, scale=1.0 / np.sqrt(D), C=C,
                 q_pos0=np.full(B, 2 * bs, dtype=np.int32))
    O, L = run_prefill(w)
    check(w, O, L, seqs=[0, 1, 2, 31337, 65533, 65534])


def test_recompute_small():
    """Recompute of an evicted middle range: chunk rows at q_pos0 in the middle
    of the context, alive blocks after the chunk hidden by the causal mask."""
    for seed in (0, 1):
        w = make_workload(6, seed=seed, size="small")
        O, L = run_prefill(w)
        check(w, O, L)
        O, L = run_prefill(w, 16)
        check(w, O, L)


def test_recompute_full_sampled():
    w = make_workload(6, seed=0)
    O, L = run_prefill(w)
    rng = np.random.default_rng(5)
    rows = np.sort(np.concatenate([[0, 1, 63, 64, 255, 511], rng.choice(512, 8, replace=False)]))
    heads = sorted(rng.choice(w.Hq, size=4, replace=False).tolist())
    check(w, O, L, seqs=[1, 2], heads=heads, rows=np.unique(rows))


def test_prefill_understated_max_ctx_len_truncates_safely():
    """As for decode: an understated max_ctx_len cuts each sequence to the
    grid's capacity (its first splits x split_blocks alive blocks in logical
    order) without touching anything outside the plan or the pool; the rows
    then see only those keys (here every kept key precedes every row)."""
    w = make_workload(3, seed=5, size="small")
    T, max_ctx = 16, 512
    cap_blocks = -(-max_ctx // 16)
    d = to_device(w, DEV)
    segs, indptr, err = msa.msa_plan_segments(d["block_table"], d["alive"], d["ctx_len"],
                                              w.block_size, w.num_phys_blocks)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    out, lse = msa.msa_prefill_chunk(d["q"], d["q_pos0"], d["k_pool"], d["v_pool"], segs, indptr,
                                     max_ctx_len=max_ctx, scale=w.scale, split_blocks=T,
                                     dev_error=err)
    torch.cuda.synchronize()
    # the cut is reported, and only the cut
    assert int(err.item()) == msa.MSA_DEVERR_TRUNCATED
    kept = w.alive.copy()
    for b in range(w.B):
        nb = -(-int(w.ctx_len[b]) // w.block_size)
        idx = [l for l in range(nb) if w.alive[b, l]]
        assert len(idx) > cap_blocks
        for l in idx[cap_blocks:]:
            kept[b, l] = 0
    Or, Lr = oracle.prefill_ref(w.q, w.q_pos0, w.k_pool, w.v_pool, w.block_table, kept, w.ctx_len,
                                w.block_size, w.scale)
    assert np.max(np.abs(from_device(out) - Or)) <= TOL
    assert np.max(np.abs(lse.cpu().numpy().astype(np.float64) - Lr)) <= TOL


@pytest.mark.parametrize("split_blocks", [0, 16])
def test_prefill_sequences_without_keys(split_blocks):
    """A sequence whose every block was evicted (the chunk's own too) and a
    sequence with ctx_len 0 (no block at all) beside ordinary ones: their
    rows see no key and get O = 0, LSE = -inf; the other sequences match the
    oracle, with and without a forced key split."""
    w = make_workload(3, seed=9, size="small", B=4, C=48)
    w.alive[1, :] = 0
    w.ctx_len[2] = 0
    q_pos0 = w.q_pos0.copy()
    q_pos0[2] = 0
    O, L = run_prefill(w, split_blocks, q_pos0=q_pos0)
    for b in (1, 2):
        assert np.all(O[b] == 0) and np.all(np.isneginf(L[b]))
    check(w, O, L, q_pos0=q_pos0)


@pytest.mark.parametrize("C", [128, 256, 1024, 2048])
def test_prefill_chunk_sizes_full_sampled(C):
    """The chunk sizes of the chunk-size curve (prefill workload with C
    varied, 8192 cached tokens): C 128 and 256 split the key stream to fill
    the chip, 1024 and 2048 run several position tiles per (KV head,
    sequence).  Sampled rows (both ends, tile edges) and heads against the
    oracle."""
    w = make_workload(3, seed=0, C=C)
    O, L = run_prefill(w)
    rng = np.random.default_rng(C)
    edges = [0, 31, 32, 63, 64, C // 2, C - 1]
    rows = np.unique(np.concatenate([edges, rng.choice(C, 6, replace=False)]))
    heads = sorted(rng.choice(w.Hq, size=3, replace=False).tolist())
    check(w, O, L, seqs=[0, 3], heads=heads, rows=rows)
