"""GPU parity of MSA decode (rows a2, a3, a5) against the fp64 oracle.

Element-by-element comparison of O and LSE on the same seeded inputs, through
the C ABI: max-abs-error <= 1e-5 for the fp32 family, <= 2e-2 for bf16 inputs
with fp32 accumulation.  Sizes span many tiles and splits with ragged tails
(partial last blocks, splits that end mid-tile, single-split and many-split
sequences); full-size families 4 and 5 are checked on sampled (sequence,
head) pairs the oracle computes one by one.  Also: empty sequences, the
maximum batch the grid takes (65535 sequences, with and without splits),
head-major pool blocks (bitwise equal to the token-major layout),
run-to-run bitwise determinism, physical-relayout invariance, and the
stand-alone merge call.
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

TOL = {"f32": 1e-5, "bf16": 2e-2}


def run_decode(w, split_blocks=0, d=None, kernel="auto"):
    d = d or to_device(w, DEV)
    segs, indptr, err = msa.msa_plan_segments(d["block_table"], d["alive"], d["ctx_len"],
                                              w.block_size, w.num_phys_blocks)
    # the plan's error word also collects the decode's (a true max_ctx_len:
    # no truncation may be reported)
    out, lse = msa.msa_decode(d["q"], d["k_pool"], d["v_pool"], segs, indptr,
                              max_ctx_len=int(w.ctx_len.max()), scale=w.scale,
                              split_blocks=split_blocks, kernel=kernel, dev_error=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    return from_device(out), lse.cpu().numpy().astype(np.float64)


def check(w, O, L, seqs=None, heads=None):
    Or, Lr = oracle.decode_ref(w.q, w.k_pool, w.v_pool, w.block_table, w.alive, w.ctx_len,
                               w.block_size, w.scale, seqs=seqs, heads=heads)
    sel = ~np.isnan(Lr)
    tol = TOL[w.dtype]
    err_o = np.max(np.abs(O - Or)[np.isfinite(Or)]) if sel.any() else 0.0
    fin = sel & np.isfinite(Lr)
    err_l = np.max(np.abs(L[fin] - Lr[fin])) if fin.any() else 0.0
    assert np.all(np.isneginf(L[sel & np.isneginf(Lr)]))
    assert err_o <= tol, f"max |O - ref| = {err_o}"
    assert err_l <= tol, f"max |LSE - ref| = {err_l}"
    return err_o, err_l


@pytest.mark.parametrize("split_blocks", [0, 16, 48])
def test_decode_cfg1_fp32(split_blocks):
    w = make_workload(1, seed=0)
    O, L = run_decode(w, split_blocks)
    check(w, O, L)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_decode_cfg1_seeds(seed):
    w = make_workload(1, seed=seed)
    O, L = run_decode(w)
    check(w, O, L)


@pytest.mark.parametrize("split_blocks", [0, 16, 32, 512])
@pytest.mark.parametrize("cfg", [2, 4, 5])
def test_decode_small(cfg, split_blocks):
    w = make_workload(cfg, seed=1, size="small")
    O, L = run_decode(w, split_blocks)
    check(w, O, L)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_decode_head_shapes(G, D):
    Hkv = 2
    w = make_workload(2, seed=5, size="small", B=3, ctx=900, Hq=Hkv * G, Hkv=Hkv, D=D)
    O, L = run_decode(w, 16)
    check(w, O, L)


def test_decode_cfg1_shapes_fp32_groups():
    for G in (1, 2, 8):
        w = make_workload(1, seed=3, Hq=2 * G, Hkv=2)
        O, L = run_decode(w, 16)
        check(w, O, L)


def test_decode_cfg2_full():
    w = make_workload(2, seed=0)
    O, L = run_decode(w)
    check(w, O, L)


@pytest.mark.parametrize("split_blocks", [64, 16])
def test_decode_cfg2_full_forced_splits(split_blocks):
    """The headline batch needs no merge under the automatic split rule; forced
    splits of 64 blocks (4 per sequence: 1024 workgroups, so the matrix-core
    kernel reads K into registers) and 16 blocks (16 per sequence) cover the
    split and merge paths at full size."""
    w = make_workload(2, seed=0)
    O, L = run_decode(w, split_blocks)
    check(w, O, L)


@pytest.mark.parametrize("cfg", [4, 5])
def test_decode_full_sampled(cfg):
    w = make_workload(cfg, seed=0)
    O, L = run_decode(w)
    rng = np.random.default_rng(cfg)
    seqs = sorted(rng.choice(w.B, size=min(w.B, 4), replace=False).tolist())
    heads = sorted(rng.choice(w.Hq, size=6, replace=False).tolist())
    check(w, O, L, seqs=seqs, heads=heads)


def test_decode_empty_and_tiny_sequences():
    w = make_workload(2, seed=2, size="small", B=5, ctx=700)
    w.alive[0, :] = 0                 # everything evicted
    w.ctx_len[1] = 1                  # a single token (the first block is always alive)
    w.ctx_len[2] = 17                 # one full block + one token
    w.ctx_len[3] = 0                  # no tokens at all
    assert w.alive[1, 0] and w.alive[2, 0]
    for split in (0, 16):
        O, L = run_decode(w, split)
        for b in (0, 3):
            assert np.all(O[b] == 0) and np.all(np.isneginf(L[b]))
        check(w, O, L, seqs=[1, 2, 4])


@pytest.mark.parametrize("split_blocks", [0, 1])
def test_decode_max_batch(split_blocks):
    """65535 sequences, the most the decode grid takes (sequence is its
    slowest dimension), each of three blocks with one of the first two
    evicted; with split_blocks=1 every alive block is its own split and the
    LSE merge runs over the same 65535 sequences."""
    w = make_workload(1, seed=3, B=65535, Hq=4, Hkv=1, nb=3, pool=3 * 65535, n_evict=1)
    O, L = run_decode(w, split_blocks)
    check(w, O, L, seqs=[0, 1, 2, 31337, 65533, 65534])


def _decode_both_layouts(w, split_blocks, kernel="auto"):
    d = to_device(w, DEV)
    segs, indptr, err = msa.msa_plan_segments(d["block_table"], d["alive"], d["ctx_len"],
                                              w.block_size, w.num_phys_blocks)
    outs = []
    for layout in ("NHD", "HND"):
        k, v = d["k_pool"], d["v_pool"]
        if layout == "HND":
            k, v = k.permute(0, 2, 1, 3).contiguous(), v.permute(0, 2, 1, 3).contiguous()
        outs.append(msa.msa_decode(d["q"], k, v, segs, indptr, max_ctx_len=int(w.ctx_len.max()),
                                   scale=w.scale, split_blocks=split_blocks, kv_layout=layout,
                                   kernel=kernel))
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    return outs


@pytest.mark.parametrize("cfg,split_blocks", [(1, 0), (1, 16), (2, 0), (2, 16), (4, 16), (5, 0)])
def test_decode_head_major_layout(cfg, split_blocks):
    """Pools in head-major blocks [P, Hkv, 16, D] (msa_decode_ex): the same
    values give bitwise the same O and LSE as the token-major layout, and
    both match the oracle.  Covers the VALU kernel (fp32), the MFMA kernel
    for 4 and 8 heads per KV head (K by row DMA on one-workgroup-per-CU
    grids, in registers otherwise), and the split merge."""
    w = make_workload(cfg, seed=6, size="small")
    (o_n, l_n), (o_h, l_h) = _decode_both_layouts(w, split_blocks)
    assert torch.equal(o_n, o_h) and torch.equal(l_n, l_h)
    check(w, from_device(o_h), l_h.cpu().numpy().astype(np.float64))


@pytest.mark.parametrize("cfg", [2, 4, 5])
def test_decode_head_major_layout_full(cfg):
    """Full-size batches (the headline one, the lognormal shared-prefix one
    with its 11 splits, the 131k-token one): head-major equals token-major
    bit for bit, and sampled (sequence, head) pairs match the oracle."""
    w = make_workload(cfg, seed=0)
    (o_n, l_n), (o_h, l_h) = _decode_both_layouts(w, 0)
    assert torch.equal(o_n, o_h) and torch.equal(l_n, l_h)
    rng = np.random.default_rng(10 + cfg)
    seqs = sorted(rng.choice(w.B, size=min(w.B, 3), replace=False).tolist())
    heads = sorted(rng.choice(w.Hq, size=4, replace=False).tolist())
    check(w, from_device(o_h), l_h.cpu().numpy().astype(np.float64), seqs=seqs, heads=heads)


def test_decode_determinism():
    w = make_workload(4, seed=1, size="small")
    d = to_device(w, DEV)
    O1, L1 = run_decode(w, 16, d)
    O2, L2 = run_decode(w, 16, d)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_decode_determinism_full():
    """Full-size headline batch, three calls: identical bits every time (the
    tile pipeline must never read a V tile before its copy has landed)."""
    w = make_workload(2, seed=0)
    d = to_device(w, DEV)
    O1, L1 = run_decode(w, 0, d)
    for _ in range(2):
        O2, L2 = run_decode(w, 0, d)
        assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_decode_relayout_invariance():
    """The same alive content under a packed layout (few long segments) and
    under one block per segment gives the same output within tolerance."""
    w = make_workload(2, seed=3, size="small")
    O1, L1 = run_decode(w)
    rng = np.random.default_rng(1)
    P = w.num_phys_blocks
    perm = rng.permutation(P)
    kp = np.full_like(w.k_pool, 0x7FC0)
    vp = np.full_like(w.v_pool, 0x7FC0)
    table = np.full_like(w.block_table, -1)
    nxt = 0
    for b in range(w.B):
        for l in range(w.max_blocks):
            if w.alive[b, l] and l * 16 < w.ctx_len[b]:
                dst = perm[nxt]
                nxt += 1
                kp[dst] = w.k_pool[w.block_table[b, l]]
                vp[dst] = w.v_pool[w.block_table[b, l]]
                table[b, l] = dst
    w.k_pool, w.v_pool, w.block_table = kp, vp, table
    O2, L2 = run_decode(w)
    assert np.max(np.abs(O1 - O2)) <= 2e-2 and np.max(np.abs(L1 - L2)) <= 1e-3


def test_merge_partials_parity():
    rng = np.random.default_rng(4)
    B, R, H, D = 3, 5, 4, 128
    counts = [3, 0, 6]
    ind = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    N = int(ind[-1])
    o = rng.standard_normal((N, R, H, D)).astype(np.float32)
    m = (rng.standard_normal((N, R, H)) * 3).astype(np.float32)
    l = rng.uniform(0.5, 20, size=(N, R, H)).astype(np.float32)
    m[1, 2, :] = -np.inf        # an empty partial (its o is garbage)
    l[1, 2, :] = 0
    o[1, 2, :] = np.nan
    m[3:, 0, 1] = -np.inf       # a row with every partial empty
    l[3:, 0, 1] = 0
    for dt, tol in ((torch.float32, 1e-5), (torch.bfloat16, 2e-2)):
        out, lse = msa.msa_merge_partials(tensor(o, DEV), tensor(m, DEV), tensor(l, DEV),
                                          tensor(ind, DEV), out_dtype=dt)
        torch.cuda.synchronize()
        Or, Lr = oracle.merge_ref(o, m, l, ind)
        Og = from_device(out)
        Lg = lse.cpu().numpy().astype(np.float64)
        assert np.max(np.abs(Og - Or)) <= tol
        fin = np.isfinite(Lr)
        assert np.max(np.abs(Lg[fin] - Lr[fin])) <= 1e-5
        assert np.all(np.isneginf(Lg[~fin]))


def test_merge_partials_many_and_ragged():
    """Sequences with 0..37 partials (the four-way split of the partial list
    gets empty, short and uneven quarters), head x dim not a multiple of the
    64-element workgroup, and an all-empty quarter."""
    rng = np.random.default_rng(11)
    B, R, H, D = 5, 2, 3, 40
    counts = [37, 1, 2, 0, 5]
    ind = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    N = int(ind[-1])
    o = rng.standard_normal((N, R, H, D)).astype(np.float32)
    m = (rng.standard_normal((N, R, H)) * 4).astype(np.float32)
    l = rng.uniform(0.5, 20, size=(N, R, H)).astype(np.float32)
    m[0:9, 1, 2] = -np.inf      # the first quarter of sequence 0 empty for one row/head
    l[0:9, 1, 2] = 0
    o[0:9, 1, 2] = np.nan
    m[30, 0, 0] = 40.0          # a late partial with a much larger maximum
    for dt, tol in ((torch.float32, 1e-5), (torch.bfloat16, 2e-2)):
        out, lse = msa.msa_merge_partials(tensor(o, DEV), tensor(m, DEV), tensor(l, DEV),
                                          tensor(ind, DEV), out_dtype=dt)
        torch.cuda.synchronize()
        Or, Lr = oracle.merge_ref(o, m, l, ind)
        Og = from_device(out)
        Lg = lse.cpu().numpy().astype(np.float64)
        assert np.max(np.abs(Og - Or)) <= tol
        fin = np.isfinite(Lr)
        assert np.max(np.abs(Lg[fin] - Lr[fin])) <= 1e-5
        assert np.all(np.isneginf(Lg[~fin]))


@pytest.mark.parametrize("cfg", [1, 2])
def test_decode_understated_max_ctx_len_truncates_safely(cfg):
    """max_ctx_len sizes the grid; a caller that understates it gets each
    sequence cut to the grid's capacity (its first splits x split_blocks
    alive blocks, in logical order) -- never an access outside the plan or
    the pool.  The result must equal the oracle over that prefix."""
    w = make_workload(cfg, seed=3, size="small")
    T, max_ctx = 16, 512  # 32 blocks of 16 tokens -> two splits of 16
    cap_blocks = -(-max_ctx // 16)
    d = to_device(w, DEV)
    segs, indptr, err = msa.msa_plan_segments(d["block_table"], d["alive"], d["ctx_len"],
                                              w.block_size, w.num_phys_blocks)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    out, lse = msa.msa_decode(d["q"], d["k_pool"], d["v_pool"], segs, indptr,
                              max_ctx_len=max_ctx, scale=w.scale, split_blocks=T, dev_error=err)
    torch.cuda.synchronize()
    # the cut is reported, and only the cut
    assert int(err.item()) == msa.MSA_DEVERR_TRUNCATED
    kept = w.alive.copy()
    cut_any = False
    for b in range(w.B):
        nb = -(-int(w.ctx_len[b]) // w.block_size)
        idx = [l for l in range(nb) if w.alive[b, l]]
        for l in idx[cap_blocks:]:
            kept[b, l] = 0
        cut_any |= len(idx) > cap_blocks
    assert cut_any, "the workload must have a sequence longer than the grid"
    Or, Lr = oracle.decode_ref(w.q, w.k_pool, w.v_pool, w.block_table, kept, w.ctx_len,
                               w.block_size, w.scale)
    tol = TOL[w.dtype]
    assert np.max(np.abs(from_device(out) - Or)) <= tol
    assert np.max(np.abs(lse.cpu().numpy().astype(np.float64) - Lr)) <= tol


@pytest.mark.parametrize("cfg,Hq,split_blocks", [(2, 32, 0), (2, 64, 0), (2, 32, 16), (5, 64, 0),
                                                 (5, 32, 0), (4, 32, 0)])
def test_decode_vector_and_matrix_kernels(cfg, Hq, split_blocks):
    """msa_decode_ex with the kernel chosen explicitly: the vector-ALU kernel
    (fp32 softmax weights), the per-KV-head matrix-core kernel and the block
    kernel (both round the weights to bf16 for P x V) on the same small
    batches, 4 and 8 query heads per KV head, with and without splits.  All
    match the oracle within the bf16 tolerance, and agree with each other
    within it too."""
    w = make_workload(cfg, seed=8, size="small", Hq=Hq)
    d = to_device(w, DEV)
    res = {}
    for kern in ("vector", "matrix", "block"):
        O, L = run_decode(w, split_blocks, d, kernel=kern)
        res[kern] = check(w, O, L) + (O, L)
    assert np.max(np.abs(res["vector"][2] - res["matrix"][2])) <= TOL["bf16"]
    assert np.max(np.abs(res["vector"][2] - res["block"][2])) <= TOL["bf16"]


@pytest.mark.parametrize("cfg", [2, 4, 5])
def test_decode_vector_and_matrix_kernels_full(cfg):
    """Full-size headline batch (4 query heads per KV head), the lognormal
    shared-prefix batch and the 131k-token batch (8 per KV head): each
    kernel against the oracle on sampled (sequence, head) pairs."""
    w = make_workload(cfg, seed=0)
    d = to_device(w, DEV)
    rng = np.random.default_rng(20 + cfg)
    seqs = sorted(rng.choice(w.B, size=min(w.B, 3), replace=False).tolist())
    heads = sorted(rng.choice(w.Hq, size=4, replace=False).tolist())
    for kern in ("vector", "matrix", "block"):
        O, L = run_decode(w, 0, d, kernel=kern)
        check(w, O, L, seqs=seqs, heads=heads)


# ---- the block kernel (one workgroup per split, whole blocks of all KV heads)

@pytest.mark.parametrize("cfg,split_blocks", [(2, 0), (2, 16), (4, 0), (5, 0), (5, 1)])
def test_decode_block_kernel_head_major(cfg, split_blocks):
    """The block kernel on head-major pool blocks gives bitwise the
    token-major result, and both match the oracle (split_blocks 1: every
    alive block its own split, the merge over the most partials)."""
    w = make_workload(cfg, seed=6, size="small")
    (o_n, l_n), (o_h, l_h) = _decode_both_layouts(w, split_blocks, kernel="block")
    assert torch.equal(o_n, o_h) and torch.equal(l_n, l_h)
    check(w, from_device(o_h), l_h.cpu().numpy().astype(np.float64))


def test_decode_block_kernel_empty_and_tiny_sequences():
    """Sequences with no alive token (all evicted, ctx_len 0) get O = 0 and
    LSE = -inf from their one workgroup; one-token and one-block-plus-one
    sequences end mid-block; automatic and forced split lengths."""
    w = make_workload(2, seed=2, size="small", B=5, ctx=700)
    w.alive[0, :] = 0
    w.ctx_len[1] = 1
    w.ctx_len[2] = 17
    w.ctx_len[3] = 0
    for split in (0, 1, 16):
        O, L = run_decode(w, split, kernel="block")
        for b in (0, 3):
            assert np.all(O[b] == 0) and np.all(np.isneginf(L[b]))
        check(w, O, L, seqs=[1, 2, 4])


@pytest.mark.parametrize("B,ctx", [(1, 5000), (3, 900), (97, 300), (257, 200), (512, 100)])
def test_decode_block_kernel_batch_sizes(B, ctx):
    """From one sequence (every workgroup on one sequence) to the 512 the
    block kernel takes (one or two splits each), across the 256 up to which
    it looks for shared prefixes; the device split rule sees every count."""
    w = make_workload(2, seed=4, size="small", B=B, ctx=ctx, pool_factor=2.0)
    O, L = run_decode(w, 0, kernel="block")
    seqs = sorted(set([0, B // 2, B - 1]))
    check(w, O, L, seqs=seqs)


def test_decode_block_kernel_understated_max_ctx_len():
    """Understated max_ctx_len with the block kernel: the same cut as the
    per-head kernels (the first splits x split_blocks alive blocks of each
    sequence), reported by MSA_DEVERR_TRUNCATED, equal to the oracle over
    that prefix."""
    w = make_workload(2, seed=3, size="small")
    T, max_ctx = 16, 512
    cap_blocks = -(-max_ctx // 16)
    d = to_device(w, DEV)
    segs, indptr, err = msa.msa_plan_segments(d["block_table"], d["alive"], d["ctx_len"],
                                              w.block_size, w.num_phys_blocks)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    for split in (T, 0):
        err.zero_()
        out, lse = msa.msa_decode(d["q"], d["k_pool"], d["v_pool"], segs, indptr,
                                  max_ctx_len=max_ctx, scale=w.scale, split_blocks=split,
                                  kernel="block", dev_error=err)
        torch.cuda.synchronize()
        assert int(err.item()) == msa.MSA_DEVERR_TRUNCATED
        if split == T:
            kept = w.alive.copy()
            for b in range(w.B):
                nb = -(-int(w.ctx_len[b]) // w.block_size)
                idx = [l for l in range(nb) if w.alive[b, l]]
                for l in idx[cap_blocks:]:
                    kept[b, l] = 0
            Or, Lr = oracle.decode_ref(w.q, w.k_pool, w.v_pool, w.block_table, kept, w.ctx_len,
                                       w.block_size, w.scale)
            assert np.max(np.abs(from_device(out) - Or)) <= TOL["bf16"]
            assert np.max(np.abs(lse.cpu().numpy().astype(np.float64) - Lr)) <= TOL["bf16"]


def test_decode_block_kernel_determinism_full():
    """The 131k-token batch (automatic choice: the block kernel), three
    calls: identical bits every time."""
    w = make_workload(5, seed=0)
    d = to_device(w, DEV)
    O1, L1 = run_decode(w, 0, d)
    for _ in range(2):
        O2, L2 = run_decode(w, 0, d)
        assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def _shared_prefix_batch(Hq, seed=0):
    """Twenty-one sequences over one pool of finite bf16 values, built so that
    the block kernel's prefix sharing meets its edge cases:
      * sequences 0-17 start on the same 20 physical blocks (17 members with
        sequence 8 left out below: a sub-group with a single member is left
        over); their private blocks follow, some evicted;
      * sequence 3 lies entirely inside 12 of those blocks, and sequence 5
        ends in a partial block inside its first segment (9 full blocks), so
        the common prefix of the group is 9 blocks;
      * sequence 8 has block 0 evicted: its first segment does not start at
        logical block 0, so it is not a member;
      * sequences 18 and 19 share only 5 blocks (fewer than the kernel
        shares);
      * sequence 20 shares nothing."""
    from workloads.gen import Workload, f32_to_bf16_bits
    rng = np.random.default_rng(seed)
    B, Hkv, D, bs, P = 21, 8, 128, 16, 640
    nbmax = 48
    table = np.full((B, nbmax), -1, np.int32)
    alive = np.zeros((B, nbmax), np.uint8)
    ctx = np.zeros(B, np.int32)
    free = list(rng.permutation(np.arange(40, P)))
    for b in range(B):
        nb = int(rng.integers(24, nbmax + 1))
        if b < 18:
            shared = list(range(0, 20))
        elif b < 20:
            shared = list(range(20, 25))
        else:
            shared = []
        priv = [int(free.pop()) for _ in range(nb - len(shared))]
        ids = shared + priv
        table[b, :nb] = ids
        alive[b, :nb] = 1
        ctx[b] = nb * bs - int(rng.integers(0, bs))
        # a few private evictions (never the last block)
        for l in rng.choice(np.arange(len(shared), nb - 1), size=3, replace=False):
            alive[b, l] = 0
    ctx[3] = 12 * bs
    alive[3, 12:] = 0
    ctx[5] = 9 * bs + 7
    alive[5, 10:] = 0
    alive[8, 0] = 0
    q = f32_to_bf16_bits(rng.standard_normal((B, Hq, D), dtype=np.float32))
    k = f32_to_bf16_bits(rng.standard_normal((P, bs, Hkv, D), dtype=np.float32))
    v = f32_to_bf16_bits(rng.standard_normal((P, bs, Hkv, D), dtype=np.float32))
    return Workload(name="shared-prefix edge cases", kind="decode", dtype="bf16", B=B, Hq=Hq,
                    Hkv=Hkv, D=D, block_size=bs, block_table=table, alive=alive, ctx_len=ctx,
                    q=q, k_pool=k, v_pool=v, scale=1.0 / np.sqrt(D))


@pytest.mark.parametrize("Hq", [32, 64])
@pytest.mark.parametrize("split_blocks", [0, 4, 16])
def test_decode_block_kernel_shared_prefixes(Hq, split_blocks):
    """Prefix sharing in the block kernel (4 and 8 query heads per KV head:
    8 and 4 member sequences per shared item): every sequence matches the
    oracle, and the per-head kernel within the bf16 tolerance."""
    w = _shared_prefix_batch(Hq)
    d = to_device(w, DEV)
    Ob, Lb = run_decode(w, split_blocks, d, kernel="block")
    check(w, Ob, Lb)
    Om, Lm = run_decode(w, split_blocks, d, kernel="matrix")
    assert np.max(np.abs(Ob - Om)) <= TOL["bf16"]
    (o_n, l_n), (o_h, l_h) = _decode_both_layouts(w, split_blocks, kernel="block")
    assert torch.equal(o_n, o_h) and torch.equal(l_n, l_h)
