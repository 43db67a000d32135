"""GPU: the gather-then-attend baseline (alive blocks copied into dense pools,
then the same decode kernel over one segment per sequence).

The copy is a byte copy, so every alive token's K/V row in the dense pools
must equal the pool row bit for bit, and the dense plan must be the
one-segment-per-sequence plan.  Decode over the dense pools walks the same
alive blocks in the same order with the same split boundaries, so its output
must equal MSA decode over the fragmented pool bit for bit (and both match
the fp64 oracle within the decode tolerances).  Head-major pool blocks
gather and decode to the same bits.
"""
import numpy as np
import pytest
import torch

import oracle
import kv_cache_attention_msa_amd as msa
from workloads import make_workload
from workloads.device import to_device, from_device

pytestmark = pytest.mark.gpu
DEV = "cuda"


def bits(t):
    """Raw element bits of a device tensor as numpy (bf16 has no numpy dtype)."""
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).cpu().numpy()


def plan(w, d):
    segs, indptr, err = msa.msa_plan_segments(d["block_table"], d["alive"], d["ctx_len"],
                                              w.block_size, w.num_phys_blocks)
    return segs, indptr, err


def dense_path(w, d, segs, indptr, bps):
    dk, dv, dsegs, dind = msa.msa_gather_alive(d["k_pool"], d["v_pool"], segs, indptr, bps)
    out, lse = msa.msa_decode(d["q"], dk, dv, dsegs, dind, max_ctx_len=int(w.ctx_len.max()),
                              scale=w.scale)
    return dk, dv, dsegs, dind, out, lse


@pytest.mark.parametrize("cfg", [1, 2, 5])
def test_gather_copy_and_bitwise_decode_small(cfg):
    w = make_workload(cfg, seed=3, size="small")
    d = to_device(w, DEV)
    segs, indptr, err = plan(w, d)
    bps = int(-(-w.ctx_len.max() // w.block_size))
    dk, dv, dsegs, dind, out_g, lse_g = dense_path(w, d, segs, indptr, bps)
    out_m, lse_m = msa.msa_decode(d["q"], d["k_pool"], d["v_pool"], segs, indptr,
                                  max_ctx_len=int(w.ctx_len.max()), scale=w.scale)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    # dense plan
    ds = dsegs.cpu().numpy()
    assert np.array_equal(dind.cpu().numpy(), np.arange(w.B + 1))
    kp, vp = bits(d["k_pool"]), bits(d["v_pool"])
    dkn, dvn = bits(dk), bits(dv)
    for b in range(w.B):
        nb = -(-int(w.ctx_len[b]) // w.block_size)
        alive_l = [l for l in range(nb) if w.alive[b, l]]
        A = sum(min(w.block_size, int(w.ctx_len[b]) - l * w.block_size) for l in alive_l)
        assert tuple(ds[b]) == (b, 0, b * bps, len(alive_l), A, 0)
        for j, l in enumerate(alive_l):   # byte copy of every alive block
            ph = w.block_table[b, l]
            assert np.array_equal(dkn[b * bps + j], kp[ph])
            assert np.array_equal(dvn[b * bps + j], vp[ph])
    # same kernel, same blocks, same order: identical bits
    assert np.array_equal(bits(out_g), bits(out_m))
    assert torch.equal(lse_g, lse_m)
    Or, Lr = oracle.decode_ref(w.q, w.k_pool, w.v_pool, w.block_table, w.alive, w.ctx_len,
                               w.block_size, w.scale)
    tol = 1e-5 if w.dtype == "f32" else 2e-2
    assert np.max(np.abs(from_device(out_g) - Or)) <= tol
    assert np.max(np.abs(lse_g.cpu().numpy() - Lr)) <= tol


def test_gather_bitwise_decode_full():
    w = make_workload(2, seed=0)
    d = to_device(w, DEV)
    segs, indptr, _ = plan(w, d)
    bps = int(-(-w.ctx_len.max() // w.block_size))
    *_, out_g, lse_g = dense_path(w, d, segs, indptr, bps)
    out_m, lse_m = msa.msa_decode(d["q"], d["k_pool"], d["v_pool"], segs, indptr,
                                  max_ctx_len=int(w.ctx_len.max()), scale=w.scale)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out_g), bits(out_m))
    assert torch.equal(lse_g, lse_m)


def test_gather_head_major_pools():
    """Head-major pool blocks: the gather copies whole blocks whatever their
    inner order, so gathering head-major pools gives the head-major image of
    the token-major dense pools, and decode over it (msa_decode_ex) equals
    the token-major dense decode bit for bit."""
    w = make_workload(2, seed=3, size="small")
    d = to_device(w, DEV)
    segs, indptr, err = plan(w, d)
    bps = int(-(-w.ctx_len.max() // w.block_size))
    dk, dv, dsegs, dind, out_n, lse_n = dense_path(w, d, segs, indptr, bps)
    kh = d["k_pool"].permute(0, 2, 1, 3).contiguous()
    vh = d["v_pool"].permute(0, 2, 1, 3).contiguous()
    dkh, dvh, dsegs_h, dind_h = msa.msa_gather_alive(kh, vh, segs, indptr, bps, kv_layout="HND")
    out_h, lse_h = msa.msa_decode(d["q"], dkh, dvh, dsegs_h, dind_h, max_ctx_len=int(w.ctx_len.max()),
                                  scale=w.scale, kv_layout="HND")
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert torch.equal(dsegs_h, dsegs) and torch.equal(dind_h, dind)
    # alive blocks of the dense pools agree (dead dense slots are never read)
    live = torch.zeros(dk.shape[0], dtype=torch.bool, device=dk.device)
    for b in range(w.B):
        n_alive = int(w.alive[b, :-(-int(w.ctx_len[b]) // w.block_size)].sum())
        live[b * bps:b * bps + n_alive] = True
    assert np.array_equal(bits(dkh[live]), bits(dk[live].permute(0, 2, 1, 3).contiguous()))
    assert np.array_equal(bits(dvh[live]), bits(dv[live].permute(0, 2, 1, 3).contiguous()))
    assert torch.equal(out_h, out_n) and torch.equal(lse_h, lse_n)
