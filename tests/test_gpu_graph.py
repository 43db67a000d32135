"""The decode step under HIP graph capture, for callers that replay a
captured serving step: msa_plan_segments and msa_decode_noalloc (no
allocation, no memset node: every buffer is written by a kernel) captured
into one graph with torch.cuda.graph, replayed three times with unrelated
eager work and synchronisations between the replays; every replay must give
the eager result bit for bit.  Covers the per-head kernel (32 x 4k shape),
the block kernel with shared prefixes and the merge (lognormal batch), and
the block kernel on the 131k-token layout, at test sizes."""
import ctypes

import pytest
import torch

import kv_cache_attention_msa_amd as msa
from kv_cache_attention_msa_amd import _lib
from workloads import make_workload
from workloads.device import to_device

pytestmark = pytest.mark.gpu
DEV = "cuda"
P = ctypes.c_void_p


def _noalloc(w, d, segs, indptr, out, lse, err):
    st = _lib.load().msa_decode_noalloc(
        P(d["q"].data_ptr()), P(d["k_pool"].data_ptr()), P(d["v_pool"].data_ptr()),
        w.num_phys_blocks, w.block_size, P(segs.data_ptr()), P(indptr.data_ptr()), w.B, w.Hq,
        w.Hkv, w.D, int(w.ctx_len.max()), _lib.MSA_BF16, float(w.scale), 0, P(out.data_ptr()),
        P(lse.data_ptr()), P(err.data_ptr()), P(torch.cuda.current_stream().cuda_stream))
    assert st == 0, st


@pytest.mark.parametrize("cfg", [2, 4, 5])
def test_plan_and_noalloc_decode_replay_in_a_graph(cfg):
    w = make_workload(cfg, seed=4, size="small")
    d = to_device(w, DEV)
    out_e = torch.empty_like(d["q"])
    lse_e = torch.empty((w.B, w.Hq), dtype=torch.float32, device=DEV)
    # eager reference; this first call also looks up the library array's
    # device address, which is not done under capture
    segs, indptr, err = msa.msa_plan_segments(d["block_table"], d["alive"], d["ctx_len"],
                                              w.block_size, w.num_phys_blocks)
    _noalloc(w, d, segs, indptr, out_e, lse_e, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0

    out_g = torch.empty_like(d["q"])
    lse_g = torch.empty((w.B, w.Hq), dtype=torch.float32, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on a side stream before capture
        s2, i2, e2 = msa.msa_plan_segments(d["block_table"], d["alive"], d["ctx_len"],
                                           w.block_size, w.num_phys_blocks)
        _noalloc(w, d, s2, i2, out_g, lse_g, e2)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        s3, i3, e3 = msa.msa_plan_segments(d["block_table"], d["alive"], d["ctx_len"],
                                           w.block_size, w.num_phys_blocks)
        _noalloc(w, d, s3, i3, out_g, lse_g, e3)
    noise = torch.randn(1 << 20, device=DEV)
    for rep in range(3):
        out_g.fill_(float("nan"))
        lse_g.fill_(float("nan"))
        noise.mul_(1.0001).add_(1.0)  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(e3.item()) == 0, rep
        assert torch.equal(out_g, out_e), rep
        assert torch.equal(lse_g, lse_e), rep
