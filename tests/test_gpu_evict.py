"""Kernel-aware eviction on the GPU path: evictions chosen by the scorer
(hit probability + recompute cost + decode cost from a latency model), by
hit probability and a longest-sequence latency model, and by hit probability
alone are applied to a decode batch, then re-planned with msa_plan_segments
and attended with msa_decode; every result must match the fp64 oracle over
the surviving tokens, and the device plan must equal the oracle's plan of
the new alive mask byte for byte."""
import numpy as np
import pytest
import torch

import oracle
import kv_cache_attention_msa_amd as msa
from kv_cache_attention_msa_amd.evict import (DecodeLatencyModel, choose_evictions,
                                              recompute_cost_us)
from workloads import make_workload
from workloads.device import to_device, from_device

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 2e-2

# a latency model of the shape the decode kernel measures (per-token cost an
# order of magnitude above the per-segment cost)
MODEL = DecodeLatencyModel(c0=1.0, c_tok=8.0e-4, c_seg=6.7e-4)
# the fitted shape on a one-split grid: the longest sequence sets the time
MODEL_MAX = DecodeLatencyModel(c0=12.0, c_tok=4.3e-4, c_seg=0.0, c_max=5.2e-3)


def _policies(w, frac):
    rng = np.random.default_rng(17)
    hit = rng.random(w.alive.shape)
    rec = [recompute_cost_us(w.alive[b], w.ctx_len[b], w.block_size, w.D, w.Hq, 1000.0)
           for b in range(w.B)]
    nb = -(-w.ctx_len.astype(np.int64) // w.block_size)
    n_alive = sum(int(w.alive[b, :nb[b] - 1].sum()) for b in range(w.B))
    n_ev = int(frac * n_alive)
    out = {}
    for name, model, kw in (("kernel_aware", MODEL, dict(alpha=float(np.mean([r.mean() for r in rec])),
                                                         beta=1.0, gamma=1000.0)),
                            ("latency_aware", MODEL_MAX, dict(alpha=1.0, beta=0.0, gamma=10.0 * w.B)),
                            ("hit_only", MODEL, dict(alpha=1.0, beta=0.0, gamma=0.0))):
        al, ev = choose_evictions(w.block_table, w.alive, w.ctx_len, w.block_size, n_ev, hit, rec,
                                  model, batch_seqs=w.B, **kw)
        assert len(ev) == n_ev
        out[name] = al
    return out


@pytest.mark.parametrize("cfg,frac", [(2, 0.1), (2, 0.3), (4, 0.2)])
def test_scorer_evictions_through_plan_and_decode(cfg, frac):
    w = make_workload(cfg, seed=12, size="small")
    d = to_device(w, DEV)
    segs_seen = {}
    for name, al in _policies(w, frac).items():
        d["alive"] = torch.from_numpy(np.ascontiguousarray(al)).to(DEV)
        segs, indptr, err = msa.msa_plan_segments(d["block_table"], d["alive"], d["ctx_len"],
                                                  w.block_size, w.num_phys_blocks)
        out, lse = msa.msa_decode(d["q"], d["k_pool"], d["v_pool"], segs, indptr,
                                  max_ctx_len=int(w.ctx_len.max()), scale=w.scale, dev_error=err)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        rs, ri = oracle.plan_ref(w.block_table, al, w.ctx_len, w.block_size)
        n = int(ri[-1])
        assert indptr.cpu().numpy().tolist() == ri.tolist()
        assert segs[:n].cpu().numpy().tobytes() == rs.tobytes()
        Or, Lr = oracle.decode_ref(w.q, w.k_pool, w.v_pool, w.block_table, al, w.ctx_len,
                                   w.block_size, w.scale)
        assert np.max(np.abs(from_device(out) - Or)) <= TOL, name
        assert np.max(np.abs(lse.cpu().numpy().astype(np.float64) - Lr)) <= TOL, name
        segs_seen[name] = n
    # the decode-cost term steers the scorer towards blocks whose eviction
    # does not split a segment
    assert segs_seen["kernel_aware"] <= segs_seen["hit_only"]
    # the longest-sequence term shortens the longest sequence at least as
    # much as hit probability alone
    from kv_cache_attention_msa_amd.evict import alive_tokens
    pol = _policies(w, frac)
    assert alive_tokens(pol["latency_aware"], w.ctx_len, w.block_size).max() <= \
        alive_tokens(pol["hit_only"], w.ctx_len, w.block_size).max()
