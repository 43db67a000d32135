"""The seeded input generator: determinism, layout validity, poisoning, and
the eviction statistics each workload family is defined by."""
import numpy as np
import pytest

from workloads import make_workload
from oracle import to_f64


def _check_layout(w):
    bs = w.block_size
    seen = {}
    for b in range(w.B):
        nb = -(-int(w.ctx_len[b]) // bs)
        assert w.alive[b, nb:].sum() == 0
        ids = w.block_table[b, :nb][w.alive[b, :nb] == 1]
        assert len(set(ids.tolist())) == len(ids)          # distinct within a sequence
        assert ids.min() >= 0 and ids.max() < w.num_phys_blocks
        for l in range(nb):
            if w.alive[b, l]:
                ntok = min(bs, int(w.ctx_len[b]) - l * bs)
                k = to_f64(w.k_pool[w.block_table[b, l]])
                assert np.isfinite(k[:ntok]).all()
                assert np.isnan(k[ntok:]).all()              # padding is poisoned
                seen[int(w.block_table[b, l])] = True
    # every block not referenced by an alive entry is poison
    unused = np.setdiff1d(np.arange(w.num_phys_blocks), np.array(sorted(seen)))
    if len(unused):
        assert np.isnan(to_f64(w.v_pool[unused[:50]])).all()


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5, 6])
def test_small_layouts(cfg):
    w = make_workload(cfg, seed=0, size="small")
    _check_layout(w)
    w2 = make_workload(cfg, seed=0, size="small")
    assert np.array_equal(w.block_table, w2.block_table)
    assert np.array_equal(w.q, w2.q)


def test_family_statistics_full_tables():
    # only the cheap parts are checked at full size (no pools for 4 and 5)
    w1 = make_workload(1, seed=0)
    assert w1.meta["alive_blocks"] == 48 and w1.num_phys_blocks == 256
    w2 = make_workload(2, seed=0)
    assert abs(w2.meta["evicted_fraction"] - 0.2) < 0.03
    assert w2.q.dtype == np.uint16 and w2.q.shape == (32, 32, 128)
    w3 = make_workload(3, seed=0)
    assert w3.kind == "prefill" and w3.C == 512 and int(w3.q_pos0[0]) == 8192
    cached = w3.alive[:, :512]
    assert abs(1 - cached.mean() - 0.15) < 0.05
    assert w3.alive[:, 512:].all()


def test_prefill_small_has_ragged_chunk():
    w = make_workload(3, seed=1, size="small", C=70)
    assert int(w.ctx_len[0]) == 1024 + 70
    _check_layout(w)


@pytest.mark.parametrize("size", ["small", "full"])
def test_recompute_chunk_in_fresh_run_with_keys_after_it(size):
    """Recompute family: the chunk's logical range is alive, sits in its own
    physical run (not adjacent to any neighbour's slot), and alive blocks
    follow it, so only the causal mask keeps them from the chunk rows."""
    w = make_workload(6, seed=1, size=size, values=False)
    bs = w.block_size
    for b in range(w.B):
        c0, cb = int(w.q_pos0[b]) // bs, -(-w.C // bs)
        nb = int(w.ctx_len[b]) // bs
        assert w.alive[b, c0:c0 + cb].all()
        ids = w.block_table[b, c0:c0 + cb]
        assert np.array_equal(ids, np.arange(ids[0], ids[0] + cb))
        if c0 > 0 and w.alive[b, c0 - 1]:
            assert w.block_table[b, c0 - 1] != ids[0] - 1
        if w.alive[b, c0 + cb]:
            assert w.block_table[b, c0 + cb] != ids[-1] + 1
        assert w.alive[b, c0 + cb:nb].sum() > 0
        assert 0 < int(w.q_pos0[b]) and int(w.q_pos0[b]) + w.C < int(w.ctx_len[b])
