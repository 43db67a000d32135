"""Pins for the oracle's attention, partials and merge (rows a3, a4, a5).

The oracle's claim is the lossless one (P2, Abstract; P1 "它在解决什么真问题"):
MSA over the alive blocks equals dense softmax attention over the alive
tokens, in logical order, causally masked by logical position.  The pins
below fix it against things other than itself:

* closed forms (one visible key, zero query, two keys, no visible key);
* a library reduction: torch's scaled_dot_product_attention in float64 on a
  dense per-position K/V, with evicted positions removed by its mask; the
  pool the oracle reads is built from that dense K/V by scattering;
* a scalar-loop brute force over logical positions on tiny inputs;
* invariants: physical relayout, dead-slot garbage, eviction + recovery at a
  new slot, GQA row equality, key-order independence, merge associativity;
* bf16 decoding against torch's own bf16 -> float64 conversion;
* mutation checks: plausible mistakes planted into a copy of the oracle make
  at least one of these pins fail.
"""
import math
import types

import numpy as np
import pytest
import torch

import oracle
from oracle import msa_oracle
from workloads import make_workload, f32_to_bf16_bits

torch.set_num_threads(4)


# ----------------------------------------------------------------------------
# building caches from dense per-position K/V (the inverse of the oracle's read)
# ----------------------------------------------------------------------------

def scatter_cache(rng, k_dense, v_dense, alive, bs, pool_blocks, poison=np.nan):
    """Place dense per-sequence K/V [B][ctx, Hkv, D] into a paged pool.

    Each alive logical block gets a random distinct physical block; dead
    blocks get -1.  Unused slots are filled with `poison`.
    """
    B = len(k_dense)
    Hkv, D = k_dense[0].shape[1:]
    nbs = [-(-len(k) // bs) for k in k_dense]
    max_nb = max(nbs)
    table = np.full((B, max_nb), -1, dtype=np.int32)
    kp = np.full((pool_blocks, bs, Hkv, D), poison, dtype=np.float64)
    vp = np.full((pool_blocks, bs, Hkv, D), poison, dtype=np.float64)
    slots = iter(rng.permutation(pool_blocks))
    for b in range(B):
        for p in range(len(k_dense[b])):
            l = p // bs
            if not alive[b, l]:
                continue
            if table[b, l] < 0:
                table[b, l] = next(slots)
            kp[table[b, l], p % bs] = k_dense[b][p]
            vp[table[b, l], p % bs] = v_dense[b][p]
    ctx = np.array([len(k) for k in k_dense], dtype=np.int32)
    return table, kp, vp, ctx


def sdpa_reference(q, qpos, k_dense, v_dense, kmask, scale, G):
    """torch SDPA, float64.  q [R, Hq, D]; k/v [N, Hkv, D]; kmask [N] keeps."""
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]        # [1,Hq,R,D]
    kt = torch.from_numpy(np.ascontiguousarray(k_dense.transpose(1, 0, 2)))
    vt = torch.from_numpy(np.ascontiguousarray(v_dense.transpose(1, 0, 2)))
    kt = kt.repeat_interleave(G, dim=0)[None]
    vt = vt.repeat_interleave(G, dim=0)[None]
    N = k_dense.shape[0]
    pos = torch.arange(N)
    mask = (pos[None, :] <= torch.from_numpy(np.asarray(qpos))[:, None]) & torch.from_numpy(kmask)[None, :]
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    s = (qt @ kt.transpose(-1, -2)) * scale
    s = s.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return out[0].permute(1, 0, 2).numpy(), lse[0].permute(1, 0).numpy()


def _random_case(seed, B=3, Hkv=2, G=3, D=8, bs=4, ctx_lo=5, ctx_hi=40, p_alive=0.7):
    rng = np.random.default_rng(seed)
    ctxs = rng.integers(ctx_lo, ctx_hi, size=B)
    kd = [rng.standard_normal((int(c), Hkv, D)) for c in ctxs]
    vd = [rng.standard_normal((int(c), Hkv, D)) for c in ctxs]
    max_nb = -(-int(ctxs.max()) // bs)
    alive = (rng.random((B, max_nb)) < p_alive).astype(np.uint8)
    for b in range(B):
        alive[b, (int(ctxs[b]) - 1) // bs] = 1
    table, kp, vp, ctx = scatter_cache(rng, kd, vd, alive, bs, pool_blocks=B * max_nb + 7)
    return rng, kd, vd, alive, table, kp, vp, ctx


# ----------------------------------------------------------------------------
# pin checks, parameterised by an oracle module so mutants can be run through
# ----------------------------------------------------------------------------

def pin_closed_forms(orc):
    rng = np.random.default_rng(1)
    D, bs = 8, 4
    scale = 0.37
    # one visible key: O = v exactly, LSE = s
    k = rng.standard_normal((1, 1, D)); v = rng.standard_normal((1, 1, D))
    q = rng.standard_normal((1, 1, D))
    table, kp, vp, ctx = scatter_cache(rng, [k], [v], np.ones((1, 1), np.uint8), bs, 3)
    O, L = orc.decode_ref(q, kp, vp, table, np.ones((1, 1), np.uint8), ctx, bs, scale)
    assert np.array_equal(O[0, 0], v[0, 0])
    assert abs(L[0, 0] - scale * float(np.dot(q[0, 0], k[0, 0]))) < 1e-14
    # zero query: O = mean of alive V, LSE = ln(n alive)
    n = 11
    kd = rng.standard_normal((n, 1, D)); vd = rng.standard_normal((n, 1, D))
    alive = np.array([[1, 0, 1]], np.uint8)
    table, kp, vp, ctx = scatter_cache(rng, [kd], [vd], alive, bs, 9)
    O, L = orc.decode_ref(np.zeros((1, 1, D)), kp, vp, table, alive, ctx, bs, scale)
    kept = [p for p in range(n) if alive[0, p // bs]]
    assert np.allclose(O[0, 0], vd[kept, 0].mean(axis=0), atol=1e-14, rtol=0)
    assert abs(L[0, 0] - math.log(len(kept))) < 1e-14
    # two keys: (e^s1 v1 + e^s2 v2) / (e^s1 + e^s2)
    kd = rng.standard_normal((2, 1, D)); vd = rng.standard_normal((2, 1, D))
    q = rng.standard_normal((1, 1, D))
    table, kp, vp, ctx = scatter_cache(rng, [kd], [vd], np.ones((1, 1), np.uint8), bs, 4)
    O, L = orc.decode_ref(q, kp, vp, table, np.ones((1, 1), np.uint8), ctx, bs, scale)
    s1 = scale * sum(q[0, 0, d] * kd[0, 0, d] for d in range(D))
    s2 = scale * sum(q[0, 0, d] * kd[1, 0, d] for d in range(D))
    e1, e2 = math.exp(s1), math.exp(s2)
    want = (e1 * vd[0, 0] + e2 * vd[1, 0]) / (e1 + e2)
    assert np.allclose(O[0, 0], want, atol=1e-14, rtol=0)
    assert abs(L[0, 0] - math.log(e1 + e2)) < 1e-13
    # prefill row before every alive key: nothing visible -> O = 0, LSE = -inf
    kd = rng.standard_normal((8, 1, D)); vd = rng.standard_normal((8, 1, D))
    alive = np.array([[0, 1]], np.uint8)
    table, kp, vp, ctx = scatter_cache(rng, [kd], [vd], alive, bs, 4)
    qq = rng.standard_normal((1, 2, 1, D))
    O, L = orc.prefill_ref(qq, np.array([2]), kp, vp, table, alive, ctx, bs, scale)
    assert np.all(O[0, :, 0] == 0) and np.all(np.isneginf(L[0, :, 0]))


def pin_sdpa_decode(orc, seed=0):
    rng, kd, vd, alive, table, kp, vp, ctx = _random_case(seed)
    B, Hkv, G, D, bs = len(kd), 2, 3, 8, 4
    q = rng.standard_normal((B, Hkv * G, D))
    scale = 1 / math.sqrt(D)
    O, L = orc.decode_ref(q, kp, vp, table, alive, ctx, bs, scale)
    for b in range(B):
        kmask = np.array([bool(alive[b, p // bs]) for p in range(int(ctx[b]))])
        o, l = sdpa_reference(q[b][None], [int(ctx[b]) - 1], kd[b], vd[b], kmask, scale, G)
        assert np.allclose(O[b], o[0], atol=1e-12, rtol=0)
        assert np.allclose(L[b], l[0], atol=1e-12, rtol=0)


def pin_sdpa_prefill(orc, seed=0):
    rng, kd, vd, alive, table, kp, vp, ctx = _random_case(seed, ctx_lo=20, ctx_hi=40)
    B, Hkv, G, D, bs = len(kd), 2, 3, 8, 4
    C = 9
    q = rng.standard_normal((B, C, Hkv * G, D))
    q_pos0 = np.array([int(rng.integers(0, int(c) - C + 1)) for c in ctx])
    scale = 0.29
    O, L = orc.prefill_ref(q, q_pos0, kp, vp, table, alive, ctx, bs, scale)
    for b in range(B):
        kmask = np.array([bool(alive[b, p // bs]) for p in range(int(ctx[b]))])
        qpos = q_pos0[b] + np.arange(C)
        o, l = sdpa_reference(q[b], qpos, kd[b], vd[b], kmask, scale, G)
        vis = np.array([kmask[:qp + 1].any() for qp in qpos])
        assert np.allclose(O[b][vis], o[vis], atol=1e-12, rtol=0)
        assert np.allclose(L[b][vis], l[vis], atol=1e-12, rtol=0)
        assert np.all(O[b][~vis] == 0) and np.all(np.isneginf(L[b][~vis]))


def pin_brute_force_loops(orc, seed=3):
    """Scalar loops over logical positions, math.exp, on a tiny cache."""
    rng, kd, vd, alive, table, kp, vp, ctx = _random_case(seed, B=2, ctx_lo=3, ctx_hi=18)
    B, Hkv, G, D, bs = 2, 2, 3, 8, 4
    scale = 0.41
    q = rng.standard_normal((B, Hkv * G, D))
    O, L = orc.decode_ref(q, kp, vp, table, alive, ctx, bs, scale)
    for b in range(B):
        for h in range(Hkv * G):
            g = h // G
            scores, vals = [], []
            for p in range(int(ctx[b])):
                if not alive[b, p // bs]:
                    continue
                blk, slot = table[b, p // bs], p % bs
                scores.append(scale * sum(q[b, h, d] * kp[blk, slot, g, d] for d in range(D)))
                vals.append([vp[blk, slot, g, d] for d in range(D)])
            mx = max(scores)
            ws = [math.exp(s - mx) for s in scores]
            tot = sum(ws)
            want = [sum(w * v[d] for w, v in zip(ws, vals)) / tot for d in range(D)]
            assert np.allclose(O[b, h], want, atol=1e-13, rtol=0)
            assert abs(L[b, h] - (mx + math.log(tot))) < 1e-13


def pin_merge(orc, seed=7):
    """Partials over arbitrary key splits, merged, equal whole attention;
    single-partial and all-empty closed forms."""
    rng = np.random.default_rng(seed)
    R, H, D, N = 3, 2, 5, 23
    q = rng.standard_normal((R, H, D)); k = rng.standard_normal((N, H, D)); v = rng.standard_normal((N, H, D))
    qpos = np.array([5, 14, 22]); kpos = np.arange(N)
    scale = 0.8
    for nparts in (1, 2, 5):
        cuts = np.sort(rng.choice(np.arange(1, N), size=nparts - 1, replace=False)) if nparts > 1 else []
        bounds = [0, *cuts, N]
        o_p = np.zeros((nparts, R, H, D)); m_p = np.zeros((nparts, R, H)); l_p = np.zeros((nparts, R, H))
        for i in range(nparts):
            sl = slice(bounds[i], bounds[i + 1])
            for h in range(H):
                m, l, o = orc.partial_ref(q[:, h], qpos, k[sl, h], v[sl, h], kpos[sl], scale)
                m_p[i, :, h], l_p[i, :, h], o_p[i, :, h] = m, l, o
        O, L = orc.merge_ref(o_p, m_p, l_p, np.array([0, nparts]))
        for h in range(H):
            o_ref, l_ref = orc.attention_ref(q[:, h], qpos, k[:, h], v[:, h], kpos, scale)
            assert np.allclose(O[0, :, h], o_ref, atol=1e-13, rtol=0)
            assert np.allclose(L[0, :, h], l_ref, atol=1e-13, rtol=0)
    # one partial: O = o / l, LSE = m + ln l
    o1 = rng.standard_normal((1, 1, 1, D)); m1 = np.array([[[0.3]]]); l1 = np.array([[[2.5]]])
    O, L = orc.merge_ref(o1, m1, l1, np.array([0, 1]))
    assert np.allclose(O[0, 0, 0], o1[0, 0, 0] / 2.5, atol=1e-15, rtol=0)
    assert abs(L[0, 0, 0] - (0.3 + math.log(2.5))) < 1e-15
    # empty partials (m = -inf) carry no weight, even with garbage o
    o2 = np.concatenate([o1, np.full((1, 1, 1, D), np.nan)])
    m2 = np.array([[[0.3]], [[-np.inf]]]); l2 = np.array([[[2.5]], [[0.0]]])
    O2, L2 = orc.merge_ref(o2, m2, l2, np.array([0, 2]))
    assert np.array_equal(O2, O) and np.array_equal(L2, L)
    # nothing at all: O = 0, LSE = -inf
    O3, L3 = orc.merge_ref(o2[1:], m2[1:], l2[1:], np.array([0, 1, 1]))
    assert np.all(O3 == 0) and np.all(np.isneginf(L3))


def pin_bf16_decoding(orc):
    rng = np.random.default_rng(2)
    x = rng.standard_normal(4096).astype(np.float32) * 10.0 ** rng.integers(-30, 30, size=4096)
    bits = f32_to_bf16_bits(x)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(orc.to_f64(bits), want)


def pin_workload_sdpa(orc):
    """A bf16 workload family at reduced size, one sequence, against SDPA on
    the positions read back through torch's own bf16 conversion."""
    w = make_workload(2, seed=4, size="small", B=2, ctx=400)
    b = 1
    G = w.Hq // w.Hkv
    ctx = int(w.ctx_len[b])
    kd = np.zeros((ctx, w.Hkv, w.D)); vd = np.zeros((ctx, w.Hkv, w.D))
    kmask = np.zeros(ctx, bool)
    tk = torch.from_numpy(w.k_pool.view(np.int16)).view(torch.bfloat16)
    tv = torch.from_numpy(w.v_pool.view(np.int16)).view(torch.bfloat16)
    for p in range(ctx):
        l = p // w.block_size
        if w.alive[b, l]:
            kmask[p] = True
            kd[p] = tk[w.block_table[b, l], p % w.block_size].double().numpy()
            vd[p] = tv[w.block_table[b, l], p % w.block_size].double().numpy()
    qd = torch.from_numpy(w.q.view(np.int16)).view(torch.bfloat16).double().numpy()
    O, L = orc.decode_ref(w.q, w.k_pool, w.v_pool, w.block_table, w.alive, w.ctx_len,
                          w.block_size, w.scale, seqs=[b])
    o, l = sdpa_reference(qd[b][None], [ctx - 1], kd, vd, kmask, w.scale, G)
    assert np.allclose(O[b], o[0], atol=1e-12, rtol=0)
    assert np.allclose(L[b], l[0], atol=1e-12, rtol=0)


PINS = [pin_closed_forms, pin_sdpa_decode, pin_sdpa_prefill, pin_brute_force_loops,
        pin_merge, pin_bf16_decoding, pin_workload_sdpa]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)


@pytest.mark.parametrize("seed", range(1, 6))
def test_sdpa_more_seeds(seed):
    pin_sdpa_decode(oracle, seed)
    pin_sdpa_prefill(oracle, seed)


# ----------------------------------------------------------------------------
# invariants
# ----------------------------------------------------------------------------

def _small_bf16():
    return make_workload(2, seed=11, size="small", B=3, ctx=700)


def test_segmentation_independence():
    """Same alive content under another physical layout (all alive blocks of a
    sequence packed contiguously vs scattered) gives the same result."""
    w = _small_bf16()
    O1, L1 = oracle.decode_ref(w.q, w.k_pool, w.v_pool, w.block_table, w.alive, w.ctx_len,
                               w.block_size, w.scale)
    rng = np.random.default_rng(0)
    for mode in ("packed", "shuffled"):
        P = w.num_phys_blocks
        kp = np.full_like(w.k_pool, 0x7FC0); vp = np.full_like(w.v_pool, 0x7FC0)
        table = np.full_like(w.block_table, -1)
        order = np.arange(P) if mode == "packed" else rng.permutation(P)
        nxt = 0
        for b in range(w.B):
            for l in range(w.max_blocks):
                if w.alive[b, l] and l * w.block_size < w.ctx_len[b]:
                    dst = order[nxt]; nxt += 1
                    kp[dst] = w.k_pool[w.block_table[b, l]]
                    vp[dst] = w.v_pool[w.block_table[b, l]]
                    table[b, l] = dst
        segs, _ = oracle.plan_ref(table, w.alive, w.ctx_len, w.block_size)
        if mode == "packed":
            assert len(segs) <= w.B * 30  # few segments: runs only split at holes
        O2, L2 = oracle.decode_ref(w.q, kp, vp, table, w.alive, w.ctx_len, w.block_size, w.scale)
        assert np.allclose(O1, O2, atol=1e-13, rtol=0)
        assert np.allclose(L1, L2, atol=1e-13, rtol=0)


def test_dead_data_independence():
    w = _small_bf16()
    O1, L1 = oracle.decode_ref(w.q, w.k_pool, w.v_pool, w.block_table, w.alive, w.ctx_len,
                               w.block_size, w.scale)
    nan_bits = np.isnan(oracle.to_f64(w.k_pool))
    kp = w.k_pool.copy(); vp = w.v_pool.copy()
    kp[nan_bits] = 0x7F80  # +inf
    vp[nan_bits] = 0x4780  # 65536.0
    O2, L2 = oracle.decode_ref(w.q, kp, vp, w.block_table, w.alive, w.ctx_len, w.block_size, w.scale)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
    assert np.all(np.isfinite(O1)) and np.all(np.isfinite(L1))


def test_eviction_recovery_round_trip():
    w = _small_bf16()
    args = (w.block_size, w.scale)
    O1, L1 = oracle.decode_ref(w.q, w.k_pool, w.v_pool, w.block_table, w.alive, w.ctx_len, *args)
    b = 1
    l = int(np.flatnonzero(w.alive[b, :w.ctx_len[b] // w.block_size - 1])[3])
    alive = w.alive.copy(); alive[b, l] = 0
    O2, _ = oracle.decode_ref(w.q, w.k_pool, w.v_pool, w.block_table, alive, w.ctx_len, *args)
    assert not np.allclose(O1[b], O2[b], atol=1e-6)
    # recover: copy the block into a free slot appended to the pool
    kp = np.concatenate([w.k_pool, w.k_pool[w.block_table[b, l]][None]])
    vp = np.concatenate([w.v_pool, w.v_pool[w.block_table[b, l]][None]])
    table = w.block_table.copy(); table[b, l] = kp.shape[0] - 1
    O3, L3 = oracle.decode_ref(w.q, kp, vp, table, w.alive, w.ctx_len, *args)
    assert np.allclose(O1, O3, atol=1e-13, rtol=0) and np.allclose(L1, L3, atol=1e-13, rtol=0)


def test_gqa_identical_rows():
    w = _small_bf16()
    q = w.q.copy()
    G = w.Hq // w.Hkv
    q[:, 1::G] = q[:, 0::G]  # second head of each group copies the first
    O, L = oracle.decode_ref(q, w.k_pool, w.v_pool, w.block_table, w.alive, w.ctx_len,
                             w.block_size, w.scale)
    assert np.array_equal(O[:, 1::G], O[:, 0::G]) and np.array_equal(L[:, 1::G], L[:, 0::G])


def test_key_order_independence():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((4, 16)); k = rng.standard_normal((50, 16)); v = rng.standard_normal((50, 16))
    qp = np.array([10, 20, 30, 60]); kp = rng.permutation(50)
    o1, l1 = oracle.attention_ref(q, qp, k, v, kp, 0.25)
    perm = rng.permutation(50)
    o2, l2 = oracle.attention_ref(q, qp, k[perm], v[perm], kp[perm], 0.25)
    assert np.allclose(o1, o2, atol=1e-14, rtol=0) and np.allclose(l1, l2, atol=1e-14, rtol=0)


# ----------------------------------------------------------------------------
# mutation checks: a planted mistake in a copy of the oracle fails a pin
# ----------------------------------------------------------------------------

MUTANTS = {
    "dropped_scale": ("s = scale * (q_rows @ keys.T)", "s = (q_rows @ keys.T)"),
    "mask_off_by_one": ("vis = np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None]\n    s = np.where(vis, s, -np.inf)\n    m = s.max(axis=1)\n    has = np.isfinite(m)\n    w = np.zeros_like(s)\n    w[has] = np.exp(s[has] - m[has, None])\n    w[~vis] = 0.0\n    den",
                        "vis = np.asarray(k_pos)[None, :] < np.asarray(q_pos)[:, None]\n    s = np.where(vis, s, -np.inf)\n    m = s.max(axis=1)\n    has = np.isfinite(m)\n    w = np.zeros_like(s)\n    w[has] = np.exp(s[has] - m[has, None])\n    w[~vis] = 0.0\n    den"),
    "gqa_mapping": ("by_kv.setdefault(h // G, [])", "by_kv.setdefault(h % Hkv, [])"),
    "lse_without_max": ("lse[has] = m[has] + np.log(den[has])", "lse[has] = np.log(den[has])"),
    "merge_unweighted_l": ("L = (w * l_part[lo:hi]).sum(axis=0)", "L = l_part[lo:hi].sum(axis=0)"),
    "bf16_shift": ("<< np.uint32(16)).view(np.float32)", "<< np.uint32(15)).view(np.float32)"),
    "slot_index": ("return phys, pos % bs, pos", "return phys, (pos + 1) % bs, pos"),
    "partial_unnormalised_o": ("    l = w.sum(axis=1)\n    o = w @ values", "    l = w.sum(axis=1)\n    o = (w @ values) / l[:, None]"),
}

PLAN_MUTANTS = {
    "plan_ignores_logical_hole": ("cur[1] + cur[3] == l and cur[2] + cur[3] == p", "cur[2] + cur[3] == p"),
    "plan_ignores_physical": ("cur[1] + cur[3] == l and cur[2] + cur[3] == p", "cur[1] + cur[3] == l"),
    "plan_start_in_blocks": ("running += cur[4]", "running += cur[3]"),
    "plan_full_last_block": ("tokens_here = min(bs, n_tok - l * bs)", "tokens_here = bs"),
}


def _mutant(old, new):
    src_path = msa_oracle.__file__
    with open(src_path) as f:
        src = f.read()
    assert src.count(old) >= 1, old
    mod = types.ModuleType("oracle_mutant")
    # the first occurrence is the one in the function the mutant targets
    exec(compile(src.replace(old, new, 1), "<mutant>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(*MUTANTS[name])
    failures = 0
    for pin in PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError):
            failures += 1
    assert failures >= 1, f"no pin catches mutant {name}"


@pytest.mark.parametrize("name", sorted(PLAN_MUTANTS))
def test_plan_mutant_is_caught(name):
    from tests.test_oracle_plan import brute_force_plan
    from workloads import random_small_case
    mod = _mutant(*PLAN_MUTANTS[name])
    caught = False
    for seed in range(60):
        rng = np.random.default_rng(1000 + seed)
        table, alive, ctx, bs, _ = random_small_case(rng, max_nb=9)
        segs, indptr = mod.plan_ref(table, alive, ctx, bs)
        bsegs, bindptr = brute_force_plan(table, alive, ctx, bs)
        if segs.tolist() != bsegs.tolist() or indptr.tolist() != bindptr.tolist():
            caught = True
            break
    assert caught, f"brute force does not catch plan mutant {name}"
