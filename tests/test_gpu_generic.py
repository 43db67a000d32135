"""GPU parity of the generic kernel against the fp64 oracle.

The (dtype, head_dim) pairs that the specialised kernels are not built for
run on one plain vector-ALU kernel in float32: decode in float32 with D 128,
prefill in bfloat16 with D 64 and in float32 with D 64 and 128.  Same bars as
the other parity tests: max-abs-error <= 1e-5 for float32 inputs and <= 2e-2
for bfloat16 inputs, on O and LSE, element by element.  Covers every GQA
group size, forced key splits (partials merged by log-sum-exp), a chunk in
the middle of the context, both pool layouts, sequences without keys and
an understated max_ctx_len (the cut is reported).
"""
import numpy as np
import pytest
import torch

import oracle
import kv_cache_attention_msa_amd as msa
from kv_cache_attention_msa_amd import _lib
from workloads import make_workload
from workloads.device import to_device, tensor, from_device

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = {"f32": 1e-5, "bf16": 2e-2}


def _plan(w, d):
    return msa.msa_plan_segments(d["block_table"], d["alive"], d["ctx_len"], w.block_size,
                                 w.num_phys_blocks)


def _hnd(d):
    d = dict(d)
    d["k_pool"] = d["k_pool"].permute(0, 2, 1, 3).contiguous()
    d["v_pool"] = d["v_pool"].permute(0, 2, 1, 3).contiguous()
    return d


def _check(O, L, Or, Lr, tol):
    sel = ~np.isnan(Lr)
    assert np.all(np.isneginf(L[sel & np.isneginf(Lr)]))
    fin = sel & np.isfinite(Lr)
    e_o = float(np.max(np.abs(O - Or)[~np.isnan(Or)])) if (~np.isnan(Or)).any() else 0.0
    e_l = float(np.max(np.abs(L[fin] - Lr[fin]))) if fin.any() else 0.0
    assert e_o <= tol, f"max |O - ref| = {e_o}"
    assert e_l <= tol, f"max |LSE - ref| = {e_l}"
    return e_o, e_l


def run_decode(w, split_blocks=0, layout="NHD", kernel="auto", max_ctx=None, expect_err=0):
    d = to_device(w, DEV)
    if layout == "HND":
        d = _hnd(d)
    segs, indptr, err = _plan(w, d)
    out, lse = msa.msa_decode(d["q"], d["k_pool"], d["v_pool"], segs, indptr,
                              max_ctx_len=int(w.ctx_len.max()) if max_ctx is None else max_ctx,
                              scale=w.scale, split_blocks=split_blocks, kv_layout=layout,
                              kernel=kernel, dev_error=err)
    torch.cuda.synchronize()
    assert int(err.item()) == expect_err
    return from_device(out), lse.cpu().numpy().astype(np.float64)


def check_decode(w, O, L):
    Or, Lr = oracle.decode_ref(w.q, w.k_pool, w.v_pool, w.block_table, w.alive, w.ctx_len,
                               w.block_size, w.scale)
    return _check(O, L, Or, Lr, TOL[w.dtype])


def run_prefill(w, split_blocks=0, layout="NHD"):
    d = to_device(w, DEV)
    if layout == "HND":
        d = _hnd(d)
    segs, indptr, err = _plan(w, d)
    out, lse = msa.msa_prefill_chunk(d["q"], d["q_pos0"], d["k_pool"], d["v_pool"], segs, indptr,
                                     max_ctx_len=max(1, int(w.ctx_len.max())), scale=w.scale,
                                     split_blocks=split_blocks, kv_layout=layout, dev_error=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    return from_device(out), lse.cpu().numpy().astype(np.float64)


def check_prefill(w, O, L):
    Or, Lr = oracle.prefill_ref(w.q, w.q_pos0, w.k_pool, w.v_pool, w.block_table, w.alive,
                                w.ctx_len, w.block_size, w.scale)
    return _check(O, L, Or, Lr, TOL[w.dtype])


def test_generic_shapes_are_available():
    assert msa.decode_available(_lib.MSA_F32, 128, 4)
    for dt, D in ((_lib.MSA_BF16, 64), (_lib.MSA_F32, 64), (_lib.MSA_F32, 128)):
        assert msa.prefill_available(dt, D, 4)


# ---- decode, float32, D 128 -------------------------------------------------

@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("split_blocks", [0, 16])
def test_decode_f32_d128(G, split_blocks):
    w = make_workload(1, seed=G, D=128, Hkv=2, Hq=2 * G, B=3, nb=40, pool=160, n_evict=10)
    O, L = run_decode(w, split_blocks)
    check_decode(w, O, L)


def test_decode_f32_d128_vector_kernel_and_head_major():
    w = make_workload(1, seed=11, D=128, B=2, nb=50, pool=200, n_evict=12)
    O1, L1 = run_decode(w, 0, kernel="vector")
    check_decode(w, O1, L1)
    O2, L2 = run_decode(w, 0, layout="HND")
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_decode_f32_d128_matrix_and_block_kernels_not_built():
    w = make_workload(1, seed=12, D=128)
    for k in ("matrix", "block"):
        with pytest.raises(msa.MsaError):
            run_decode(w, 0, kernel=k)


def test_decode_f32_d128_truncation_is_reported():
    # max_ctx_len 128 tokens: the automatic split gives the grid room for 32
    # alive blocks per sequence (one split of 32), below the 35 each holds,
    # so every sequence is cut there and the cut is reported
    w = make_workload(1, seed=13, D=128, B=2, nb=40, pool=160, n_evict=5)
    O, L = run_decode(w, 0, max_ctx=128, expect_err=_lib.MSA_DEVERR_TRUNCATED)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))


# ---- prefill, bf16 D 64 and float32 D 64 / 128 ------------------------------

PREFILL_SHAPES = [("bf16", 64), ("f32", 64), ("f32", 128)]


@pytest.mark.parametrize("dtype,D", PREFILL_SHAPES)
@pytest.mark.parametrize("split_blocks", [0, 16])
def test_prefill_generic_small(dtype, D, split_blocks):
    w = make_workload(3, seed=5, size="small", dtype=dtype, D=D, Hq=8, Hkv=2, C=40)
    O, L = run_prefill(w, split_blocks)
    check_prefill(w, O, L)


@pytest.mark.parametrize("dtype,D", PREFILL_SHAPES)
@pytest.mark.parametrize("G", [1, 2, 8])
def test_prefill_generic_group_sizes(dtype, D, G):
    w = make_workload(3, seed=6 + G, size="small", dtype=dtype, D=D, Hkv=2, Hq=2 * G, C=33,
                      cached=512)
    O, L = run_prefill(w)
    check_prefill(w, O, L)


@pytest.mark.parametrize("dtype,D", PREFILL_SHAPES)
def test_prefill_generic_mid_context_and_head_major(dtype, D):
    # the chunk sits in the middle of the context: later alive blocks are
    # hidden by the causal mask alone
    w = make_workload(6, seed=9, size="small", dtype=dtype, D=D, Hq=8, Hkv=2)
    O1, L1 = run_prefill(w)
    check_prefill(w, O1, L1)
    O2, L2 = run_prefill(w, layout="HND")
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_prefill_generic_sequence_without_keys():
    # every block of sequence 0 evicted: its rows see no key (O = 0, LSE = -inf)
    w = make_workload(3, seed=21, size="small", dtype="f32", D=64, Hq=8, Hkv=2, C=32, cached=256)
    w.alive[0, :] = 0
    O, L = run_prefill(w)
    assert np.all(O[0] == 0) and np.all(np.isneginf(L[0]))
    check_prefill(w, O, L)
