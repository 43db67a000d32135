"""The Python binding's checks of caller-supplied buffers (CPU, no kernel runs).

The library trusts the sizes it is handed, so the binding must refuse an
output, plan or workspace buffer that is smaller than what the kernels will
write, a buffer on another device, and host tensors (there is no CPU path).
Every case here fails in the binding before any pointer reaches libmsa.
"""
import os

import pytest
import torch

import kv_cache_attention_msa_amd as msa
from kv_cache_attention_msa_amd import _lib

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="libmsa.so not built")


def i32(*shape):
    return torch.zeros(shape, dtype=torch.int32)


def bf16(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def plan_inputs(B=2, nb=8):
    return i32(B, nb), torch.zeros((B, nb), dtype=torch.uint8), i32(B)


def test_plan_refuses_segs_shorter_than_the_capacity():
    t, a, c = plan_inputs()
    with pytest.raises(ValueError, match="seg_capacity 16 exceeds the 4 rows"):
        msa.msa_plan_segments(t, a, c, 16, 100, seg_capacity=16, segs=i32(4, 6))


def test_plan_takes_the_capacity_from_a_given_segs_buffer():
    # without seg_capacity the capacity is the buffer's row count, not
    # B * max_blocks; the call then stops only at the host-tensor check
    t, a, c = plan_inputs()
    with pytest.raises(ValueError, match="device"):
        msa.msa_plan_segments(t, a, c, 16, 100, segs=i32(4, 6))


@pytest.mark.parametrize("kw,msg", [
    (dict(segs=i32(16, 5)), r"segs must be \[N, 6\]"),
    (dict(seg_indptr=i32(2)), r"seg_indptr must have shape \(3,\)"),
    (dict(dev_error=i32(2)), r"dev_error must have shape \(1,\)"),
])
def test_plan_refuses_misshapen_buffers(kw, msg):
    t, a, c = plan_inputs()
    with pytest.raises(ValueError, match=msg):
        msa.msa_plan_segments(t, a, c, 16, 100, **kw)


def test_plan_refuses_host_tensors():
    t, a, c = plan_inputs()
    with pytest.raises(ValueError, match="device"):
        msa.msa_plan_segments(t, a, c, 16, 100)


def decode_inputs(B=2, Hq=8, Hkv=2, D=64, P=10):
    return bf16(B, Hq, D), bf16(P, 16, Hkv, D), bf16(P, 16, Hkv, D), i32(8, 6), i32(B + 1)


@pytest.mark.parametrize("kw,msg", [
    (dict(out=bf16(2, 8, 32)), r"out must have shape \(2, 8, 64\)"),
    (dict(out=torch.zeros((2, 8, 64))), "out must be torch.bfloat16"),
    (dict(lse=torch.zeros((2, 4))), r"lse must have shape \(2, 8\)"),
    (dict(lse=bf16(2, 8)), "lse must be torch.float32"),
])
def test_decode_refuses_misshapen_outputs(kw, msg):
    q, k, v, segs, ind = decode_inputs()
    with pytest.raises(ValueError, match=msg):
        msa.msa_decode(q, k, v, segs, ind, max_ctx_len=64, **kw)


def test_decode_refuses_a_bad_segment_table_and_host_tensors():
    q, k, v, segs, ind = decode_inputs()
    with pytest.raises(ValueError, match=r"segs must be \[N, 6\]"):
        msa.msa_decode(q, k, v, i32(8, 4), ind, max_ctx_len=64)
    with pytest.raises(ValueError, match="device"):
        msa.msa_decode(q, k, v, segs, ind, max_ctx_len=64)


@pytest.mark.parametrize("kw,msg", [
    (dict(out=bf16(2, 16, 8, 64)), r"out must have shape \(2, 32, 8, 64\)"),
    (dict(lse=torch.zeros((2, 32, 4))), r"lse must have shape \(2, 32, 8\)"),
])
def test_prefill_refuses_misshapen_outputs(kw, msg):
    q = bf16(2, 32, 8, 64)
    _, k, v, segs, ind = decode_inputs()
    with pytest.raises(ValueError, match=msg):
        msa.msa_prefill_chunk(q, i32(2), k, v, segs, ind, max_ctx_len=64, **kw)


@pytest.mark.parametrize("kw,msg", [
    (dict(out=torch.zeros((2, 1, 4, 32))), r"out must have shape \(2, 1, 4, 64\)"),
    (dict(lse=torch.zeros((2, 1, 3))), r"lse must have shape \(2, 1, 4\)"),
])
def test_merge_refuses_misshapen_outputs(kw, msg):
    o, m, l = torch.zeros((5, 1, 4, 64)), torch.zeros((5, 1, 4)), torch.zeros((5, 1, 4))
    with pytest.raises(ValueError, match=msg):
        msa.msa_merge_partials(o, m, l, i32(3), **kw)


@pytest.mark.parametrize("kw,msg", [
    (dict(dense_k=bf16(15, 16, 2, 64)), r"dense_k must have shape \(16, 16, 2, 64\)"),
    (dict(dense_segs=i32(1, 6)), r"dense_segs must have shape \(2, 6\)"),
    (dict(dense_indptr=i32(2)), r"dense_indptr must have shape \(3,\)"),
])
def test_gather_refuses_misshapen_outputs(kw, msg):
    _, k, v, segs, ind = decode_inputs()
    with pytest.raises(ValueError, match=msg):
        msa.msa_gather_alive(k, v, segs, ind, 8, **kw)


def test_layout_argument():
    q, k, v, segs, ind = decode_inputs()
    with pytest.raises(ValueError, match="kv_layout must be 'NHD' or 'HND'"):
        msa.msa_decode(q, k, v, segs, ind, max_ctx_len=64, kv_layout="NDH")
    # head-major pools [P, Hkv, 16, D]: the shapes are read in that order, so
    # a well-formed call only stops at the host-tensor check
    kh, vh = k.permute(0, 2, 1, 3).contiguous(), v.permute(0, 2, 1, 3).contiguous()
    with pytest.raises(ValueError, match="device"):
        msa.msa_decode(q, kh, vh, segs, ind, max_ctx_len=64, kv_layout="HND")
    # a head dimension that disagrees with q's is refused
    with pytest.raises(ValueError, match="shape mismatch"):
        msa.msa_decode(q, bf16(10, 2, 16, 32), bf16(10, 2, 16, 32), segs, ind, max_ctx_len=64,
                       kv_layout="HND")


def test_unprefixed_names_are_the_same_calls():
    for short in ("plan_segments", "decode", "prefill_chunk", "merge_partials", "prefill_chunk_rows",
                  "gather_alive"):
        assert getattr(msa, short) is getattr(msa, "msa_" + short)
        assert short in msa.__all__
