"""Multi-Segment Attention (MSA) on MI355X: thin PyTorch binding of libmsa.

The calls mirror the C ABI in include/msa.h one to one; this module
only checks tensor shapes/dtypes/devices, allocates outputs and workspaces
with torch (device memory plumbing), and passes raw pointers plus the
current HIP stream.  Every step of the computation runs in libmsa's HIP
kernels; there is no CPU or PyTorch fallback, and a missing library raises.

  msa_plan_segments   block table + alive mask -> segment list (a1)
  msa_decode          decode attention over the segments (a2, a3, a5)
  msa_prefill_chunk   chunked-prefill attention over the segments (a2, a4, a5)
  msa_merge_partials  log-sum-exp merge of (m, l, o) partials (a5)
  msa_gather_alive    gather-then-attend baseline: alive blocks -> dense pools

Each is also reachable without the prefix (plan_segments, decode,
prefill_chunk, merge_partials, prefill_chunk_rows, gather_alive).
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import (MsaError, MSA_F32, MSA_BF16, MSA_DEVERR_PHYS_RANGE, MSA_DEVERR_CAPACITY,
                   MSA_DEVERR_CTX_RANGE, MSA_DEVERR_TRUNCATED, MSA_LAYOUT_NHD, MSA_LAYOUT_HND,
                   MSA_DECODE_AUTO, MSA_DECODE_VECTOR, MSA_DECODE_MATRIX,
                   MSA_DECODE_BLOCK)

__all__ = ["msa_plan_segments", "msa_decode", "msa_prefill_chunk", "msa_merge_partials",
           "msa_prefill_chunk_rows",
           "msa_plan_workspace_size", "msa_decode_workspace_size", "msa_prefill_workspace_size",
           "MsaError", "MSA_F32", "MSA_BF16", "MSA_DEVERR_PHYS_RANGE", "MSA_DEVERR_CAPACITY",
           "MSA_DEVERR_CTX_RANGE", "MSA_DEVERR_TRUNCATED", "MSA_LAYOUT_NHD", "MSA_LAYOUT_HND",
           "MSA_DECODE_AUTO", "MSA_DECODE_VECTOR", "MSA_DECODE_MATRIX", "MSA_DECODE_BLOCK", "SEG_FIELDS",
           "library_path", "prefill_available", "decode_available",
           "plan_segments", "decode", "prefill_chunk", "merge_partials", "prefill_chunk_rows",
           "gather_alive"]

SEG_FIELDS = ("seq", "logical_block", "phys_block", "num_blocks", "num_tokens",
              "alive_token_start")


def library_path() -> str:
    return _lib.LIB_PATH


def prefill_available(dtype: int = MSA_BF16, D: int = 128, G: int = 4) -> bool:
    """True if libmsa was built with the chunked-prefill kernel for this shape."""
    return bool(_lib.load().msa_attention_supported(1, dtype, D, G, 16))


def decode_available(dtype: int = MSA_BF16, D: int = 128, G: int = 4) -> bool:
    """True if libmsa was built with the decode kernel for this shape."""
    return bool(_lib.load().msa_attention_supported(0, dtype, D, G, 16))


def _lib_handle():
    return _lib.load()


def _dev_ptr(t: torch.Tensor | None, name: str):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_enum(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MSA_BF16
    if t.dtype == torch.float32:
        return MSA_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _expect(t, dtype, name, ndim=None):
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")


def _expect_shape(t, shape, dtype, name):
    """A caller-supplied buffer must be exactly what the kernels will write:
    the library trusts the sizes it is given, so a short buffer would be
    written past its end on the device."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _same_device(dev, **tensors):
    for name, t in tensors.items():
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")


def _segs_table(segs):
    _expect(segs, torch.int32, "segs", 2)
    if segs.shape[1] != 6:
        raise ValueError(f"segs must be [N, 6] int32 records, got shape {tuple(segs.shape)}")


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


_LAYOUTS = {"NHD": MSA_LAYOUT_NHD, "HND": MSA_LAYOUT_HND}
_KERNELS = {"auto": MSA_DECODE_AUTO, "vector": MSA_DECODE_VECTOR, "matrix": MSA_DECODE_MATRIX,
            "block": MSA_DECODE_BLOCK}


def _pool_dims(k_pool, kv_layout):
    """(P, block_size, Hkv, D) of a pool in layout "NHD" ([P, bs, Hkv, D]) or
    "HND" ([P, Hkv, bs, D]), and the layout's msa_kv_layout value."""
    if kv_layout not in _LAYOUTS:
        raise ValueError(f"kv_layout must be 'NHD' or 'HND', got {kv_layout!r}")
    if kv_layout == "HND":
        P, Hkv, bs, D = k_pool.shape
    else:
        P, bs, Hkv, D = k_pool.shape
    return P, bs, Hkv, D, _LAYOUTS[kv_layout]


# ---------------------------------------------------------------------------
# a1: plan
# ---------------------------------------------------------------------------

def msa_plan_workspace_size(B: int) -> int:
    return int(_lib_handle().msa_plan_workspace_size(B))


def msa_plan_segments(block_table: torch.Tensor, alive: torch.Tensor, ctx_len: torch.Tensor,
                      block_size: int, num_phys_blocks: int, seg_capacity: int | None = None,
                      segs: torch.Tensor | None = None, seg_indptr: torch.Tensor | None = None,
                      dev_error: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                      stream=None):
    """Segment plan.  Returns (segs int32 [seg_capacity, 6], seg_indptr int32 [B+1],
    dev_error int32 [1]); rows of segs beyond seg_indptr[B] are unspecified."""
    lib = _lib_handle()
    _expect(block_table, torch.int32, "block_table", 2)
    _expect(alive, torch.uint8, "alive", 2)
    _expect(ctx_len, torch.int32, "ctx_len", 1)
    B, max_blocks = block_table.shape
    if tuple(alive.shape) != (B, max_blocks) or ctx_len.shape[0] != B:
        raise ValueError("block_table, alive and ctx_len disagree on shape")
    dev = block_table.device
    if segs is not None:
        _segs_table(segs)
        if seg_capacity is None:
            seg_capacity = segs.shape[0]
        elif int(seg_capacity) > segs.shape[0]:
            raise ValueError(f"seg_capacity {seg_capacity} exceeds the {segs.shape[0]} rows of segs")
    cap = B * max_blocks if seg_capacity is None else int(seg_capacity)
    _expect_shape(seg_indptr, (B + 1,), torch.int32, "seg_indptr")
    _expect_shape(dev_error, (1,), torch.int32, "dev_error")
    _same_device(dev, alive=alive, ctx_len=ctx_len, segs=segs, seg_indptr=seg_indptr,
                 dev_error=dev_error, workspace=workspace)
    if segs is None:
        segs = torch.empty((max(cap, 1), 6), dtype=torch.int32, device=dev)
    if seg_indptr is None:
        seg_indptr = torch.empty(B + 1, dtype=torch.int32, device=dev)
    if dev_error is None:
        dev_error = torch.empty(1, dtype=torch.int32, device=dev)
    wsb = int(lib.msa_plan_workspace_size(B))
    if workspace is None:
        workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    st = lib.msa_plan_segments(_dev_ptr(block_table, "block_table"), _dev_ptr(alive, "alive"),
                               _dev_ptr(ctx_len, "ctx_len"), B, max_blocks, block_size,
                               num_phys_blocks, _dev_ptr(segs, "segs"), cap,
                               _dev_ptr(seg_indptr, "seg_indptr"), _dev_ptr(dev_error, "dev_error"),
                               _dev_ptr(workspace, "workspace"), _nbytes(workspace),
                               _stream(stream, dev))
    _lib.check(st, "msa_plan_segments")
    return segs, seg_indptr, dev_error


# ---------------------------------------------------------------------------
# a2/a3/a5: decode
# ---------------------------------------------------------------------------

def msa_decode_workspace_size(B, Hq, Hkv, D, max_ctx_len, block_size=16, split_blocks=0) -> int:
    return int(_lib_handle().msa_decode_workspace_size(B, Hq, Hkv, D, max_ctx_len, block_size,
                                                       split_blocks))


def msa_decode(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, segs: torch.Tensor,
               seg_indptr: torch.Tensor, max_ctx_len: int, scale: float = 0.0,
               split_blocks: int = 0, out: torch.Tensor | None = None,
               lse: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
               want_lse: bool = True, kv_layout: str = "NHD", kernel: str = "auto",
               dev_error: torch.Tensor | None = None, stream=None):
    """Decode attention.  q [B, Hq, D]; pools [P, 16, Hkv, D] (kv_layout "NHD")
    or [P, Hkv, 16, D] ("HND"), same dtype as q.  kernel: "auto", "vector",
    "matrix" or "block" (msa_decode_kernel).  dev_error: optional int32 [1] device word
    into which MSA_DEVERR_TRUNCATED is ORed (pass the plan's).
    Returns (out [B, Hq, D], lse [B, Hq] float32 or None)."""
    lib = _lib_handle()
    if kernel not in _KERNELS:
        raise ValueError(f"kernel must be one of {sorted(_KERNELS)}, got {kernel!r}")
    if q.dim() != 3 or k_pool.dim() != 4 or v_pool.shape != k_pool.shape:
        raise ValueError("q must be [B,Hq,D]; k_pool/v_pool [P,bs,Hkv,D] of equal shape")
    if q.dtype != k_pool.dtype or v_pool.dtype != k_pool.dtype:
        raise ValueError("q, k_pool and v_pool must share a dtype")
    _segs_table(segs)
    _expect(seg_indptr, torch.int32, "seg_indptr", 1)
    B, Hq, D = q.shape
    P, bs, Hkv, Dk, layout = _pool_dims(k_pool, kv_layout)
    if Dk != D or seg_indptr.shape[0] != B + 1:
        raise ValueError("shape mismatch between q, pools and seg_indptr")
    dev = q.device
    _expect_shape(out, (B, Hq, D), q.dtype, "out")
    _expect_shape(lse, (B, Hq), torch.float32, "lse")
    _expect_shape(dev_error, (1,), torch.int32, "dev_error")
    _same_device(dev, k_pool=k_pool, v_pool=v_pool, segs=segs, seg_indptr=seg_indptr, out=out,
                 lse=lse, workspace=workspace, dev_error=dev_error)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    wsb = int(lib.msa_decode_workspace_size(B, Hq, Hkv, D, max_ctx_len, bs, split_blocks))
    if workspace is None and wsb > 0:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
    st = lib.msa_decode_ex(_dev_ptr(q, "q"), _dev_ptr(k_pool, "k_pool"), _dev_ptr(v_pool, "v_pool"),
                           P, bs, _dev_ptr(segs, "segs"), _dev_ptr(seg_indptr, "seg_indptr"),
                           B, Hq, Hkv, D, int(max_ctx_len), _dtype_enum(q), float(scale),
                           int(split_blocks), _dev_ptr(out, "out"), _dev_ptr(lse, "lse"),
                           _dev_ptr(workspace, "workspace"), _nbytes(workspace), layout,
                           _KERNELS[kernel], _dev_ptr(dev_error, "dev_error"), _stream(stream, dev))
    _lib.check(st, "msa_decode_ex")
    return out, lse


# ---------------------------------------------------------------------------
# a2/a4/a5: chunked prefill
# ---------------------------------------------------------------------------

def msa_prefill_workspace_size(B, C, Hq, Hkv, D, max_ctx_len, block_size=16, split_blocks=0) -> int:
    return int(_lib_handle().msa_prefill_workspace_size(B, C, Hq, Hkv, D, max_ctx_len, block_size,
                                                        split_blocks))


def msa_prefill_chunk(q: torch.Tensor, q_pos0: torch.Tensor, k_pool: torch.Tensor,
                      v_pool: torch.Tensor, segs: torch.Tensor, seg_indptr: torch.Tensor,
                      max_ctx_len: int, scale: float = 0.0, split_blocks: int = 0,
                      out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None, want_lse: bool = True,
                      kv_layout: str = "NHD", dev_error: torch.Tensor | None = None, stream=None):
    """Chunked-prefill attention.  q [B, C, Hq, D] bf16 or float32 (the pools'
    dtype); q_pos0 int32 [B]; pools
    and dev_error as for msa_decode.
    Returns (out [B, C, Hq, D], lse [B, C, Hq] float32 or None)."""
    lib = _lib_handle()
    if q.dim() != 4 or k_pool.dim() != 4 or v_pool.shape != k_pool.shape:
        raise ValueError("q must be [B,C,Hq,D]; k_pool/v_pool [P,bs,Hkv,D] of equal shape")
    if q.dtype != k_pool.dtype or v_pool.dtype != k_pool.dtype:
        raise ValueError("q, k_pool and v_pool must share a dtype")
    _expect(q_pos0, torch.int32, "q_pos0", 1)
    _segs_table(segs)
    _expect(seg_indptr, torch.int32, "seg_indptr", 1)
    B, C, Hq, D = q.shape
    P, bs, Hkv, Dk, layout = _pool_dims(k_pool, kv_layout)
    if Dk != D or seg_indptr.shape[0] != B + 1 or q_pos0.shape[0] != B:
        raise ValueError("shape mismatch between q, pools, q_pos0 and seg_indptr")
    dev = q.device
    _expect_shape(out, (B, C, Hq, D), q.dtype, "out")
    _expect_shape(lse, (B, C, Hq), torch.float32, "lse")
    _expect_shape(dev_error, (1,), torch.int32, "dev_error")
    _same_device(dev, q_pos0=q_pos0, k_pool=k_pool, v_pool=v_pool, segs=segs,
                 seg_indptr=seg_indptr, out=out, lse=lse, workspace=workspace, dev_error=dev_error)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, C, Hq), dtype=torch.float32, device=dev)
    wsb = int(lib.msa_prefill_workspace_size(B, C, Hq, Hkv, D, max_ctx_len, bs, split_blocks))
    if workspace is None and wsb > 0:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
    st = lib.msa_prefill_chunk_ex(_dev_ptr(q, "q"), C, _dev_ptr(q_pos0, "q_pos0"),
                                  _dev_ptr(k_pool, "k_pool"), _dev_ptr(v_pool, "v_pool"), P, bs,
                                  _dev_ptr(segs, "segs"), _dev_ptr(seg_indptr, "seg_indptr"),
                                  B, Hq, Hkv, D, int(max_ctx_len), _dtype_enum(q), float(scale),
                                  int(split_blocks), _dev_ptr(out, "out"), _dev_ptr(lse, "lse"),
                                  _dev_ptr(workspace, "workspace"), _nbytes(workspace), layout,
                                  _dev_ptr(dev_error, "dev_error"), _stream(stream, dev))
    _lib.check(st, "msa_prefill_chunk_ex")
    return out, lse


def msa_prefill_chunk_rows(B: int, Hq: int, Hkv: int, remaining_tokens: int, max_rows: int = 8192,
                           compute_units: int = 0) -> int:
    """Chunk length for the next prefill chunk of an adaptive chunking
    scheduler (msa_prefill_chunk_rows in include/msa.h): the smallest whole
    number of the kernel's position tiles whose workgroups cover every
    compute unit, capped at max_rows and remaining_tokens."""
    r = int(_lib_handle().msa_prefill_chunk_rows(B, Hq, Hkv, remaining_tokens, max_rows,
                                                 compute_units))
    if r < 0:
        raise MsaError(r, "msa_prefill_chunk_rows")
    return r


# ---------------------------------------------------------------------------
# a5: merge
# ---------------------------------------------------------------------------

def msa_merge_partials(o_part: torch.Tensor, m_part: torch.Tensor, l_part: torch.Tensor,
                       part_indptr: torch.Tensor, out_dtype: torch.dtype = torch.float32,
                       out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                       want_lse: bool = True, stream=None):
    """Merge partials o [N, R, H, D], m/l [N, R, H] (float32) per part_indptr [B+1].
    Returns (out [B, R, H, D] out_dtype, lse [B, R, H] float32 or None)."""
    lib = _lib_handle()
    for t, n in ((o_part, "o_part"), (m_part, "m_part"), (l_part, "l_part")):
        _expect(t, torch.float32, n)
    _expect(part_indptr, torch.int32, "part_indptr", 1)
    N, R, H, D = o_part.shape
    if tuple(m_part.shape) != (N, R, H) or tuple(l_part.shape) != (N, R, H):
        raise ValueError("m_part/l_part must be [N, R, H]")
    B = part_indptr.shape[0] - 1
    dev = o_part.device
    if out is not None:
        out_dtype = out.dtype
    _expect_shape(out, (B, R, H, D), out_dtype, "out")
    _expect_shape(lse, (B, R, H), torch.float32, "lse")
    _same_device(dev, m_part=m_part, l_part=l_part, part_indptr=part_indptr, out=out, lse=lse)
    if out is None:
        out = torch.empty((B, R, H, D), dtype=out_dtype, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, R, H), dtype=torch.float32, device=dev)
    st = lib.msa_merge_partials(_dev_ptr(o_part, "o_part"), _dev_ptr(m_part, "m_part"),
                                _dev_ptr(l_part, "l_part"), _dev_ptr(part_indptr, "part_indptr"),
                                B, R, H, D, _dtype_enum(out), _dev_ptr(out, "out"),
                                _dev_ptr(lse, "lse"), _stream(stream, dev))
    _lib.check(st, "msa_merge_partials")
    return out, lse


# ---------------------------------------------------------------------------
# gather-then-attend baseline (the detour MSA avoids; not on the MSA path)
# ---------------------------------------------------------------------------

def msa_gather_alive(k_pool: torch.Tensor, v_pool: torch.Tensor, segs: torch.Tensor,
                     seg_indptr: torch.Tensor, blocks_per_seq: int,
                     dense_k: torch.Tensor | None = None, dense_v: torch.Tensor | None = None,
                     dense_segs: torch.Tensor | None = None,
                     dense_indptr: torch.Tensor | None = None, kv_layout: str = "NHD",
                     stream=None):
    """Copy each sequence's alive blocks, in logical order, into dense pools
    of B * blocks_per_seq blocks in the layout of the source pools (whole
    blocks are copied) and write the one-segment-per-sequence plan of those
    pools.  Returns (dense_k, dense_v, dense_segs [B, 6], dense_indptr [B + 1])."""
    lib = _lib_handle()
    if k_pool.dim() != 4 or v_pool.shape != k_pool.shape or v_pool.dtype != k_pool.dtype:
        raise ValueError("k_pool/v_pool must be [P,bs,Hkv,D] of equal shape and dtype")
    _segs_table(segs)
    _expect(seg_indptr, torch.int32, "seg_indptr", 1)
    P, bs, Hkv, D, _ = _pool_dims(k_pool, kv_layout)
    B = seg_indptr.shape[0] - 1
    dev = k_pool.device
    shape = (B * int(blocks_per_seq),) + tuple(k_pool.shape[1:])
    _expect_shape(dense_k, shape, k_pool.dtype, "dense_k")
    _expect_shape(dense_v, shape, k_pool.dtype, "dense_v")
    _expect_shape(dense_segs, (B, 6), torch.int32, "dense_segs")
    _expect_shape(dense_indptr, (B + 1,), torch.int32, "dense_indptr")
    _same_device(dev, v_pool=v_pool, segs=segs, seg_indptr=seg_indptr, dense_k=dense_k,
                 dense_v=dense_v, dense_segs=dense_segs, dense_indptr=dense_indptr)
    if dense_k is None:
        dense_k = torch.empty(shape, dtype=k_pool.dtype, device=dev)
    if dense_v is None:
        dense_v = torch.empty(shape, dtype=k_pool.dtype, device=dev)
    if dense_segs is None:
        dense_segs = torch.empty((B, 6), dtype=torch.int32, device=dev)
    if dense_indptr is None:
        dense_indptr = torch.empty(B + 1, dtype=torch.int32, device=dev)
    st = lib.msa_gather_alive(_dev_ptr(k_pool, "k_pool"), _dev_ptr(v_pool, "v_pool"), P, bs,
                              _dev_ptr(segs, "segs"), _dev_ptr(seg_indptr, "seg_indptr"), B, Hkv, D,
                              _dtype_enum(k_pool), int(blocks_per_seq), _dev_ptr(dense_k, "dense_k"),
                              _dev_ptr(dense_v, "dense_v"), _dev_ptr(dense_segs, "dense_segs"),
                              _dev_ptr(dense_indptr, "dense_indptr"), _stream(stream, dev))
    _lib.check(st, "msa_gather_alive")
    return dense_k, dense_v, dense_segs, dense_indptr


# the same calls without the C prefix
plan_segments = msa_plan_segments
decode = msa_decode
prefill_chunk = msa_prefill_chunk
merge_partials = msa_merge_partials
prefill_chunk_rows = msa_prefill_chunk_rows
gather_alive = msa_gather_alive
