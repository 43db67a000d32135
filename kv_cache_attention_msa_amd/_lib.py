"""ctypes loader for libmsa.so (the C ABI declared in include/msa.h).

The library must have been built in-tree (kv_cache_attention_msa_amd/libmsa.so).
There is no fallback: if it is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmsa.so")

MSA_OK = 0
MSA_ERR_INVALID_ARG = -1
MSA_ERR_UNSUPPORTED = -2
MSA_ERR_CAPACITY = -3
MSA_ERR_DEVICE = -4

MSA_F32 = 0
MSA_BF16 = 1

MSA_LAYOUT_NHD = 0  # pool blocks [P, block_size, Hkv, D]
MSA_LAYOUT_HND = 1  # pool blocks [P, Hkv, block_size, D]

MSA_DEVERR_PHYS_RANGE = 1
MSA_DEVERR_CAPACITY = 2
MSA_DEVERR_CTX_RANGE = 4
MSA_DEVERR_TRUNCATED = 8

MSA_DECODE_AUTO = 0    # decode kernel chosen per shape and split count
MSA_DECODE_VECTOR = 1  # vector-ALU decode kernel
MSA_DECODE_MATRIX = 2  # matrix-core decode kernel (bf16, D 128, Hq/Hkv 4 or 8)
MSA_DECODE_BLOCK = 3   # matrix-core decode kernel streaming whole KV blocks (bf16, D 128, Hkv 8, Hq/Hkv 4 or 8, B <= 1024)

# every symbol include/msa.h declares, with (restype, argtypes)
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t
_p = ctypes.c_void_p
_f = ctypes.c_float

SIGNATURES = {
    "msa_version": (ctypes.c_int, []),
    "msa_attention_supported": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _i32, _i32, _i32]),
    "msa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "msa_plan_workspace_size": (_sz, [_i32]),
    "msa_plan_segments": (ctypes.c_int, [_p, _p, _p, _i32, _i32, _i32, _i32, _p, _i32, _p, _p, _p, _sz, _p]),
    "msa_decode_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "msa_decode": (ctypes.c_int, [_p, _p, _p, _i32, _i32, _p, _p, _i32, _i32, _i32, _i32, _i32,
                                  ctypes.c_int, _f, _i32, _p, _p, _p, _sz, _p, _p]),
    "msa_decode_ex": (ctypes.c_int, [_p, _p, _p, _i32, _i32, _p, _p, _i32, _i32, _i32, _i32, _i32,
                                     ctypes.c_int, _f, _i32, _p, _p, _p, _sz, ctypes.c_int,
                                     ctypes.c_int, _p, _p]),
    "msa_decode_noalloc_capacity": (_sz, []),
    "msa_decode_noalloc": (ctypes.c_int, [_p, _p, _p, _i32, _i32, _p, _p, _i32, _i32, _i32, _i32,
                                          _i32, ctypes.c_int, _f, _i32, _p, _p, _p, _p]),
    "msa_prefill_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "msa_prefill_chunk": (ctypes.c_int, [_p, _i32, _p, _p, _p, _i32, _i32, _p, _p, _i32, _i32, _i32,
                                         _i32, _i32, ctypes.c_int, _f, _i32, _p, _p, _p, _sz, _p,
                                         _p]),
    "msa_prefill_chunk_ex": (ctypes.c_int, [_p, _i32, _p, _p, _p, _i32, _i32, _p, _p, _i32, _i32,
                                            _i32, _i32, _i32, ctypes.c_int, _f, _i32, _p, _p, _p,
                                            _sz, ctypes.c_int, _p, _p]),
    "msa_prefill_chunk_rows": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "msa_merge_partials": (ctypes.c_int, [_p, _p, _p, _p, _i32, _i32, _i32, _i32, ctypes.c_int, _p, _p, _p]),
    "msa_gather_alive": (ctypes.c_int, [_p, _p, _i32, _i32, _p, _p, _i32, _i32, _i32, ctypes.c_int, _i32,
                                        _p, _p, _p, _p, _p]),
}

_LIB = None


class MsaError(RuntimeError):
    """A libmsa call returned a non-zero msa_status."""

    def __init__(self, status: int, where: str):
        self.status = status
        msg = load().msa_status_string(status).decode() if _LIB is not None else str(status)
        super().__init__(f"{where}: {msg} ({status})")


def load():
    """Load libmsa.so once and declare its signatures; raises if it is absent."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first "
            "(python -c 'import __graft_entry__ as g; g.build()' or "
            "python kv_cache_attention_msa_amd/build.py)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def check(status: int, where: str):
    if status != MSA_OK:
        raise MsaError(status, where)
