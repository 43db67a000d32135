"""GPU check of the bench's matrix-core rate instrument (libmsa_peaks.so).

It is not part of the attention path; the check is that it runs, and that
what it computes is the deterministic product it claims to repeat: every
workgroup holds the same values (the operands depend only on the lane), and
doubling the iteration count doubles each accumulator sum exactly (the
operands are multiples of 1/64 of at most 1/4, so every partial sum is exact in
float32)."""
import ctypes
import os

import pytest
import torch

from kv_cache_attention_msa_amd import build as _build

pytestmark = pytest.mark.gpu


def _run(lib, wgs, iters):
    st = torch.cuda.current_stream()
    sink = torch.full((wgs * 256,), float("nan"), dtype=torch.float32, device="cuda")
    rc = lib.msa_peaks_mfma_bf16(wgs, iters, ctypes.c_void_p(sink.data_ptr()),
                                 ctypes.c_void_p(st.cuda_stream))
    assert rc == 0
    torch.cuda.synchronize()
    return sink.view(wgs, 256).cpu()


def test_mfma_rate_instrument_runs_and_repeats_one_product():
    assert os.path.exists(_build.PEAKS_LIB), "libmsa_peaks.so not built"
    lib = ctypes.CDLL(_build.PEAKS_LIB)
    lib.msa_peaks_mfma_bf16.restype = ctypes.c_int
    lib.msa_peaks_mfma_bf16.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    a = _run(lib, 300, 4)
    b = _run(lib, 300, 8)
    assert torch.isfinite(a).all() and torch.isfinite(b).all()
    assert (a != 0).any()
    assert torch.equal(a, a[0].expand_as(a))
    assert torch.equal(b, 2 * a)
