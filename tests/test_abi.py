"""The C-ABI library: it loads, exports every function include/msa.h declares,
and rejects bad arguments on the host before touching the GPU (these calls
return before any HIP runtime call, so they run without a GPU)."""
import ctypes
import os
import re

import pytest

from kv_cache_attention_msa_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libmsa.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("msa_plan_segments", "msa_decode", "msa_prefill_chunk", "msa_merge_partials"):
        assert n in names


def test_every_declared_symbol_is_exported():
    lib = _lib.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(_lib.SIGNATURES)


def test_version_and_strings():
    lib = _lib.load()
    assert lib.msa_version() == 2
    assert b"INVALID" in lib.msa_status_string(-1)


NULL = None
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def test_plan_rejects_bad_args():
    lib = _lib.load()
    ws = lib.msa_plan_workspace_size(4)
    assert ws >= 32
    # null table
    assert lib.msa_plan_segments(NULL, FAKE, FAKE, 4, 8, 16, 100, FAKE, 32, FAKE, FAKE, FAKE, ws, NULL) == _lib.MSA_ERR_INVALID_ARG
    # B = 0
    assert lib.msa_plan_segments(FAKE, FAKE, FAKE, 0, 8, 16, 100, FAKE, 32, FAKE, FAKE, FAKE, ws, NULL) == _lib.MSA_ERR_INVALID_ARG
    # null dev_error
    assert lib.msa_plan_segments(FAKE, FAKE, FAKE, 4, 8, 16, 100, FAKE, 32, FAKE, NULL, FAKE, ws, NULL) == _lib.MSA_ERR_INVALID_ARG
    # workspace too small
    assert lib.msa_plan_segments(FAKE, FAKE, FAKE, 4, 8, 16, 100, FAKE, 32, FAKE, FAKE, FAKE, ws - 1, NULL) == _lib.MSA_ERR_CAPACITY
    # max_blocks * block_size overflows int32
    assert lib.msa_plan_segments(FAKE, FAKE, FAKE, 4, 1 << 20, 1 << 12, 100, FAKE, 32, FAKE, FAKE, FAKE, ws, NULL) == _lib.MSA_ERR_INVALID_ARG


def _decode(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, P=100, bs=16, segs=FAKE, indptr=FAKE, B=2, Hq=32, Hkv=8, D=128,
             maxctx=4096, dtype=_lib.MSA_BF16, scale=0.0, split=0, out=FAKE, lse=NULL, ws=FAKE,
             wsb=1 << 30, err=NULL, stream=NULL)
    a.update(kw)
    return lib.msa_decode(a["q"], a["k"], a["v"], a["P"], a["bs"], a["segs"], a["indptr"], a["B"],
                          a["Hq"], a["Hkv"], a["D"], a["maxctx"], a["dtype"], a["scale"], a["split"],
                          a["out"], a["lse"], a["ws"], a["wsb"], a["err"], a["stream"])


def _decode_ex(lib, layout=_lib.MSA_LAYOUT_NHD, kernel=_lib.MSA_DECODE_AUTO, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, P=100, bs=16, segs=FAKE, indptr=FAKE, B=2, Hq=32, Hkv=8, D=128,
             maxctx=4096, dtype=_lib.MSA_BF16, scale=0.0, split=0, out=FAKE, lse=NULL, ws=FAKE,
             wsb=1 << 30, err=NULL, stream=NULL)
    a.update(kw)
    return lib.msa_decode_ex(a["q"], a["k"], a["v"], a["P"], a["bs"], a["segs"], a["indptr"],
                             a["B"], a["Hq"], a["Hkv"], a["D"], a["maxctx"], a["dtype"], a["scale"],
                             a["split"], a["out"], a["lse"], a["ws"], a["wsb"], layout, kernel,
                             a["err"], a["stream"])


def test_decode_rejects_bad_args():
    lib = _lib.load()
    assert _decode(lib, q=NULL) == _lib.MSA_ERR_INVALID_ARG
    assert _decode(lib, Hq=30) == _lib.MSA_ERR_INVALID_ARG          # Hq % Hkv
    assert _decode(lib, B=0) == _lib.MSA_ERR_INVALID_ARG
    assert _decode(lib, split=-1) == _lib.MSA_ERR_INVALID_ARG
    assert _decode(lib, scale=float("nan")) == _lib.MSA_ERR_INVALID_ARG
    assert _decode(lib, bs=32) == _lib.MSA_ERR_UNSUPPORTED
    assert _decode(lib, D=96) == _lib.MSA_ERR_UNSUPPORTED
    assert _decode(lib, Hq=24) == _lib.MSA_ERR_UNSUPPORTED          # G = 3
    assert _decode(lib, dtype=_lib.MSA_F32, D=96) == _lib.MSA_ERR_UNSUPPORTED
    assert _decode(lib, dtype=_lib.MSA_F32, D=256) == _lib.MSA_ERR_UNSUPPORTED
    assert _decode(lib, dtype=7) == _lib.MSA_ERR_UNSUPPORTED
    assert _decode(lib, split=100000) == _lib.MSA_ERR_INVALID_ARG
    need = lib.msa_decode_workspace_size(2, 32, 8, 128, 4096, 16, 0)
    assert need > 0
    assert _decode(lib, wsb=need - 1) == _lib.MSA_ERR_CAPACITY
    assert _decode(lib, ws=NULL) == _lib.MSA_ERR_CAPACITY


def test_layout_entry_points_reject_an_unknown_layout():
    lib = _lib.load()
    ws = 1 << 30
    # everything else valid: only the layout is wrong
    assert _decode_ex(lib, layout=2) == _lib.MSA_ERR_INVALID_ARG
    assert lib.msa_prefill_chunk_ex(FAKE, 512, FAKE, FAKE, FAKE, 100, 16, FAKE, FAKE, 4, 32, 8,
                                    128, 8704, _lib.MSA_BF16, 0.0, 0, FAKE, NULL, FAKE, ws, -1,
                                    NULL, None) == _lib.MSA_ERR_INVALID_ARG
    # argument errors are still found first with a valid layout
    assert _decode_ex(lib, layout=_lib.MSA_LAYOUT_HND, q=NULL) == _lib.MSA_ERR_INVALID_ARG


def test_decode_kernel_choice_is_validated():
    """msa_decode_ex's kernel argument: unknown values are argument errors;
    the matrix-core kernel exists only for bf16 with D 128 and 4 or 8 query
    heads per KV head; the vector kernel for every supported shape."""
    lib = _lib.load()
    assert _decode_ex(lib, kernel=4) == _lib.MSA_ERR_INVALID_ARG
    assert _decode_ex(lib, kernel=-1) == _lib.MSA_ERR_INVALID_ARG
    for hq, d, dt in ((16, 128, _lib.MSA_BF16), (8, 128, _lib.MSA_BF16), (32, 64, _lib.MSA_BF16),
                      (32, 64, _lib.MSA_F32)):
        assert _decode_ex(lib, kernel=_lib.MSA_DECODE_MATRIX, Hq=hq, D=d,
                          dtype=dt) == _lib.MSA_ERR_UNSUPPORTED, (hq, d, dt)
    # the block kernel: bf16, D 128, 8 KV heads, 4 or 8 query heads per KV
    # head, at most 512 sequences
    for kw in (dict(Hq=16, Hkv=4), dict(Hq=64, Hkv=16), dict(D=64), dict(dtype=_lib.MSA_F32, D=64),
               dict(Hq=16), dict(B=513)):
        assert _decode_ex(lib, kernel=_lib.MSA_DECODE_BLOCK, **kw) == _lib.MSA_ERR_UNSUPPORTED, kw
    # the shape checks still come first
    assert _decode_ex(lib, kernel=_lib.MSA_DECODE_VECTOR, Hq=24) == _lib.MSA_ERR_UNSUPPORTED
    assert _decode_ex(lib, kernel=_lib.MSA_DECODE_MATRIX, B=0) == _lib.MSA_ERR_INVALID_ARG
    assert _decode_ex(lib, kernel=_lib.MSA_DECODE_BLOCK, B=0) == _lib.MSA_ERR_INVALID_ARG


def _aligned(*nbytes):
    return sum(-(-n // 256) * 256 for n in nbytes)


def test_decode_workspace_arithmetic():
    lib = _lib.load()
    # one split covers the context -> no workspace at all
    assert lib.msa_decode_workspace_size(1, 8, 2, 64, 1024, 16, 64) == 0
    # explicit split, a shape the block kernel does not cover (4 KV heads):
    # B*S partials of Hq*(D+2) floats (each array 256-B aligned)
    B, Hq, D, ctx, T = 3, 16, 128, 4096, 32
    S = -(-(ctx // 16) // T)
    per_head = _aligned(4 * B * S * Hq * D, 4 * B * S * Hq, 4 * B * S * Hq)
    assert lib.msa_decode_workspace_size(B, Hq, 4, D, ctx, 16, T) == per_head
    # 8 KV heads (the block kernel may run): the larger of that and the block
    # kernel's, which holds its partials -- at most cap*B/T + 2B, cap = S*T
    # alive blocks per sequence in at most two ranges -- and B+1 offsets
    Hq = 32
    per_head = _aligned(4 * B * S * Hq * D, 4 * B * S * Hq, 4 * B * S * Hq)
    nwg = -(-(S * T * B) // T) + 2 * B
    block = _aligned(4 * nwg * Hq * D, 4 * nwg * Hq, 4 * nwg * Hq, 4 * (B + 1))
    assert lib.msa_decode_workspace_size(B, Hq, 8, D, ctx, 16, T) == max(per_head, block)
    # automatic split: the grid aims at max(256, 2B) workgroups; the partials
    # hold twice that (+ 2B: a shared prefix and the rest per sequence)
    for B in (1, 32, 300):
        nparts = 2 * max(256, 2 * B) + 2 * B
        block = _aligned(4 * nparts * Hq * D, 4 * nparts * Hq, 4 * nparts * Hq, 4 * (B + 1))
        assert lib.msa_decode_workspace_size(B, Hq, 8, D, 4096, 16, 0) >= block
        assert lib.msa_decode_workspace_size(B, Hq, 8, 64, 4096, 16, 0) < block


def test_merge_rejects_bad_args():
    lib = _lib.load()
    assert lib.msa_merge_partials(NULL, FAKE, FAKE, FAKE, 1, 1, 1, 64, _lib.MSA_F32, FAKE, NULL, NULL) == _lib.MSA_ERR_INVALID_ARG
    assert lib.msa_merge_partials(FAKE, FAKE, FAKE, FAKE, 0, 1, 1, 64, _lib.MSA_F32, FAKE, NULL, NULL) == _lib.MSA_ERR_INVALID_ARG
    assert lib.msa_merge_partials(FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 64, 9, FAKE, NULL, NULL) == _lib.MSA_ERR_UNSUPPORTED


def _splits_from_workspace(lib, B, Hq, Hkv, D, ctx):
    """Number of key splits the automatic rule picks, read back from the
    decode workspace size (B*S partials of Hq*(D+2) floats, 256-B aligned)."""
    ws = lib.msa_decode_workspace_size(B, Hq, Hkv, D, ctx, 16, 0)
    if ws == 0:
        return 1
    for S in range(2, 100000):
        want = sum(-(-n * 4 // 256) * 256 for n in (B * S * Hq * D, B * S * Hq, B * S * Hq))
        if want == ws:
            return S
    raise AssertionError(ws)


def test_decode_automatic_split_rule():
    # The per-KV-head kernels' split rule (it also sets how many alive blocks
    # a sequence may use), read back at D 64, where the workspace is theirs
    # alone; the rule does not depend on D.
    lib = _lib.load()
    # the (sequence, KV head) pairs fill the 256 CUs and contexts are short:
    # one split, no merge workspace
    assert _splits_from_workspace(lib, 32, 32, 8, 64, 4096) == 1
    # long contexts: splits of at most 128 blocks (192 when the pairs alone
    # cover the 256 CUs), never a multiple of 8
    for B, Hq, ctx in ((4, 64, 131072), (64, 32, 32768), (4, 32, 65536), (2, 16, 20000)):
        S = _splits_from_workspace(lib, B, Hq, 8, 64, ctx)
        nbm = -(-ctx // 16)
        assert S > 1 and S % 8 != 0
        assert -(-nbm // S) <= (192 if B * 8 >= 256 else 128)
    # the 64-sequence batch with contexts up to 32k: 192-block splits
    assert _splits_from_workspace(lib, 64, 32, 8, 64, 32768) == 11
    # the 4-sequence 131k batch keeps 120-block splits (128 would give 64 splits)
    assert _splits_from_workspace(lib, 4, 64, 8, 64, 131072) == 69


def test_gather_rejects_bad_args():
    lib = _lib.load()

    def g(**kw):
        a = dict(k=FAKE, v=FAKE, P=100, bs=16, segs=FAKE, indptr=FAKE, B=2, Hkv=8, D=128,
                 dtype=_lib.MSA_BF16, bps=16, dk=FAKE, dv=FAKE, dsegs=FAKE, dind=FAKE)
        a.update(kw)
        return lib.msa_gather_alive(a["k"], a["v"], a["P"], a["bs"], a["segs"], a["indptr"], a["B"],
                                    a["Hkv"], a["D"], a["dtype"], a["bps"], a["dk"], a["dv"],
                                    a["dsegs"], a["dind"], NULL)

    assert g(k=NULL) == _lib.MSA_ERR_INVALID_ARG
    assert g(dind=NULL) == _lib.MSA_ERR_INVALID_ARG
    assert g(B=0) == _lib.MSA_ERR_INVALID_ARG
    assert g(bps=0) == _lib.MSA_ERR_INVALID_ARG
    assert g(bs=32) == _lib.MSA_ERR_UNSUPPORTED
    assert g(dtype=5) == _lib.MSA_ERR_UNSUPPORTED


def _prefill(lib, **kw):
    a = dict(q=FAKE, C=512, qpos=FAKE, k=FAKE, v=FAKE, P=100, bs=16, segs=FAKE, indptr=FAKE, B=4,
             Hq=32, Hkv=8, D=128, maxctx=8704, dtype=_lib.MSA_BF16, scale=0.0, split=0, out=FAKE,
             lse=NULL, ws=FAKE, wsb=1 << 30, err=NULL, stream=NULL)
    a.update(kw)
    return lib.msa_prefill_chunk(a["q"], a["C"], a["qpos"], a["k"], a["v"], a["P"], a["bs"], a["segs"],
                                 a["indptr"], a["B"], a["Hq"], a["Hkv"], a["D"], a["maxctx"], a["dtype"],
                                 a["scale"], a["split"], a["out"], a["lse"], a["ws"], a["wsb"], a["err"],
                                 a["stream"])


def test_prefill_rejects_bad_args():
    lib = _lib.load()
    assert _prefill(lib, q=NULL) == _lib.MSA_ERR_INVALID_ARG
    assert _prefill(lib, qpos=NULL) == _lib.MSA_ERR_INVALID_ARG
    assert _prefill(lib, C=0) == _lib.MSA_ERR_INVALID_ARG
    assert _prefill(lib, Hq=30) == _lib.MSA_ERR_INVALID_ARG        # Hq % Hkv
    assert _prefill(lib, scale=float("inf")) == _lib.MSA_ERR_INVALID_ARG
    assert _prefill(lib, D=96) == _lib.MSA_ERR_UNSUPPORTED
    assert _prefill(lib, dtype=_lib.MSA_F32, D=256) == _lib.MSA_ERR_UNSUPPORTED
    assert _prefill(lib, Hq=24) == _lib.MSA_ERR_UNSUPPORTED        # G = 3
    assert _prefill(lib, Hq=128, Hkv=8) == _lib.MSA_ERR_UNSUPPORTED  # G = 16
    # a small chunk splits the key stream: the workspace must hold the partials
    need = lib.msa_prefill_workspace_size(1, 16, 32, 8, 128, 8192, 16, 0)
    assert need > 0
    assert _prefill(lib, B=1, C=16, maxctx=8192, wsb=need - 1) == _lib.MSA_ERR_CAPACITY
    assert _prefill(lib, B=1, C=16, maxctx=8192, ws=NULL) == _lib.MSA_ERR_CAPACITY
    # launch-grid limits: (sequence, split) pairs above 65535, or a split chunk
    # with more rows than the merge grid takes
    assert _prefill(lib, B=40000, C=16, maxctx=1 << 20, split=64) == _lib.MSA_ERR_UNSUPPORTED
    assert _prefill(lib, B=1, C=70000, maxctx=1 << 20, split=64) == _lib.MSA_ERR_UNSUPPORTED



def test_supported_set_is_every_dtype_and_head_dim_pair():
    """Every (dtype, head_dim) of {bf16, f32} x {64, 128} with block size 16
    and 1, 2, 4 or 8 query heads per KV head is built for decode and prefill
    (the pairs the specialised kernels do not cover run on the generic
    kernel); other dtypes, head dims, group sizes and block sizes are not."""
    lib = _lib.load()
    for prefill in (0, 1):
        for dt in (_lib.MSA_BF16, _lib.MSA_F32):
            for D in (64, 128):
                for G in (1, 2, 4, 8):
                    assert lib.msa_attention_supported(prefill, dt, D, G, 16) == 1, (prefill, dt, D, G)
                assert lib.msa_attention_supported(prefill, dt, D, 3, 16) == 0
                assert lib.msa_attention_supported(prefill, dt, D, 16, 16) == 0
                assert lib.msa_attention_supported(prefill, dt, D, 4, 32) == 0
            for D in (32, 96, 256):
                assert lib.msa_attention_supported(prefill, dt, D, 4, 16) == 0
        assert lib.msa_attention_supported(prefill, 7, 128, 4, 16) == 0

def test_header_compiles_as_c_and_cpp(tmp_path):
    import shutil
    import subprocess
    for cc, lang, std in (("gcc", "c", "-std=c99"), ("g++", "c++", "-std=c++11")):
        if shutil.which(cc) is None:
            pytest.skip(f"{cc} not available")
        src = tmp_path / f"use.{lang[0]}"
        src.write_text('#include "msa.h"\nint use(void) { return msa_version(); }\n')
        r = subprocess.run([cc, "-x", lang, std, "-Wall", "-Werror", "-pedantic", "-fsyntax-only",
                            "-I", os.path.join(ROOT, "include"), str(src)], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def test_peaks_header_matches_its_library(tmp_path):
    # the bench's instrument library: its header compiles as C and C++, and
    # the library exports exactly the function the header declares
    import shutil
    import subprocess
    from kv_cache_attention_msa_amd import build as _build
    hdr = os.path.join(ROOT, "include", "msa_peaks.h")
    src = re.sub(r"/\*.*?\*/", "", open(hdr).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(msa_[a-z_0-9]+)\s*\(", src)))
    assert names == ["msa_peaks_mfma_bf16"]
    if os.path.exists(_build.PEAKS_LIB):
        lib = ctypes.CDLL(_build.PEAKS_LIB)
        for n in names:
            assert hasattr(lib, n), n
    for cc, lang, std in (("gcc", "c", "-std=c99"), ("g++", "c++", "-std=c++11")):
        if shutil.which(cc) is None:
            pytest.skip(f"{cc} not available")
        f = tmp_path / f"use_peaks.{lang[0]}"
        f.write_text('#include "msa_peaks.h"\nint use(float* s) { return msa_peaks_mfma_bf16(1, 1, s, 0); }\n')
        r = subprocess.run([cc, "-x", lang, std, "-Wall", "-Werror", "-pedantic", "-fsyntax-only",
                            "-I", os.path.join(ROOT, "include"), str(f)], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
