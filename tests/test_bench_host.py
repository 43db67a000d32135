"""Host-side parts of bench.py: the one-GPU guard, the algorithmic work
counts (checked by brute force on small workloads) and the CPU-oracle
baseline records.  No GPU is touched."""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import make_workload  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout.strip() == ""


def _visible_brute(w, rows):
    tot = 0
    for b in range(w.B):
        for i in rows:
            qpos = int(w.q_pos0[b]) + int(i)
            for p in range(int(w.ctx_len[b])):
                if w.alive[b, p // w.block_size] and p <= qpos:
                    tot += 1
    return tot


def test_visible_pairs_matches_brute_force():
    for fam in (3, 6):
        w = make_workload(fam, seed=2, size="small", values=False)
        assert bench.visible_pairs(w) == _visible_brute(w, range(w.C))
        rows = np.arange(0, w.C, 7)
        assert bench.visible_pairs(w, rows) == _visible_brute(w, rows)


def test_alive_tokens_per_seq_matches_plan_definition():
    w = make_workload(2, seed=1, size="small", values=False)
    per = bench.alive_tokens_per_seq(w)
    for b in range(w.B):
        n = int(w.ctx_len[b])
        want = sum(1 for p in range(n) if w.alive[b, p // w.block_size])
        assert per[b] == want


def test_prefill_cpu_baseline_record():
    w = make_workload(3, seed=0, size="small")
    rec = bench.prefill_cpu_baseline(w, row_step=8, budget_s=0.5, max_reps=1)
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOP/s"
    assert rec["value"] > 0 and rec["cores"] >= 1
    json.dumps(rec)


def test_peaks_instrument_loads_and_checks_its_arguments():
    # the matrix-core rate kernel the bench reports beside the published peak:
    # built next to libmsa.so, and its argument checks return before any HIP
    # call, so they run without a GPU
    import ctypes
    import pytest
    from kv_cache_attention_msa_amd import build as _build
    if not os.path.exists(_build.PEAKS_LIB):
        pytest.skip("libmsa_peaks.so not built")
    lib = ctypes.CDLL(_build.PEAKS_LIB)
    fn = lib.msa_peaks_mfma_bf16
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    sink = ctypes.c_void_p(0x1000)  # never dereferenced: each call below is rejected first
    assert fn(0, 1, sink, None) == -1
    assert fn(1, 0, sink, None) == -1
    assert fn((1 << 20) + 1, 1, sink, None) == -1
    assert fn(1, (1 << 20) + 1, sink, None) == -1
    assert fn(1, 1, None, None) == -1
