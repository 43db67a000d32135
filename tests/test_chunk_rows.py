"""The adaptive chunk-size chooser (msa_prefill_chunk_rows): the chunk length
an adaptive chunking scheduler asks for next.  Host only, no GPU.

Pins: the rule is checked against the prefill launch it serves -- at the
chosen length the library's own split rule needs no key split (no partials,
workspace size 0) while one position tile less would split the key stream
-- and against the worked shapes of the prefill workload (batch 4, 32 query
/ 8 KV heads: 512 rows, where the measured chunk-size curve reaches its
plateau), plus the caps, the tail rule and the argument errors."""
import os

import pytest

from kv_cache_attention_msa_amd import _lib

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libmsa.so not built")

CACHED = 8192  # a long cached context, so a short chunk would have to split its keys


def rows(B, Hq, Hkv, remaining, max_rows=1 << 20, cus=0):
    return _lib.load().msa_prefill_chunk_rows(B, Hq, Hkv, remaining, max_rows, cus)


def ws(B, C, Hq, Hkv):
    return _lib.load().msa_prefill_workspace_size(B, C, Hq, Hkv, 128, CACHED + C, 16, 0)


def test_worked_shapes():
    # the prefill workload: 8 position tiles of 64 rows x 8 KV heads x 4 sequences = 256
    assert rows(4, 32, 8, 100000) == 512
    assert rows(1, 32, 8, 100000) == 2048
    assert rows(8, 32, 8, 100000) == 256
    assert rows(64, 32, 8, 100000) == 64
    assert rows(4, 64, 8, 100000) == 256   # 8 query heads per KV head: 32-row tiles
    assert rows(4, 8, 8, 100000) == 2048   # no grouping: 256-row tiles


@pytest.mark.parametrize("B", [1, 2, 3, 4, 5, 8, 13, 32])
@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (64, 8), (16, 8), (8, 8), (32, 4), (28, 4)])
def test_chosen_length_is_the_smallest_that_needs_no_key_split(B, Hq, Hkv):
    G = Hq // Hkv
    if G not in (1, 2, 4, 8):
        assert rows(B, Hq, Hkv, 100000) == _lib.MSA_ERR_UNSUPPORTED
        return
    npos = 256 // G
    C = rows(B, Hq, Hkv, 1 << 20)
    assert C % npos == 0
    # the launch at C covers the chip: the automatic split rule keeps one split
    assert ws(B, C, Hq, Hkv) == 0
    # one position tile less no longer does
    if C > npos:
        assert ws(B, C - npos, Hq, Hkv) > 0


def test_caps_and_tail():
    assert rows(4, 32, 8, 300) == 300            # the rest of the prompt is shorter
    assert rows(4, 32, 8, 100000, max_rows=200) == 200
    assert rows(4, 32, 8, 530) == 530            # an 18-row tail rides along
    assert rows(4, 32, 8, 530, max_rows=512) == 512  # ... unless max_rows forbids it
    assert rows(4, 32, 8, 600) == 512            # an 88-row remainder is its own chunk
    assert rows(4, 32, 8, 0) == 0


def test_compute_units_argument():
    assert rows(4, 32, 8, 100000, cus=128) == 256
    assert rows(4, 32, 8, 100000, cus=304) == 640  # 304 CUs: 10 tiles x 32 items = 320 >= 304
    assert rows(4, 32, 8, 100000, cus=0) == rows(4, 32, 8, 100000, cus=256)


def test_argument_errors():
    E = _lib.MSA_ERR_INVALID_ARG
    assert rows(0, 32, 8, 10) == E
    assert rows(4, 0, 8, 10) == E
    assert rows(4, 32, 0, 10) == E
    assert rows(4, 30, 8, 10) == E               # Hq % Hkv
    assert rows(4, 32, 8, -1) == E
    assert rows(4, 32, 8, 10, max_rows=0) == E
    assert rows(4, 128, 8, 10) == _lib.MSA_ERR_UNSUPPORTED  # 16 query heads per KV head
