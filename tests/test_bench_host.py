"""Host-side pieces of bench.py (no GPU): FLOP and byte counts, and the input rotation sizing
that keeps HBM-bound timings from reading their inputs out of the Infinity Cache."""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from attention_forward_fwd_amd import inputs  # noqa: E402


def test_flops_dense_and_causal():
    w = inputs.mha_prefill(4, 8192, False)
    f = bench.flops(w.batch, w.n_q_heads, w.seq_len, w.head_dim, w.mode)
    assert f == 4 * 4 * 16 * 8192 ** 2 * 128 == 2199023255552
    assert bench.flops(4, 16, 8192, 128, "causal") == f / 2


def test_algorithmic_bytes():
    # Q and O for every query head, K and V for every KV head, 2-byte elements
    assert bench.alg_bytes(inputs.mha_prefill(4, 8192, False)) == 536870912
    g = inputs.gqa_prefill(4, 8192, 4, False)
    assert bench.alg_bytes(g) == 2 * 4 * 8192 * 32 * 128 * 2 + 2 * 4 * 8192 * 4 * 128 * 2
    # the bitmask adds one 32-bit word per 32 keys of every row of every query head
    m = inputs.short_masked(1000)
    assert bench.alg_bytes(m) == 4 * 16 * 1000 * 16 * 64 * 2 + 16 * 16 * 1000 * 32 * 4 == 163840000


@pytest.mark.parametrize("S,sets", [(512, 8), (1000, 4)])
def test_rotation_exceeds_infinity_cache(S, sets):
    w = inputs.short_masked(S)
    drawn = bench.rotation_sets(w, lambda i: i)
    assert drawn == list(range(sets))
    assert len(drawn) >= 4 and len(drawn) * bench.alg_bytes(w) > 2 * bench.MALL_BYTES
