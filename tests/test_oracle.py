"""CPU checks of the oracle against facts fixed outside it (see oracle_pins.py, mask_pins.py)."""

import pytest

import mask_pins
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS + mask_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin()


@pytest.mark.parametrize("S", [1, 7, 128, 1000])
def test_flop_count_against_kept_pairs(S):
    # 4*d FLOPs per (query, key) pair: the dense count is every pair of the keep matrix of mode
    # none; the causal convention (half the dense count) is within 1/S of the pairs the causal
    # keep matrix holds (S(S+1)/2); bitmask mode is counted dense.
    import numpy as np
    from oracle import attention_flops, keep_rows
    d = 64
    rows = np.arange(S)
    dense = 4 * d * int(keep_rows("none", rows, S).sum())
    causal = 4 * d * int(keep_rows("causal", rows, S).sum())
    assert attention_flops(1, 1, S, d, "none") == dense
    assert attention_flops(1, 1, S, d, "bitmask") == dense
    assert abs(attention_flops(1, 1, S, d, "causal") - causal) <= causal / S
    assert attention_flops(3, 5, S, d, "none") == 15 * dense


@pytest.mark.parametrize("mode", ["none", "causal", "bitmask"])
def test_threaded_oracle_split_matches_one_call(mode):
    # The GPU tests call the oracle per (batch, query head) slice on host threads; that split
    # must reproduce one whole-tensor call (GQA head mapping and mask slicing included).
    import numpy as np
    import oracle
    from attention_forward_fwd_amd import inputs
    from gpu_util import oracle_rows
    w = inputs.Workload("split-check", "bf16", mode, 2, 77, 6, 2, 64, seed=31)
    q, k, v = inputs.make_qkv(w)
    m = inputs.make_bitmask(w) if mode == "bitmask" else None
    rows = np.array([0, 5, 33, 76])
    want_o, want_l = oracle.attention_rows(q, k, v, mode, w.scale, m, rows=rows, return_lse=True)
    got_o, got_l = oracle_rows(q, k, v, mode, w.scale, m, rows=rows, return_lse=True)
    np.testing.assert_allclose(got_o, want_o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(got_l, want_l, rtol=0, atol=1e-13)
    np.testing.assert_allclose(oracle_rows(q, k, v, mode, w.scale, m),
                               oracle.attention(q, k, v, mode, w.scale, m), rtol=0, atol=1e-13)
