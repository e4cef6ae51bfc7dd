"""The lazy running max is exact in real arithmetic (CPU, fp64).

The kernel's online softmax moves a row's running max only when a 64-key tile's max exceeds it
by more than a slack (8 in the exp2 domain), so the weights it accumulates are 2^(s c - m) with
a lagging m.  The normalised output and the log-sum-exp do not depend on which m was used, as
long as every tile's contribution is rescaled by 2^(m_old - m_new) when m moves.  This test runs
that recurrence tile by tile in float64 (no rounding to bf16) for several slacks and checks it
against the oracle's plain definition: a missing rescale of O or of the row sum shows up far
above 1e-12.  (Which value the max moves to does not matter for exactness; the second test
checks that the weights stay below 2^slack, which is what keeps them representable.)"""

import numpy as np
import pytest

import oracle
from attention_forward_fwd_amd import inputs

LOG2E = 1.4426950408889634


def online_lazy(q, k, v, scale, keep, slack, tile=64):
    """One (batch, head): q [S, D], k/v [S, D], keep [S, S] bool.  Returns O [S, D], LSE [S]."""
    S, D = q.shape
    c = abs(scale) * LOG2E
    qs = q * np.sign(scale) if scale != 0 else q
    m = np.full(S, -1e30)
    l = np.zeros(S)
    o = np.zeros((S, D))
    for t0 in range(0, S, tile):
        s = (qs @ k[t0:t0 + tile].T) * c                      # exp2-domain scores
        s = np.where(keep[:, t0:t0 + tile], s, -np.inf)
        mt = s.max(axis=1)
        m_new = np.where(mt > m + slack, mt, m)
        alpha = np.exp2(m - m_new)
        p = np.exp2(s - m_new[:, None])
        l = l * alpha + p.sum(axis=1)
        o = o * alpha[:, None] + p @ v[t0:t0 + tile]
        m = m_new
    out = np.where(l[:, None] > 0, o / np.where(l > 0, l, 1)[:, None], 0.0)
    lse = np.where(l > 0, (m + np.log2(np.where(l > 0, l, 1))) * np.log(2), -np.inf)
    return out, lse


@pytest.mark.parametrize("slack", [0.0, 8.0, 30.0])
@pytest.mark.parametrize("mode", ["none", "causal", "bitmask"])
@pytest.mark.parametrize("grow", [False, True])
def test_lazy_online_softmax_equals_definition(slack, mode, grow):
    w = inputs.Workload("lazy", "bf16", mode, 1, 300, 2, 1, 32, seed=31000 + int(slack) + 7 * grow)
    q, k, v = inputs.make_qkv(w)
    if grow:
        k = inputs.growing_keys(k, 20.0)
    mask = inputs.empty_rows(inputs.make_bitmask(w), [5, 299]) if mode == "bitmask" else None
    scale = 0.7
    want_o, want_lse = oracle.attention_lse(q, k, v, mode, scale, mask)
    S = w.seq_len
    rows = np.arange(S)
    for h in range(w.n_q_heads):
        words = None if mask is None else mask[0, h].numpy().view(np.uint32)
        keep = oracle.keep_rows(mode, rows, S, words)
        qq, kk, vv = (t.double().numpy()[0, :, hh, :] for t, hh in ((q, h), (k, 0), (v, 0)))
        o, lse = online_lazy(qq, kk, vv, scale, keep, slack)
        np.testing.assert_allclose(o, want_o[0, :, h, :], rtol=0, atol=1e-12)
        fin = np.isfinite(want_lse[0, h])
        assert np.array_equal(np.isfinite(lse), fin)
        np.testing.assert_allclose(lse[fin], want_lse[0, h][fin], rtol=1e-12, atol=1e-12)


def test_lazy_max_moves_and_bounds_the_weights():
    # growing keys: the lazy max moves several times, and every weight stays below 2^slack
    w = inputs.Workload("lazy", "bf16", "none", 1, 2048, 1, 1, 64, seed=31100)
    q, k, v = inputs.make_qkv(w)
    k = inputs.growing_keys(k, 20.0)
    c = w.scale * LOG2E
    s = (q.double().numpy()[0, :, 0] @ k.double().numpy()[0, :, 0].T) * c
    moves, worst = [], 0.0
    for row in s[::97]:
        m, n = -1e30, 0
        for t0 in range(0, len(row), 64):
            mt = row[t0:t0 + 64].max()
            if mt > m + 8.0:
                m, n = mt, n + 1
            worst = max(worst, float((row[t0:t0 + 64] - m).max()))
        moves.append(n)
    assert min(moves) >= 3 and worst <= 8.0
