"""The lazy running max with an after-the-fact sum check is exact in real arithmetic (CPU, fp64).

The kernel's online softmax forms each 64-key tile's weights 2^(s c - m) with the running max m
as it stands, without the tile's row max.  A lane's partial sum of its (non-negative) weights
bounds each of them, so when every lane's sum of a wave (32 rows; each row's 64 keys split over
two lane halves, keys with (key / 4) % 2 == half) stays within a bound T the tile is accepted
with alpha = 1; otherwise the wave recomputes it with m moved to max(m, tile row max) for each
of its rows, rescaling O and the row sum by 2^(m_old - m_new).  m starts at the first tile's
row max (the kernel's start; with the -1e30 floor instead, that tile is the first redo).  The
normalised output and the
log-sum-exp do not depend on which m was used, as long as every change of m is rescaled.  This
test runs that recurrence in float64 (no rounding to bf16) for several bounds and checks it
against the oracle's plain definition: a missing rescale of O or of the row sum shows up far
above 1e-12.  The second test checks that every accepted weight stays within the bound, which is
what keeps the kernel's weights finite in fp16."""

import numpy as np
import pytest

import oracle
from attention_forward_fwd_amd import inputs

LOG2E = 1.4426950408889634


def lane_sums(p):
    """Per-row partial sums of a tile's weights [rows, 64] over the two lane halves."""
    half = (np.arange(p.shape[1]) // 4) % 2
    return np.stack([p[:, half == 0].sum(axis=1), p[:, half == 1].sum(axis=1)], axis=1)


def online_sum_checked(q, k, v, scale, keep, bound, tile=64, wave=32, first_max=True):
    """One (batch, head): q [S, D], k/v [S, D], keep [S, S] bool.  Returns O [S, D], LSE [S], the
    largest accepted weight and the number of recomputed (wave, tile) pairs.  first_max: m
    starts at the first tile's row max of kept scores (a row with none keeps the floor)."""
    S, D = q.shape
    c = abs(scale) * LOG2E
    qs = q * np.sign(scale) if scale != 0 else q
    m = np.full(S, -1e30)
    if first_max:
        s0 = np.where(keep[:, :tile], (qs @ k[:tile].T) * c, -np.inf)
        m = np.maximum(m, s0.max(axis=1))
    l = np.zeros(S)
    o = np.zeros((S, D))
    worst, redo = 0.0, 0
    for t0 in range(0, S, tile):
        s = (qs @ k[t0:t0 + tile].T) * c                      # exp2-domain scores
        s = np.where(keep[:, t0:t0 + tile], s, -np.inf)
        with np.errstate(over="ignore"):
            p = np.exp2(s - m[:, None])
        for w0 in range(0, S, wave):
            rows = slice(w0, w0 + wave)
            if not (lane_sums(p[rows]) <= bound).all():       # the wave recomputes the tile
                redo += 1
                m_new = np.maximum(m[rows], s[rows].max(axis=1))
                alpha = np.exp2(m[rows] - m_new)
                l[rows] *= alpha
                o[rows] *= alpha[:, None]
                m[rows] = m_new
                p[rows] = np.exp2(s[rows] - m_new[:, None])
        worst = max(worst, float(p.max()))
        l = l + p.sum(axis=1)
        o = o + p @ v[t0:t0 + tile]
    out = np.where(l[:, None] > 0, o / np.where(l > 0, l, 1)[:, None], 0.0)
    lse = np.where(l > 0, (m + np.log2(np.where(l > 0, l, 1))) * np.log(2), -np.inf)
    return out, lse, worst, redo


@pytest.mark.parametrize("bound", [1.0, 2.0 ** 15, 2.0 ** 60])
@pytest.mark.parametrize("mode", ["none", "causal", "bitmask"])
@pytest.mark.parametrize("grow", [False, True])
@pytest.mark.parametrize("first_max", [True, False])
def test_sum_checked_online_softmax_equals_definition(bound, mode, grow, first_max):
    w = inputs.Workload("lazy", "bf16", mode, 1, 300, 2, 1, 32, seed=31000 + int(np.log2(bound)) + 7 * grow)
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
        o, lse, worst, _ = online_sum_checked(qq, kk, vv, scale, keep, bound, first_max=first_max)
        assert worst <= bound
        np.testing.assert_allclose(o, want_o[0, :, h, :], rtol=0, atol=1e-12)
        fin = np.isfinite(want_lse[0, h])
        assert np.array_equal(np.isfinite(lse), fin)
        np.testing.assert_allclose(lse[fin], want_lse[0, h][fin], rtol=1e-12, atol=1e-12)


def test_sum_check_moves_the_max_and_bounds_the_weights():
    # growing keys with a sharp scale: the max is recomputed several times per wave past the
    # first tile, and every accepted weight stays within the kernel's bound 2^15
    w = inputs.Workload("lazy", "bf16", "none", 1, 2048, 1, 1, 64, seed=31100)
    q, k, v = inputs.make_qkv(w)
    k = inputs.growing_keys(k, 20.0)
    qq, kk, vv = (t.double().numpy()[0, :, 0, :] for t in (q, k, v))
    keep = np.ones((2048, 2048), dtype=bool)
    _, _, worst, redo_floor = online_sum_checked(qq, kk, vv, 1.5, keep, 2.0 ** 15, first_max=False)
    _, _, worst_first, redo = online_sum_checked(qq, kk, vv, 1.5, keep, 2.0 ** 15)
    n_waves = 2048 // 32
    assert worst <= 2.0 ** 15 and worst_first <= 2.0 ** 15
    assert redo_floor >= 3 * n_waves  # the first tile of every wave, and more as the keys grow
    # starting from the first tile's max saves exactly that first redo of every wave
    assert redo == redo_floor - n_waves
