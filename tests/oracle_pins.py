"""Pins for the CPU oracle: checks against facts fixed outside the oracle itself.

Each `pin_*` function raises AssertionError when the oracle disagrees with:
  * a hand-derived example (tests/golden/hand_example.json),
  * a 50-digit brute force on tiny inputs,
  * closed forms (one kept key -> that value row; zero scale -> mean of kept values;
    causal row 0 -> V[0]),
  * invariants of softmax attention (weights sum to 1, constant V, key permutation,
    all-ones mask == no mask, causal == lower-triangular mask, padding bits ignored,
    fully masked row == 0, GQA == MHA with K/V repeated per head group, shift of all
    scores by a constant leaves O unchanged even when exp would overflow),
  * a library routine (torch scaled_dot_product_attention in float64 on the CPU, on rows
    with at least one kept key);
and, for the log-sum-exp of each row, the hand example's values, the brute force, the zero
scale (log of the kept-key count), one kept key (its scaled dot product), a shift of all
scores, torch.logsumexp in float64, and exp(score - LSE) == the oracle's weights.

They are plain functions so that tests/test_oracle_mutations.py can plant mistakes in the
oracle and check that at least one pin fails for each.
"""

from __future__ import annotations

import json
import os

import numpy as np
import torch

import oracle
from oracle import masked_attention as oatt

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_example.json")


def _rng(seed):
    return np.random.default_rng(seed)


def _rand_case(seed, B=1, S=7, Hq=2, Hkv=1, D=4, mode="bitmask", density=0.5):
    r = _rng(seed)
    q = r.standard_normal((B, S, Hq, D))
    k = r.standard_normal((B, S, Hkv, D))
    v = r.standard_normal((B, S, Hkv, D))
    W = oracle.mask_words(S)
    bits = r.random((B, Hq, S, W * 32)) < density
    words = (bits.astype(np.uint64) << np.arange(32 * W, dtype=np.uint64) % 32)
    words = words.reshape(B, Hq, S, W, 32).sum(-1).astype(np.uint32)
    return q, k, v, (words if mode == "bitmask" else None)


def _pack_bool(keep):
    """[.., S] bool -> [.., ceil(S/32)] uint32, bit j%32 of word j//32 (test-side packing)."""
    S = keep.shape[-1]
    W = (S + 31) // 32
    padded = np.zeros(keep.shape[:-1] + (W * 32,), dtype=np.uint64)
    padded[..., :S] = keep
    shifts = (np.arange(W * 32) % 32).astype(np.uint64)
    return (padded << shifts).reshape(keep.shape[:-1] + (W, 32)).sum(-1).astype(np.uint32)


# --------------------------------------------------------------------------- hand example
def pin_hand_example():
    g = json.load(open(GOLDEN))
    q = np.array([[g["q_row"]] * 3])[:, :, None, :]      # [1, 3, 1, 2]
    k = np.array([g["k"]])[:, :, None, :]
    v = np.array([g["v"]])[:, :, None, :]
    for mode in ("none", "causal", "bitmask"):
        for words in ([g["mask_words"], g["mask_words_padded"]] if mode == "bitmask" else [None]):
            mask = None if words is None else np.array(words, dtype=np.uint32).reshape(1, 1, 3, 1)
            o = oracle.attention(q, k, v, mode, g["scale"], mask)[0, :, 0, :]
            np.testing.assert_allclose(o, np.array(g["expected"][mode]), rtol=1e-13, atol=1e-13,
                                       err_msg=f"hand example, mode {mode}")


# --------------------------------------------------------------------------- brute force
def _brute_compare(seed, B, S, Hq, Hkv, D, mode, scale, density=0.5):
    q, k, v, mask = _rand_case(seed, B, S, Hq, Hkv, D, mode, density)
    want = oracle.attention_brute(q.tolist(), k.tolist(), v.tolist(), mode, scale,
                                  None if mask is None else mask.tolist())
    want = np.array([[[[float(x) for x in row] for row in hh] for hh in ii] for ii in want])
    got = oracle.attention(q, k, v, mode, scale, mask)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13,
                               err_msg=f"brute force {mode} S={S} Hq={Hq} Hkv={Hkv}")


def pin_brute_force_small():
    for i, mode in enumerate(("none", "causal", "bitmask")):
        _brute_compare(10 + i, 1, 6, 4, 2, 3, mode, 0.7)          # GQA, group 2
        _brute_compare(20 + i, 2, 5, 2, 2, 4, mode, -1.3)         # MHA, negative scale


def pin_brute_force_two_words():
    # S = 37 spans two mask words, so the word index (key // 32) is exercised.
    _brute_compare(31, 1, 37, 2, 1, 2, "bitmask", 0.9, density=0.3)
    _brute_compare(32, 1, 37, 1, 1, 2, "causal", 0.9)


def pin_brute_force_large_scores():
    # Scores of several hundred: exp overflows float64 unless the row max is subtracted.
    _brute_compare(41, 1, 6, 2, 2, 3, "none", 400.0)
    _brute_compare(42, 1, 6, 2, 2, 3, "bitmask", 400.0, density=0.4)


# --------------------------------------------------------------------------- closed forms
def pin_single_kept_key():
    q, k, v, _ = _rand_case(51, B=1, S=40, Hq=3, Hkv=1, D=5, mode="none")
    S = 40
    rng = _rng(52)
    keep = np.zeros((1, 3, S, S), dtype=bool)
    picks = rng.integers(0, S, size=(3, S))
    for h in range(3):
        keep[0, h, np.arange(S), picks[h]] = True
    o = oracle.attention(q, k, v, "bitmask", 0.8, _pack_bool(keep))
    for h in range(3):
        np.testing.assert_array_equal(o[0, :, h, :], v[0, picks[h], 0, :],
                                      err_msg="one kept key must return that value row")


def pin_zero_scale_is_mean():
    q, k, v, mask = _rand_case(61, B=1, S=35, Hq=2, Hkv=2, D=3, mode="bitmask", density=0.3)
    o = oracle.attention(q, k, v, "bitmask", 0.0, mask)
    for h in range(2):
        for i in range(35):
            kept = [j for j in range(35) if (int(mask[0, h, i, j // 32]) >> (j % 32)) & 1]
            want = v[0, kept, h, :].mean(axis=0) if kept else np.zeros(3)
            np.testing.assert_allclose(o[0, i, h], want, rtol=1e-12, atol=1e-14)


def pin_causal_first_row():
    q, k, v, _ = _rand_case(71, B=2, S=9, Hq=4, Hkv=2, D=3, mode="none")
    o = oracle.attention(q, k, v, "causal", 0.5)
    for h in range(4):
        np.testing.assert_array_equal(o[:, 0, h, :], v[:, 0, h // 2, :])


# --------------------------------------------------------------------------- invariants
def pin_weights_sum_to_one():
    q, k, v, mask = _rand_case(81, B=1, S=33, Hq=2, Hkv=1, D=4, mode="bitmask")
    for mode in ("none", "causal", "bitmask"):
        _, w = oatt.attention_rows(q, k, v, mode, 0.6, mask, return_weights=True)
        s = w.sum(axis=-1)
        kept_any = s > 0
        np.testing.assert_allclose(s[kept_any], 1.0, rtol=0, atol=1e-12)
        assert (w >= 0).all()


def pin_constant_v():
    q, k, _, mask = _rand_case(91, B=1, S=20, Hq=2, Hkv=2, D=4, mode="bitmask")
    v = np.full(k.shape, 3.25)
    for mode in ("none", "causal", "bitmask"):
        o = oracle.attention(q, k, v, mode, 1.1, mask)
        if mode == "bitmask":
            rows_kept = np.array([[[any((int(mask[0, h, i, 0]) >> j) & 1 for j in range(20))]
                                   for h in range(2)] for i in range(20)])[None, :, :, 0]
        else:
            rows_kept = np.ones((1, 20, 2), dtype=bool)
        np.testing.assert_allclose(o[rows_kept], 3.25, rtol=1e-14)
        assert (o[~rows_kept] == 0).all()


def pin_all_ones_mask_equals_none():
    q, k, v, _ = _rand_case(101, B=2, S=45, Hq=2, Hkv=1, D=4, mode="none")
    ones = np.full((2, 2, 45, 2), 0xFFFFFFFF, dtype=np.uint32)
    np.testing.assert_allclose(oracle.attention(q, k, v, "bitmask", 0.4, ones),
                               oracle.attention(q, k, v, "none", 0.4), rtol=1e-14, atol=1e-15)


def pin_causal_equals_lower_triangular_mask():
    q, k, v, _ = _rand_case(111, B=1, S=40, Hq=2, Hkv=2, D=3, mode="none")
    tri = np.tril(np.ones((40, 40), dtype=bool))
    mask = _pack_bool(np.broadcast_to(tri, (1, 2, 40, 40)))
    np.testing.assert_allclose(oracle.attention(q, k, v, "causal", 0.9),
                               oracle.attention(q, k, v, "bitmask", 0.9, mask),
                               rtol=1e-14, atol=1e-15)


def pin_padding_bits_ignored():
    for S in (33, 40):
        q, k, v, mask = _rand_case(120 + S, B=1, S=S, Hq=2, Hkv=1, D=3, mode="bitmask")
        flipped = mask.copy()
        lastw = flipped[..., -1]
        pad = np.uint32(0xFFFFFFFF) << np.uint32(S % 32)
        flipped[..., -1] = lastw ^ pad
        np.testing.assert_array_equal(oracle.attention(q, k, v, "bitmask", 0.5, mask),
                                      oracle.attention(q, k, v, "bitmask", 0.5, flipped))


def pin_fully_masked_rows_zero():
    q, k, v, mask = _rand_case(131, B=1, S=30, Hq=2, Hkv=1, D=4, mode="bitmask")
    base = oracle.attention(q, k, v, "bitmask", 0.5, mask)
    m2 = mask.copy()
    m2[:, :, [0, 17, 29], :] = 0
    o = oracle.attention(q, k, v, "bitmask", 0.5, m2)
    assert (o[:, [0, 17, 29]] == 0).all()
    others = [i for i in range(30) if i not in (0, 17, 29)]
    np.testing.assert_array_equal(o[:, others], base[:, others])


def pin_key_permutation():
    S = 36
    q, k, v, mask = _rand_case(141, B=1, S=S, Hq=2, Hkv=1, D=4, mode="bitmask")
    perm = _rng(142).permutation(S)
    keep = np.zeros((1, 2, S, S), dtype=bool)
    for h in range(2):
        for i in range(S):
            keep[0, h, i] = [(int(mask[0, h, i, j // 32]) >> (j % 32)) & 1 for j in range(S)]
    m_perm = _pack_bool(keep[..., perm])
    for mode, m0, m1 in (("none", None, None), ("bitmask", mask, m_perm)):
        a = oracle.attention(q, k, v, mode, 0.7, m0)
        b = oracle.attention(q, k[:, perm], v[:, perm], mode, 0.7, m1)
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


def pin_query_permutation():
    S = 20
    q, k, v, mask = _rand_case(151, B=1, S=S, Hq=2, Hkv=2, D=4, mode="bitmask")
    perm = _rng(152).permutation(S)
    a = oracle.attention(q, k, v, "bitmask", 0.7, mask)
    b = oracle.attention(q[:, perm], k, v, "bitmask", 0.7, mask[:, :, perm])
    np.testing.assert_allclose(a[:, perm], b, rtol=1e-13, atol=1e-15)


def pin_gqa_equals_repeated_mha():
    for G, Hkv in ((4, 2), (8, 1), (2, 3)):
        Hq = G * Hkv
        q, k, v, mask = _rand_case(160 + G, B=2, S=17, Hq=Hq, Hkv=Hkv, D=3, mode="bitmask")
        krep = np.repeat(k, G, axis=2)
        vrep = np.repeat(v, G, axis=2)
        for mode in ("none", "causal", "bitmask"):
            np.testing.assert_allclose(oracle.attention(q, k, v, mode, 0.8, mask),
                                       oracle.attention(q, krep, vrep, mode, 0.8, mask),
                                       rtol=1e-14, atol=1e-15)


def pin_score_shift_invariance():
    # Append a coordinate with q = c, k = 1 to every row: all scores of a row move by scale*c,
    # which softmax must ignore, even when that shift is large enough to overflow exp.
    q, k, v, mask = _rand_case(171, B=1, S=12, Hq=2, Hkv=1, D=3, mode="bitmask")
    base = oracle.attention(q, k, v, "bitmask", 0.5, mask)
    for c in (5.0, 3000.0):
        q2 = np.concatenate([q, np.full(q.shape[:-1] + (1,), c)], axis=-1)
        k2 = np.concatenate([k, np.ones(k.shape[:-1] + (1,))], axis=-1)
        v2 = np.concatenate([v, np.zeros(v.shape[:-1] + (1,))], axis=-1)
        o2 = oracle.attention(q2, k2, v2, "bitmask", 0.5, mask)
        np.testing.assert_allclose(o2[..., :-1], base, rtol=1e-9, atol=1e-12)
        assert (o2[..., -1] == 0).all()


# --------------------------------------------------------------------------- library routine
def pin_torch_sdpa_float64():
    import torch.nn.functional as F
    q, k, v, mask = _rand_case(181, B=2, S=50, Hq=4, Hkv=2, D=8, mode="bitmask", density=0.4)
    G = 2
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(np.repeat(k, G, axis=2)).permute(0, 2, 1, 3)
    tv = torch.from_numpy(np.repeat(v, G, axis=2)).permute(0, 2, 1, 3)
    scale = 0.35
    ref_none = F.scaled_dot_product_attention(tq, tk, tv, scale=scale).permute(0, 2, 1, 3)
    ref_causal = F.scaled_dot_product_attention(tq, tk, tv, scale=scale,
                                                is_causal=True).permute(0, 2, 1, 3)
    np.testing.assert_allclose(oracle.attention(q, k, v, "none", scale), ref_none.numpy(),
                               rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(oracle.attention(q, k, v, "causal", scale), ref_causal.numpy(),
                               rtol=1e-11, atol=1e-12)
    keep = np.zeros((2, 4, 50, 50), dtype=bool)
    for b in range(2):
        for h in range(4):
            for i in range(50):
                keep[b, h, i] = [(int(mask[b, h, i, j // 32]) >> (j % 32)) & 1 for j in range(50)]
    ref_mask = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(keep),
                                              scale=scale).permute(0, 2, 1, 3).numpy()
    got = oracle.attention(q, k, v, "bitmask", scale, mask)
    rows = keep.any(-1).transpose(0, 2, 1)     # [B, S, H]
    np.testing.assert_allclose(got[rows], ref_mask[rows], rtol=1e-11, atol=1e-12)


# --------------------------------------------------------------------------- log-sum-exp
def _lse_value(text):
    """'ln N' -> ln N, '-inf' -> -inf (the hand example states its values in these forms)."""
    return -np.inf if text == "-inf" else float(np.log(float(text.split()[1])))


def pin_lse_hand_example():
    g = json.load(open(GOLDEN))
    q = np.array([[g["q_row"]] * 3])[:, :, None, :]
    k = np.array([g["k"]])[:, :, None, :]
    v = np.array([g["v"]])[:, :, None, :]
    for mode in ("none", "causal", "bitmask"):
        mask = (np.array(g["mask_words"], dtype=np.uint32).reshape(1, 1, 3, 1)
                if mode == "bitmask" else None)
        _, lse = oracle.attention_lse(q, k, v, mode, g["scale"], mask)
        want = np.array([_lse_value(t) for t in g["expected_lse"][mode]])
        np.testing.assert_allclose(lse[0, 0], want, rtol=0, atol=1e-14,
                                   err_msg=f"hand example LSE, mode {mode}")


def _brute_lse_compare(seed, B, S, Hq, Hkv, D, mode, scale, density=0.5, empty_rows=()):
    q, k, v, mask = _rand_case(seed, B, S, Hq, Hkv, D, mode, density)
    if mask is not None and empty_rows:
        mask[:, :, list(empty_rows), :] = 0
    _, want = oracle.attention_brute(q.tolist(), k.tolist(), v.tolist(), mode, scale,
                                     None if mask is None else mask.tolist(), with_lse=True)
    want = np.array([[[float(x) for x in row] for row in hh] for hh in want])
    _, got = oracle.attention_lse(q, k, v, mode, scale, mask)
    np.testing.assert_array_equal(np.isinf(got), np.isinf(want))
    fin = np.isfinite(want)
    np.testing.assert_allclose(got[fin], want[fin], rtol=1e-13, atol=1e-13,
                               err_msg=f"brute force LSE {mode} S={S}")


def pin_lse_brute_force():
    for i, mode in enumerate(("none", "causal", "bitmask")):
        _brute_lse_compare(210 + i, 1, 6, 4, 2, 3, mode, 0.7)       # GQA, group 2
        _brute_lse_compare(220 + i, 2, 5, 2, 2, 4, mode, -1.3)      # negative scale
        _brute_lse_compare(230 + i, 1, 6, 2, 2, 3, mode, 400.0)     # exp overflows without the max
    _brute_lse_compare(241, 1, 37, 2, 1, 2, "bitmask", 0.9, density=0.3, empty_rows=(0, 36))


def pin_lse_zero_scale_counts_kept_keys():
    # Every score is 0, so the sum of exp over kept keys is their count.
    q, k, v, mask = _rand_case(251, B=1, S=40, Hq=2, Hkv=1, D=3, mode="bitmask", density=0.3)
    mask[0, 1, 5, :] = 0
    for mode in ("none", "causal", "bitmask"):
        _, lse = oracle.attention_lse(q, k, v, mode, 0.0, mask)
        for h in range(2):
            for i in range(40):
                if mode == "none":
                    n = 40
                elif mode == "causal":
                    n = i + 1
                else:
                    n = sum((int(mask[0, h, i, j // 32]) >> (j % 32)) & 1 for j in range(40))
                want = np.log(n) if n else -np.inf
                assert lse[0, h, i] == want or abs(lse[0, h, i] - want) < 1e-14, (mode, h, i)


def pin_lse_single_kept_key():
    # One kept key: the log-sum-exp is that key's scaled dot product, summed by hand here.
    S, D = 30, 5
    q, k, v, _ = _rand_case(261, B=1, S=S, Hq=2, Hkv=1, D=D, mode="none")
    picks = _rng(262).integers(0, S, size=(2, S))
    keep = np.zeros((1, 2, S, S), dtype=bool)
    for h in range(2):
        keep[0, h, np.arange(S), picks[h]] = True
    _, lse = oracle.attention_lse(q, k, v, "bitmask", -0.45, _pack_bool(keep))
    for h in range(2):
        for i in range(S):
            dot = 0.0
            for t in range(D):
                dot += float(q[0, i, h, t]) * float(k[0, picks[h, i], 0, t])
            assert abs(lse[0, h, i] - (-0.45) * dot) < 1e-12, (h, i)


def pin_lse_shift_of_scores():
    # A coordinate with q = c, k = 1 moves every score of a row by scale*c: the log-sum-exp
    # moves by exactly that, even when exp of the raw scores would overflow.
    q, k, v, mask = _rand_case(271, B=1, S=12, Hq=2, Hkv=1, D=3, mode="bitmask")
    _, base = oracle.attention_lse(q, k, v, "bitmask", 0.5, mask)
    for c in (5.0, 3000.0):
        q2 = np.concatenate([q, np.full(q.shape[:-1] + (1,), c)], axis=-1)
        k2 = np.concatenate([k, np.ones(k.shape[:-1] + (1,))], axis=-1)
        v2 = np.concatenate([v, np.zeros(v.shape[:-1] + (1,))], axis=-1)
        _, lse2 = oracle.attention_lse(q2, k2, v2, "bitmask", 0.5, mask)
        fin = np.isfinite(base)
        np.testing.assert_allclose(lse2[fin], base[fin] + 0.5 * c, rtol=1e-12, atol=1e-9)
        assert np.array_equal(np.isinf(lse2), np.isinf(base))


def pin_lse_torch_logsumexp():
    # Library routine: torch.logsumexp in float64 over the scores with masked entries at -inf.
    q, k, v, mask = _rand_case(281, B=2, S=45, Hq=4, Hkv=2, D=6, mode="bitmask", density=0.4)
    mask[1, 2, 7, :] = 0
    scale = 0.8
    for mode in ("none", "causal", "bitmask"):
        _, lse = oracle.attention_lse(q, k, v, mode, scale, mask)
        tq = torch.from_numpy(q).permute(0, 2, 1, 3)                       # [B, Hq, S, D]
        tk = torch.from_numpy(np.repeat(k, 2, axis=2)).permute(0, 2, 1, 3)
        sc = scale * (tq @ tk.transpose(-1, -2))
        i = torch.arange(45)
        if mode == "causal":
            sc = sc.masked_fill(i[None, :] > i[:, None], float("-inf"))
        elif mode == "bitmask":
            keep = np.zeros((2, 4, 45, 45), dtype=bool)
            for b in range(2):
                for h in range(4):
                    for r in range(45):
                        keep[b, h, r] = [(int(mask[b, h, r, j // 32]) >> (j % 32)) & 1
                                         for j in range(45)]
            sc = sc.masked_fill(~torch.from_numpy(keep), float("-inf"))
        ref = torch.logsumexp(sc, dim=-1).numpy()
        np.testing.assert_array_equal(np.isinf(lse), np.isinf(ref))
        fin = np.isfinite(ref)
        np.testing.assert_allclose(lse[fin], ref[fin], rtol=1e-12, atol=1e-12)


def pin_lse_rebuilds_the_weights():
    # exp(score - LSE) must be the attention weights the oracle uses for O.
    q, k, v, mask = _rand_case(291, B=1, S=33, Hq=2, Hkv=1, D=4, mode="bitmask")
    for mode in ("none", "causal", "bitmask"):
        _, w, lse = oatt.attention_rows(q, k, v, mode, 0.6, mask, return_weights=True,
                                        return_lse=True)
        s = 0.6 * np.einsum("bihd,bjd->bihj", q, k[:, :, 0, :])
        with np.errstate(invalid="ignore"):
            rebuilt = np.where(w > 0, np.exp(s - lse[..., None]), 0.0)
        np.testing.assert_allclose(rebuilt, w, rtol=1e-12, atol=1e-15)


ALL_PINS = [f for n, f in sorted(globals().items()) if n.startswith("pin_") and callable(f)]
