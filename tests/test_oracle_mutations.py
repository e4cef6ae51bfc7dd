"""Plant plausible mistakes in the CPU oracle and check that the pins catch every one.

Each mutation replaces one helper of oracle/masked_attention.py (on the CPU, for the duration of
one test) with a subtly wrong version; at least one pin in oracle_pins.py must then fail.
"""

import numpy as np
import pytest

import mask_pins
import oracle_pins
from oracle import mask_pack as opack
from oracle import masked_attention as oatt


def _wrong_kv_head(h, n_q_heads, n_kv_heads):
    # interleaved grouping: query head h reads KV head h mod n_kv_heads
    return h % n_kv_heads


def _msb_first_bits(words_row, seq_len):
    j = np.arange(seq_len)
    return ((words_row[..., j >> 5] >> (31 - (j & 31)).astype(np.uint32)) & np.uint32(1)).astype(bool)


def _inverted_polarity(words_row, seq_len):
    return ~_orig_bit_of(words_row, seq_len)


def _padding_kept(words_row, seq_len):
    # reads the bits past seq_len as if they were keys (then truncates wrongly)
    W = words_row.shape[-1]
    j = np.arange(W * 32)
    bits = ((words_row[..., j >> 5] >> (j & 31).astype(np.uint32)) & np.uint32(1)).astype(bool)
    return np.roll(bits, -(W * 32 - seq_len), axis=-1)[..., :seq_len]


def _strict_causal(mode, rows, seq_len, mask_rows=None):
    if mode == "causal":
        return np.arange(seq_len)[None, :] < np.asarray(rows)[:, None]
    return _orig_keep_rows(mode, rows, seq_len, mask_rows)


def _upper_causal(mode, rows, seq_len, mask_rows=None):
    if mode == "causal":
        return np.arange(seq_len)[None, :] >= np.asarray(rows)[:, None]
    return _orig_keep_rows(mode, rows, seq_len, mask_rows)


def _no_max_subtraction(scores, keep):
    any_kept = keep.any(axis=1)
    with np.errstate(over="ignore", invalid="ignore"):
        w = np.where(keep, np.exp(scores), 0.0)
        den = w.sum(axis=1)
        return np.where(any_kept[:, None], w / np.where(any_kept, den, 1.0)[:, None], 0.0)


def _masked_row_mean(scores, keep):
    # the finite-fill reading: a fully masked row averages every key
    out = _orig_masked_softmax(scores, keep)
    empty = ~keep.any(axis=1)
    out[empty] = 1.0 / scores.shape[1]
    return out


def _masked_not_excluded_from_max(scores, keep):
    m = scores.max(axis=1)
    w = np.where(keep, np.exp(scores - m[:, None]), 0.0)
    den = w.sum(axis=1)
    return np.where(den[:, None] > 0, w / np.where(den > 0, den, 1.0)[:, None], 0.0)


def _missing_normalisation(scores, keep):
    any_kept = keep.any(axis=1)
    m = np.where(keep, scores, -np.inf).max(axis=1)
    m = np.where(any_kept, m, 0.0)
    return np.where(keep, np.exp(scores - m[:, None]), 0.0)


def _lse_log2(scores, keep):
    return _orig_masked_logsumexp(scores, keep) / np.log(2.0)


def _lse_without_max(scores, keep):
    out = _orig_masked_logsumexp(scores, keep)
    m = np.where(keep, scores, -np.inf).max(axis=1)
    return np.where(np.isfinite(out), out - m, out)


def _lse_masked_in_sum(scores, keep):
    return _orig_masked_logsumexp(scores, np.ones_like(keep) & keep.any(axis=1)[:, None])


def _lse_empty_row_zero(scores, keep):
    out = _orig_masked_logsumexp(scores, keep)
    return np.where(np.isinf(out), 0.0, out)


_orig_bit_of = oatt.bit_of
_orig_keep_rows = oatt.keep_rows
_orig_masked_softmax = oatt.masked_softmax
_orig_masked_logsumexp = oatt.masked_logsumexp

MUTATIONS = {
    "gqa_head_modulo": ("kv_head_index", _wrong_kv_head),
    "mask_msb_first": ("bit_of", _msb_first_bits),
    "mask_polarity": ("bit_of", _inverted_polarity),
    "mask_padding_read": ("bit_of", _padding_kept),
    "causal_drops_diagonal": ("keep_rows", _strict_causal),
    "causal_transposed": ("keep_rows", _upper_causal),
    "softmax_no_max_shift": ("masked_softmax", _no_max_subtraction),
    "masked_row_mean": ("masked_softmax", _masked_row_mean),
    "softmax_unnormalised": ("masked_softmax", _missing_normalisation),
    "masked_scores_in_max": ("masked_softmax", _masked_not_excluded_from_max),
    "lse_log2": ("masked_logsumexp", _lse_log2),
    "lse_without_max": ("masked_logsumexp", _lse_without_max),
    "lse_masked_in_sum": ("masked_logsumexp", _lse_masked_in_sum),
    "lse_empty_row_zero": ("masked_logsumexp", _lse_empty_row_zero),
}


def _any_pin_fails():
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except AssertionError:
            failed.append(pin.__name__)
    return failed


def _keep_only_ones(mask_bytes):
    # only the byte value 1 keeps (other nonzero values dropped)
    if hasattr(mask_bytes, "detach"):
        mask_bytes = mask_bytes.detach().cpu().numpy()
    return np.asarray(mask_bytes) == 1


def _summary_32_rows(mask_bytes):
    # row blocks of 32 instead of 64 (the first half of every block only)
    keep = _orig_keep_of(mask_bytes).copy()
    S = keep.shape[-1]
    for r0 in range(32, S, 64):
        keep[:, :, r0:r0 + 32, :] = False
    return _orig_tile_summary(keep.astype(np.uint8))


def _summary_transposed(mask_bytes):
    keep = _orig_keep_of(mask_bytes)
    return _orig_tile_summary(np.swapaxes(keep, -1, -2).astype(np.uint8))


def _pack_msb_first(mask_bytes):
    w = _orig_pack_mask(mask_bytes)
    out = np.zeros_like(w)
    for k in range(32):
        out |= ((w >> np.uint32(k)) & np.uint32(1)) << np.uint32(31 - k)
    return out


_orig_keep_of = opack.keep_of
_orig_tile_summary = opack.tile_summary
_orig_pack_mask = opack.pack_mask

PACK_MUTATIONS = {
    "pack_only_byte_one": ("keep_of", _keep_only_ones),
    "pack_msb_first": ("pack_mask", _pack_msb_first),
    "summary_32_rows": ("tile_summary", _summary_32_rows),
    "summary_transposed": ("tile_summary", _summary_transposed),
}


@pytest.mark.parametrize("name", sorted(PACK_MUTATIONS))
def test_pack_mutation_is_caught(name, monkeypatch):
    import oracle
    attr, fn = PACK_MUTATIONS[name]
    monkeypatch.setattr(opack, attr, fn)
    if hasattr(oracle, attr):
        monkeypatch.setattr(oracle, attr, fn)
    failed = []
    for pin in mask_pins.ALL_PINS:
        try:
            pin()
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name!r} in oracle.mask_pack.{attr} passed every pin"


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(oatt, attr, fn)
    failed = _any_pin_fails()
    assert failed, f"planted mistake {name!r} in oracle.{attr} passed every pin"


def test_scale_dropped_is_caught(monkeypatch):
    orig = oatt.attention_rows

    def no_scale(q, k, v, mode, scale, *a, **kw):
        return orig(q, k, v, mode, 1.0, *a, **kw)
    monkeypatch.setattr(oatt, "attention_rows", no_scale)
    assert _any_pin_fails()
