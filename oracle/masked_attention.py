"""Plain fp64 CPU oracle for masked softmax attention (the FlashAttention forward result).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with the HIP
path and never calls it.

Pages cited (by URL and section heading):
  [custom-mask]  https://yunpan.plus/t/19526-1-1  -- a random custom-mask, short-sequence
                 FlashAttention kernel.  Section "AI生成的代码质量如何？", excerpt 2
                 (in-register scale, mask and row max) fixes the mask semantics: one bit per
                 (query row, key column), word = key / 32, bit = key % 32 counted from the
                 least significant bit, a set bit keeps the score, and keys/rows at or past
                 seq_len are never kept.
  [avo]          https://yetianai.com/news/16520  -- section "传统进化搜索的天花板" states
                 the FlashAttention idea (block-wise attention, the full score matrix is never
                 stored); section "七天跑出的成绩单" gives the prefill grid (head dim 128,
                 causal and non-causal, MHA with 16 heads; GQA with 32 query heads sharing 4
                 or 8 KV heads).

What is computed (the plain definition; tiling and the online softmax of the pages only
reorder this computation, so the oracle is the definition itself):

    for every batch b, query head h, query row i < S:
        g      = h // G                      (G = Hq / Hkv query heads share one KV head)
        s[j]   = scale * sum_d Q[b,i,h,d] * K[b,j,g,d]          for keys j < S
        keep   = none: all j;  causal: j <= i;  bitmask: bit (j % 32) of word mask[b,h,i,j//32]
        if no j is kept: O[b,i,h,:] = 0
        else:  w[j] = exp(s[j] - max_kept s) for kept j, 0 otherwise;  O = sum_j w[j] V[b,j,g,:] / sum_j w[j]
        LSE[b,h,i] = ln sum_{kept j} exp(s[j])  (= max_kept s + ln sum_j w[j]);  -inf if no j is kept

The log-sum-exp is the single-pass softmax state (running max and running sum) that the
pages' online softmax carries from tile to tile ([avo], "传统进化搜索的天花板": the correction
step rescales by that state); a forward that also returns it lets a later pass rebuild the
weights as exp(s[j] - LSE).

Readings where the pages leave a step open (each is listed with its reason in the design notes):
  * a fully masked row outputs exactly 0 (the custom-mask excerpt's finite fill value would
    instead average the masked keys; the stated problem defines the row as 0);
  * mask layout is [B, Hq, S, W] uint32 with W = ceil(S/32); bits for keys >= S are ignored;
  * consecutive query heads share a KV head: g = h // G;
  * causal keeps the diagonal (j <= i) with one common sequence length for queries and keys;
  * the scale multiplies the raw dot product before masking; any finite scale is allowed.

Layouts: q [B, S, Hq, D], k and v [B, S, Hkv, D], o [B, S, Hq, D]; any real dtype is upcast
to float64 exactly (bf16/fp16 values are exactly representable in float64).
"""

from __future__ import annotations

import numpy as np

MODES = ("none", "causal", "bitmask")

# Query rows processed per block.  Only bounds memory (rows x S fp64 scores); it does not
# change the arithmetic of any single row.
ROW_BLOCK = 256


def _f64(x) -> np.ndarray:
    """Exact upcast of a numpy array or a CPU torch tensor (bf16 included) to float64."""
    if hasattr(x, "detach"):  # torch tensor without importing torch here
        x = x.detach()
        if str(x.dtype) in ("torch.bfloat16", "torch.float16"):
            x = x.float()
        x = x.cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def _u32(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    a = np.asarray(x)
    if a.dtype == np.uint32:
        return a
    if a.dtype in (np.int32,):
        return a.view(np.uint32)
    return a.astype(np.int64).astype(np.uint32)


def mask_words(seq_len: int) -> int:
    """Words per mask row: one bit per key, 32 keys per uint32 word, rounded up."""
    return (seq_len + 31) // 32


def kv_head_index(h: int, n_q_heads: int, n_kv_heads: int) -> int:
    """KV head shared by query head h: each run of n_q_heads / n_kv_heads consecutive query
    heads forms one group."""
    return h // (n_q_heads // n_kv_heads)


def bit_of(words_row: np.ndarray, seq_len: int) -> np.ndarray:
    """Unpack mask words [..., W] (uint32) into a bool per key j < seq_len: [..., seq_len].

    Key j lives in word j // 32 at bit j % 32, least significant bit first; a set bit keeps.
    Bits for keys at or beyond seq_len are dropped."""
    j = np.arange(seq_len)
    return ((words_row[..., j >> 5] >> (j & 31).astype(np.uint32)) & np.uint32(1)).astype(bool)


def keep_rows(mode: str, rows: np.ndarray, seq_len: int, mask_rows=None) -> np.ndarray:
    """Boolean keep matrix [len(rows), seq_len] for query rows `rows`.

    mask_rows: for bitmask mode, the [len(rows), W] uint32 words of those rows."""
    if mode == "none":
        return np.ones((len(rows), seq_len), dtype=bool)
    if mode == "causal":
        return np.arange(seq_len)[None, :] <= np.asarray(rows)[:, None]
    if mode == "bitmask":
        return bit_of(np.asarray(mask_rows), seq_len)
    raise ValueError(f"unknown mode {mode!r}")


def masked_softmax(scores: np.ndarray, keep: np.ndarray) -> np.ndarray:
    """Row-wise softmax over kept entries only.  Rows with no kept entry become all zeros."""
    any_kept = keep.any(axis=1)
    m = np.where(keep, scores, -np.inf).max(axis=1)
    m = np.where(any_kept, m, 0.0)
    w = np.exp(np.where(keep, scores - m[:, None], -np.inf))
    den = w.sum(axis=1)
    return np.where(any_kept[:, None], w / np.where(any_kept, den, 1.0)[:, None], 0.0)


def masked_logsumexp(scores: np.ndarray, keep: np.ndarray) -> np.ndarray:
    """Row-wise ln(sum of exp(score)) over kept entries only; -inf for a row with none kept.

    Written as max + ln(sum exp(score - max)) so large scores do not overflow."""
    any_kept = keep.any(axis=1)
    m = np.where(keep, scores, -np.inf).max(axis=1)
    m = np.where(any_kept, m, 0.0)
    den = np.exp(np.where(keep, scores - m[:, None], -np.inf)).sum(axis=1)
    with np.errstate(divide="ignore"):
        return np.where(any_kept, m + np.log(np.where(any_kept, den, 1.0)), -np.inf)


def _check(q, k, v, mode, mask):
    if mode not in MODES:
        raise ValueError(f"unknown mode {mode!r}")
    B, S, Hq, D = q.shape
    Bk, Sk, Hkv, Dk = k.shape
    if (Bk, Sk, Dk) != (B, S, D) or v.shape != k.shape:
        raise ValueError("k/v shape does not match q")
    if Hq % Hkv:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    if mode == "bitmask":
        if mask is None or tuple(mask.shape) != (B, Hq, S, mask_words(S)):
            raise ValueError("bitmask mode needs mask of shape [B, Hq, S, ceil(S/32)]")
    return B, S, Hq, Hkv, D


def attention_rows(q, k, v, mode: str, scale: float, mask=None, rows=None, heads=None,
                   batches=None, return_weights: bool = False, return_lse: bool = False):
    """Oracle output for a selection of query rows.

    Computes O[b, i, h, :] for b in `batches`, h in `heads`, i in `rows` (all when None),
    as a float64 array [len(batches), len(rows), len(heads), D].  With return_weights=True
    also returns the attention weights [nb, nrows, nheads, S] (tiny shapes only); with
    return_lse=True also the log-sum-exp of each row's kept scores [nb, nrows, nheads].
    Returns O, then the weights, then the LSE, each only when asked for."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    mask = None if mask is None else _u32(mask)
    B, S, Hq, Hkv, D = _check(q, k, v, mode, mask)
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = np.arange(Hq) if heads is None else np.asarray(heads, dtype=np.int64)
    batches = np.arange(B) if batches is None else np.asarray(batches, dtype=np.int64)
    out = np.zeros((len(batches), len(rows), len(heads), D), dtype=np.float64)
    wts = np.zeros((len(batches), len(rows), len(heads), S)) if return_weights else None
    lse = np.zeros((len(batches), len(rows), len(heads))) if return_lse else None
    for bi, b in enumerate(batches):
        for hi, h in enumerate(heads):
            g = kv_head_index(int(h), Hq, Hkv)
            kk = k[b, :, g, :]
            vv = v[b, :, g, :]
            for r0 in range(0, len(rows), ROW_BLOCK):
                rr = rows[r0:r0 + ROW_BLOCK]
                scores = scale * (q[b, rr, h, :] @ kk.T)
                keep = keep_rows(mode, rr, S, None if mask is None else mask[b, h, rr, :])
                w = masked_softmax(scores, keep)
                out[bi, r0:r0 + len(rr), hi, :] = w @ vv
                if return_weights:
                    wts[bi, r0:r0 + len(rr), hi, :] = w
                if return_lse:
                    lse[bi, r0:r0 + len(rr), hi] = masked_logsumexp(scores, keep)
    res = (out,) + ((wts,) if return_weights else ()) + ((lse,) if return_lse else ())
    return res if len(res) > 1 else out


def attention(q, k, v, mode: str, scale: float, mask=None) -> np.ndarray:
    """Full oracle output O [B, S, Hq, D] in float64."""
    return attention_rows(q, k, v, mode, scale, mask)


def attention_lse(q, k, v, mode: str, scale: float, mask=None):
    """Full oracle output and log-sum-exp: O [B, S, Hq, D] and LSE [B, Hq, S], float64."""
    o, lse = attention_rows(q, k, v, mode, scale, mask, return_lse=True)
    return o, np.ascontiguousarray(lse.transpose(0, 2, 1))


def attention_flops(batch: int, n_q_heads: int, seq_len: int, head_dim: int, mode: str) -> float:
    """Dense FLOP count used for throughput: 4*B*Hq*S^2*d, half of it for causal.

    Bitmask mode is counted dense (no discount for masked pairs)."""
    f = 4.0 * batch * n_q_heads * seq_len * seq_len * head_dim
    return f / 2 if mode == "causal" else f
