"""CPU oracle for packing a byte mask into the bit layout of the attention kernel, and for the
per-tile summary of a packed mask.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with the HIP path.

Pages cited (by URL and section heading):
  [custom-mask]  https://yunpan.plus/t/19526-1-1, section "AI生成的代码质量如何？", excerpt 2:
                 the mask holds one bit per (query row, key column); key j is bit j % 32 of
                 word j / 32, counted from the least significant bit; a set bit keeps the
                 score; keys at or past seq_len are never kept.  Excerpt 1: a tile whose
                 mask bits are all clear is skipped (no matrix work for it).

What is computed (plain definitions):
  pack:     words[b,h,i,w] = sum over k < 32 with 32w + k < S of [bytes[b,h,i,32w+k] != 0] << k
            (so padding bits of the last word are 0)
  summary:  any[b,h,r,t] = 1 iff some kept bit lies in rows [64r, 64r+64) x keys [64t, 64t+64)
            (both clipped to S), stored as bit t % 32 of word t / 32 of
            tiles[b,h,r, :] with ceil(ceil(S/64) / 32) words per row block.

Readings: a byte mask holds one byte per (query, key), nonzero = keep (the pages' own masks
are random bits given as words; a byte or bool mask is the form a caller usually has); the
summary's 64 x 64 block matches the 64-key tile the attention kernel walks.
"""

from __future__ import annotations

import numpy as np

TILE = 64


def packed_words(seq_len: int) -> int:
    return (seq_len + 31) // 32


def tile_words(seq_len: int) -> int:
    """Summary words per row block: one bit per 64-key tile."""
    n_kt = (seq_len + TILE - 1) // TILE
    return (n_kt + 31) // 32


def keep_of(mask_bytes) -> np.ndarray:
    """Boolean keep matrix of a byte mask (numpy or CPU torch): nonzero keeps."""
    if hasattr(mask_bytes, "detach"):
        mask_bytes = mask_bytes.detach().cpu().numpy()
    return np.asarray(mask_bytes) != 0


def pack_mask(mask_bytes) -> np.ndarray:
    """[..., S] bytes -> [..., ceil(S/32)] uint32 words, key j at bit j % 32 of word j // 32."""
    keep = keep_of(mask_bytes)
    S = keep.shape[-1]
    W = packed_words(S)
    bits = np.zeros(keep.shape[:-1] + (W * 32,), dtype=np.uint64)
    bits[..., :S] = keep
    weights = np.uint64(1) << (np.arange(W * 32, dtype=np.uint64) % np.uint64(32))
    return (bits * weights).reshape(keep.shape[:-1] + (W, 32)).sum(axis=-1).astype(np.uint32)


def tile_summary(mask_bytes) -> np.ndarray:
    """[B, H, S, S] bytes -> [B, H, ceil(S/64), tile_words(S)] uint32 summary words."""
    keep = keep_of(mask_bytes)
    B, H, S, S2 = keep.shape
    assert S == S2, "square mask expected"
    n_rb = (S + TILE - 1) // TILE
    n_kt = n_rb
    out = np.zeros((B, H, n_rb, tile_words(S)), dtype=np.uint32)
    for r in range(n_rb):
        rows = keep[:, :, r * TILE:(r + 1) * TILE, :]
        for t in range(n_kt):
            anyk = rows[:, :, :, t * TILE:(t + 1) * TILE].any(axis=(2, 3))
            out[:, :, r, t // 32] |= anyk.astype(np.uint32) << np.uint32(t % 32)
    return out
