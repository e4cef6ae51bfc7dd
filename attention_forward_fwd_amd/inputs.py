"""Seeded synthetic inputs for the attention forward workloads.

This module holds no attention arithmetic: it only draws random tensors (and zeroes whole
mask words or rows for the structured variants).  The HIP path and the CPU oracle both take
their inputs from here, on the CPU, so both see bit-identical values.

Workloads follow the prefill grid of https://yetianai.com/news/16520 (section
"七天跑出的成绩单": head dim 128, bf16, 32768 tokens split over batch x sequence length
for S in {4096, 8192, 16384, 32768}, MHA with 16 heads, causal and non-causal, GQA with
32 query heads over 4 or 8 KV heads) and the short random-mask case of
https://yunpan.plus/t/19526-1-1 (section introduction: random per-(query, key) masks,
context below 1k).  The pages give no value distribution; Q, K, V ~ N(0, 1) stands in.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "bf16" | "f16"
    mode: str             # "none" | "causal" | "bitmask"
    batch: int
    seq_len: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    seed: int
    keep_prob: float = 0.5  # bitmask only; 0.5 draws every bit independently and uniformly
    extra: dict = field(default_factory=dict, compare=False)

    @property
    def scale(self) -> float:
        return self.head_dim ** -0.5

    @property
    def label(self) -> str:
        return (f"{self.name}:{self.mode}:{self.dtype}:B{self.batch}xS{self.seq_len}:"
                f"H{self.n_q_heads}/{self.n_kv_heads}:d{self.head_dim}")


TORCH_DTYPE = {"bf16": torch.bfloat16, "f16": torch.float16}


def mask_words(seq_len: int) -> int:
    return (seq_len + 31) // 32


def make_qkv(w: Workload):
    """Q [B,S,Hq,D], K and V [B,S,Hkv,D] on the CPU, drawn as fp32 N(0,1) then rounded."""
    g = torch.Generator(device="cpu").manual_seed(w.seed)
    dt = TORCH_DTYPE[w.dtype]
    q = torch.randn((w.batch, w.seq_len, w.n_q_heads, w.head_dim), generator=g).to(dt)
    k = torch.randn((w.batch, w.seq_len, w.n_kv_heads, w.head_dim), generator=g).to(dt)
    v = torch.randn((w.batch, w.seq_len, w.n_kv_heads, w.head_dim), generator=g).to(dt)
    return q, k, v


def make_qkv_device(w: Workload, device):
    """Q, K, V of the same shapes and N(0,1) distribution drawn directly on `device` (seeded
    device generator).  For timing runs at sizes where drawing on the CPU would be slow; the
    values differ from make_qkv's."""
    g = torch.Generator(device=device).manual_seed(w.seed)
    dt = TORCH_DTYPE[w.dtype]
    shape_q = (w.batch, w.seq_len, w.n_q_heads, w.head_dim)
    shape_kv = (w.batch, w.seq_len, w.n_kv_heads, w.head_dim)
    return tuple(torch.randn(sh, generator=g, device=device, dtype=torch.float32).to(dt)
                 for sh in (shape_q, shape_kv, shape_kv))


def make_bitmask(w: Workload, seed_offset: int = 7):
    """Random packed mask [B, Hq, S, ceil(S/32)] as int32 words (uint32 bit patterns).

    With keep_prob 0.5 every bit, padding bits past S included, is an independent fair coin:
    a uniformly random 32-bit word.  Other keep probabilities draw one Bernoulli byte per bit
    position and assemble words without any attention-specific arithmetic."""
    g = torch.Generator(device="cpu").manual_seed(w.seed * 1009 + seed_offset)
    shape = (w.batch, w.n_q_heads, w.seq_len, mask_words(w.seq_len))
    if w.keep_prob == 0.5:
        words = torch.randint(0, 2 ** 32, shape, generator=g, dtype=torch.int64)
    else:
        bits = (torch.rand(shape + (32,), generator=g) < w.keep_prob).to(torch.int64)
        words = (bits * (2 ** torch.arange(32, dtype=torch.int64))).sum(-1)
    return words.to(torch.uint32).view(torch.int32)


def empty_rows(mask: torch.Tensor, rows) -> torch.Tensor:
    """Copy of `mask` with the given query rows fully masked (all words zero) in every head."""
    m = mask.clone()
    m[:, :, list(rows), :] = 0
    return m


def empty_tiles(mask: torch.Tensor, tile: int, prob: float, seed: int) -> torch.Tensor:
    """Copy of `mask` in which random whole (tile x tile) query/key blocks are cleared.

    tile must be a multiple of 32 so a block covers whole words."""
    assert tile % 32 == 0
    B, H, S, W = mask.shape
    g = torch.Generator(device="cpu").manual_seed(seed)
    nb = (S + tile - 1) // tile
    wpt = tile // 32
    clear = torch.rand((B, H, nb, nb), generator=g) < prob
    m = mask.clone()
    for b, h, qi, kj in clear.nonzero().tolist():
        m[b, h, qi * tile:(qi + 1) * tile, kj * wpt:(kj + 1) * wpt] = 0
    return m


def document_mask(mask: torch.Tensor, n_docs: int, seed: int) -> torch.Tensor:
    """Copy of `mask` restricted to a block diagonal of n_docs documents per batch (a packed
    batch of sequences: a query sees only keys of its own document).  Document boundaries are
    drawn at random (seeded); every document holds at least one position."""
    B, H, S, W = mask.shape
    assert 1 <= n_docs <= S
    g = torch.Generator(device="cpu").manual_seed(seed)
    m = mask.clone()
    key0 = torch.arange(W, dtype=torch.int64) * 32
    for b in range(B):
        cuts = sorted((torch.randperm(S - 1, generator=g)[:n_docs - 1] + 1).tolist())
        bounds = [0] + cuts + [S]
        for s0, s1 in zip(bounds[:-1], bounds[1:]):
            lo = (s0 - key0).clamp(0, 32)
            hi = (s1 - key0).clamp(0, 32)
            keep = (torch.ones_like(hi) << hi) - (torch.ones_like(lo) << lo)   # bits [lo, hi)
            m[b, :, s0:s1, :] &= keep.to(torch.uint32).view(torch.int32)
    return m


def band_mask(mask: torch.Tensor, half_width: int) -> torch.Tensor:
    """Copy of `mask` (any device) keeping only keys j with |j - i| <= half_width for query row
    i (a sliding window); the random bits inside the band are kept as drawn."""
    B, H, S, W = mask.shape
    i = torch.arange(S, device=mask.device, dtype=torch.int64)[:, None]
    key0 = torch.arange(W, device=mask.device, dtype=torch.int64)[None, :] * 32
    lo = (i - half_width - key0).clamp(0, 32)          # first kept bit of each word
    hi = (i + half_width + 1 - key0).clamp(0, 32)      # one past the last kept bit
    hi = torch.maximum(hi, lo)
    keep = (torch.ones_like(hi) << hi) - (torch.ones_like(lo) << lo)
    return mask & keep.to(torch.uint32).view(torch.int32)


def growing_keys(k: torch.Tensor, gain: float) -> torch.Tensor:
    """Copy of K [B,S,H,D] with key row j multiplied by 1 + gain * j / S (then rounded back to
    K's dtype): the scores' spread, and so each query's running maximum over the keys seen so
    far, keeps growing along the sequence instead of settling after the first few keys."""
    S = k.shape[1]
    f = 1.0 + gain * torch.arange(S, dtype=torch.float32) / S
    return (k.float() * f[None, :, None, None]).to(k.dtype)


def make_bitmask_device(w: Workload, device):
    """Random packed mask words like make_bitmask (keep probability 0.5, every bit a fair coin),
    drawn directly on `device` for sizes where the CPU would be slow; values differ from
    make_bitmask's."""
    g = torch.Generator(device=device).manual_seed(w.seed * 1009 + 7)
    shape = (w.batch, w.n_q_heads, w.seq_len, mask_words(w.seq_len))
    return torch.randint(-2 ** 31, 2 ** 31, shape, generator=g, device=device, dtype=torch.int64).to(torch.int32)


# The benchmark grid.  Seed = 1000 * config + variant.
def tiny_masked() -> Workload:
    return Workload("tiny-masked", "f16", "bitmask", 1, 128, 1, 1, 64, seed=1000)


def short_masked(seq_len: int = 512) -> Workload:
    return Workload("short-masked", "f16", "bitmask", 16, seq_len, 16, 16, 64,
                    seed=2000 + (0 if seq_len == 512 else 1))


def document_masked(seq_len: int = 1000, n_docs: int = 4) -> Workload:
    """The short random-mask shape with the mask confined to n_docs packed documents per
    sequence (random bits inside each document's diagonal block)."""
    return Workload("document-masked", "f16", "bitmask", 16, seq_len, 16, 16, 64,
                    seed=2100 + n_docs, extra={"n_docs": n_docs})


PREFILL_SHAPES = ((8, 4096), (4, 8192), (2, 16384), (1, 32768))


def mha_prefill(batch: int, seq_len: int, causal: bool) -> Workload:
    cfg = 4 if causal else 3
    variant = [s for _, s in PREFILL_SHAPES].index(seq_len)
    return Workload("mha-prefill", "bf16", "causal" if causal else "none", batch, seq_len,
                    16, 16, 128, seed=1000 * cfg + variant)


def gqa_prefill(batch: int, seq_len: int, n_kv_heads: int, causal: bool) -> Workload:
    variant = [s for _, s in PREFILL_SHAPES].index(seq_len) + (0 if n_kv_heads == 4 else 4) \
        + (8 if causal else 0)
    return Workload("gqa-prefill", "bf16", "causal" if causal else "none", batch, seq_len,
                    32, n_kv_heads, 128, seed=5000 + variant)
