"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle on seeded inputs.

Bounds (max-abs / mean-abs): bf16 2e-2 / 2e-3, fp16 5e-3 / 5e-4.  Small and short-sequence
workloads are compared on every output element; the long prefill workloads on sampled rows
(all batches and heads, rows at tile edges, the ends, the middle and seeded random rows) at
full key length, in the same launch configuration the benchmark times.
"""

import numpy as np
import pytest
import torch

from attention_forward_fwd_amd import inputs
from gpu_util import check_full, check_sampled, log, oracle_rows, run_gpu, to64, compare
import oracle

pytestmark = pytest.mark.gpu


def _qkv(B, S, Hq, Hkv, D, dtype, seed):
    w = inputs.Workload("edge", dtype, "none", B, S, Hq, Hkv, D, seed=seed)
    return inputs.make_qkv(w)


def _mask(B, Hq, S, seed):
    w = inputs.Workload("edge", "f16", "bitmask", B, S, Hq, Hq, 64, seed=seed)
    return inputs.make_bitmask(w)


# ----------------------------------------------------------------- the five workloads
def test_tiny_masked():
    w = inputs.tiny_masked()
    q, k, v = inputs.make_qkv(w)
    m = inputs.make_bitmask(w)
    log(f"case {w.label}")
    check_full(q, k, v, "bitmask", w.scale, m, w.label)
    m2 = inputs.empty_rows(m, [0, 17, w.seq_len - 1])
    _, o = check_full(q, k, v, "bitmask", w.scale, m2, w.label + " rows 0,17,S-1 empty")
    assert (to64(o)[0, [0, 17, w.seq_len - 1]] == 0).all()


@pytest.mark.parametrize("S", [512, 1000])
def test_short_masked(S):
    w = inputs.short_masked(S)
    q, k, v = inputs.make_qkv(w)
    m = inputs.make_bitmask(w)
    log(f"case {w.label}")
    check_full(q, k, v, "bitmask", w.scale, m, w.label)


def test_short_masked_empty_tiles():
    # Whole 64x64 blocks cleared: the wave ballot skips them; the result must not change.
    w = inputs.short_masked(512)
    q, k, v = inputs.make_qkv(w)
    m = inputs.empty_tiles(inputs.make_bitmask(w), 64, 0.4, seed=w.seed + 50)
    log(f"case {w.label} empty 64x64 tiles")
    check_full(q, k, v, "bitmask", w.scale, m, w.label + " empty tiles")


@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
@pytest.mark.parametrize("B,S", inputs.PREFILL_SHAPES, ids=lambda x: str(x))
def test_mha_prefill(B, S, causal):
    w = inputs.mha_prefill(B, S, causal)
    q, k, v = inputs.make_qkv(w)
    log(f"case {w.label}")
    check_sampled(q, k, v, w.mode, w.scale, None, w.label, seed=w.seed)


@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
@pytest.mark.parametrize("Hkv", [4, 8])
@pytest.mark.parametrize("B,S", inputs.PREFILL_SHAPES, ids=lambda x: str(x))
def test_gqa_prefill(B, S, Hkv, causal):
    w = inputs.gqa_prefill(B, S, Hkv, causal)
    q, k, v = inputs.make_qkv(w)
    log(f"case {w.label}")
    check_sampled(q, k, v, w.mode, w.scale, None, w.label, seed=w.seed)


# ----------------------------------------------------------------- edge cases
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mode", ["none", "causal", "bitmask"])
@pytest.mark.parametrize("S", [1, 2, 31, 33, 64, 65, 127, 129, 200, 1000])
def test_ragged_lengths(S, mode, D, dtype):
    B, Hq, Hkv = 2, 6, 2   # group of 3: rows of one tile mix positions and heads unevenly
    seed = 7000 + S * 7 + D + (1 if dtype == "f16" else 0)
    q, k, v = _qkv(B, S, Hq, Hkv, D, dtype, seed)
    m = _mask(B, Hq, S, seed) if mode == "bitmask" else None
    label = f"ragged S={S} {mode} d={D} {dtype} B={B} H={Hq}/{Hkv}"
    log(f"case {label}")
    check_full(q, k, v, mode, D ** -0.5, m, label)


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (8, 1), (32, 4), (12, 3), (5, 5)])
@pytest.mark.parametrize("mode", ["none", "causal", "bitmask"])
def test_head_groupings(Hq, Hkv, mode):
    S, D = 300, 128
    q, k, v = _qkv(1, S, Hq, Hkv, D, "bf16", 8000 + Hq * 10 + Hkv)
    m = _mask(1, Hq, S, 8100 + Hq) if mode == "bitmask" else None
    label = f"heads {Hq}/{Hkv} {mode} S={S}"
    log(f"case {label}")
    check_full(q, k, v, mode, D ** -0.5, m, label)


@pytest.mark.parametrize("B,S,Hq,Hkv", [(1, 512, 8, 1), (1, 1000, 4, 2), (1, 2048, 8, 1)])
def test_causal_few_heads_split_over_xcds(B, S, Hq, Hkv):
    # One head's causal row tiles span several XCD shares of the grid (64 x 8 = 512, 2 x 16 =
    # 32 and 128 workgroups): the tiles of a head are then dealt over those XCDs.
    q, k, v = _qkv(B, S, Hq, Hkv, 128, "bf16", seed=8100 + S)
    label = f"causal xcd split B{B} S{S} H{Hq}/{Hkv}"
    log(f"case {label}")
    if S <= 1000:
        check_full(q, k, v, "causal", 128 ** -0.5, None, label)
    else:
        check_sampled(q, k, v, "causal", 128 ** -0.5, None, label)


@pytest.mark.parametrize("S,Hq,Hkv,mode,D,dtype", [
    (400, 4, 4, "none", 128, "bf16"),       # 400 rows per KV head: 128-row tiles, V's rows
    (1500, 4, 4, "none", 128, "bf16"),      # 1500 rows: 256-row workgroups, V's rows
    (1500, 4, 4, "bitmask", 64, "f16"),     # 1500 rows: 128-row tiles, d64 bitmask
    (4500, 2, 2, "causal", 64, "f16"),      # 4500 rows: 128-row tiles, packed V
    (700, 8, 1, "none", 128, "bf16"),       # 5600 rows: 256-row workgroups, V's rows
    (600, 8, 1, "bitmask", 64, "f16"),      # 4800 rows: 256-row workgroups, V's rows
    (1100, 16, 2, "none", 128, "bf16"),     # 8800 rows: 256-row workgroups, packed V
    (2100, 16, 2, "causal", 128, "bf16"),   # 16800 rows: 256-row workgroups, causal
    (1030, 8, 1, "bitmask", 64, "f16"),     # 8240 rows: 256-row workgroups, bitmask
    (1024, 8, 1, "bitmask", 64, "f16"),     # 8192 rows: 256-row workgroups, packed V, bitmask
    (1030, 8, 1, "bitmask", 128, "bf16"),
])
def test_workgroup_shapes_ragged(S, Hq, Hkv, mode, D, dtype):
    # Ragged lengths (not a multiple of 64) on each workgroup shape the library picks from the
    # number of rows per KV head (sequence length x group size).
    q, k, v = _qkv(1, S, Hq, Hkv, D, dtype, seed=8200 + S + Hq)
    m = _mask(1, Hq, S, 8300 + S) if mode == "bitmask" else None
    label = f"shape {mode} S{S} H{Hq}/{Hkv} d{D} {dtype}"
    log(f"case {label}")
    check_full(q, k, v, mode, D ** -0.5, m, label)


@pytest.mark.parametrize("scale", [0.0, -0.125, 1.0, 2.5])
@pytest.mark.parametrize("mode", ["none", "causal", "bitmask"])
def test_scales(scale, mode):
    S, D = 257, 64
    q, k, v = _qkv(1, S, 4, 2, D, "f16", 9000)
    m = _mask(1, 4, S, 9001) if mode == "bitmask" else None
    label = f"scale={scale} {mode}"
    log(f"case {label}")
    check_full(q, k, v, mode, scale, m, label)


def test_padding_bits_ignored():
    S = 1000
    q, k, v = _qkv(2, S, 4, 4, 64, "f16", 9100)
    m = _mask(2, 4, S, 9101)
    m_flip = m.clone()
    m_flip[..., -1] = m_flip[..., -1] ^ torch.tensor(-(1 << (S % 32)), dtype=torch.int32)
    a = run_gpu(q, k, v, "bitmask", 0.125, m)
    b = run_gpu(q, k, v, "bitmask", 0.125, m_flip)
    assert torch.equal(a, b), "bits for keys >= S changed the output"


@pytest.mark.parametrize("D,dtype", [(64, "f16"), (128, "bf16")])
def test_masked_keys_with_huge_scores(D, dtype):
    # Bitmask mode forms every key's weight and clears the masked ones afterwards.  Here some keys
    # are scaled up so far that their weights overflow (to infinity in fp32, and in fp16 / bf16)
    # against the running max, and every row masks them out: they must contribute exactly
    # nothing, the kept keys must still give the oracle's result, and no NaN may appear.
    S, H = 700, 2
    q, k, v = _qkv(1, S, H, H, D, dtype, 9250 + D)
    huge = torch.arange(S) % 37 == 5                      # every 37th key, from key 5
    k = k.clone()
    k[0, huge] = (k[0, huge].float() * 400.0).to(k.dtype)  # scores of hundreds of exp2 units
    words = _mask(1, H, S, 9251 + D).numpy().view(np.uint32).copy()
    for j in np.nonzero(huge.numpy())[0]:
        words[..., j // 32] &= ~np.uint32(1 << (j % 32))  # masked for every row
    m = torch.from_numpy(words.view(np.int32))
    label = f"huge masked scores d{D} {dtype}"
    log(f"case {label}")
    _, o = check_full(q, k, v, "bitmask", D ** -0.5, m, label)
    assert bool(torch.isfinite(o).all())


def test_single_kept_key_returns_value_row():
    S, H, D = 150, 2, 128
    q, k, v = _qkv(1, S, H, H, D, "bf16", 9200)
    rng = np.random.default_rng(9201)
    picks = rng.integers(0, S, size=(H, S))
    words = np.zeros((1, H, S, (S + 31) // 32), dtype=np.uint32)
    for h in range(H):
        for i in range(S):
            j = picks[h, i]
            words[0, h, i, j // 32] = np.uint32(1) << np.uint32(j % 32)
    m = torch.from_numpy(words.view(np.int32))
    o = run_gpu(q, k, v, "bitmask", 0.3, m).cpu()
    for h in range(H):
        assert torch.equal(o[0, :, h], v[0, picks[h], h]), "one kept key must return V[j] exactly"


def test_causal_equals_lower_triangular_bitmask():
    S, H = 333, 4
    q, k, v = _qkv(1, S, H, H, 128, "bf16", 9300)
    tri = np.tril(np.ones((S, S), dtype=bool))
    W = (S + 31) // 32
    padded = np.zeros((S, W * 32), dtype=np.uint64)
    padded[:, :S] = tri
    words = (padded << (np.arange(W * 32) % 32).astype(np.uint64)).reshape(S, W, 32).sum(-1)
    m = torch.from_numpy(np.broadcast_to(words.astype(np.uint32), (1, H, S, W)).copy().view(np.int32))
    a = run_gpu(q, k, v, "causal", 0.1, None)
    b = run_gpu(q, k, v, "bitmask", 0.1, m)
    assert torch.equal(a, b), "causal must equal the lower-triangular bitmask bit for bit"


def test_deterministic():
    w = inputs.mha_prefill(8, 4096, True)
    q, k, v = inputs.make_qkv(w)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    from attention_forward_fwd_amd import fa_fwd
    a = fa_fwd(qd, kd, vd, mode="causal")
    b = fa_fwd(qd, kd, vd, mode="causal")
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("S", [33, 1000])
def test_no_out_of_bounds_writes(S):
    B, Hq, Hkv, D = 1, 3, 1, 128
    q, k, v = _qkv(B, S, Hq, Hkv, D, "bf16", 9400 + S)
    n = q.numel()
    pad = 4096
    dev = torch.device("cuda:0")
    buf = torch.full((n + 2 * pad,), 12345.0, dtype=torch.bfloat16, device=dev)
    out = buf[pad:pad + n].view(q.shape)
    run_gpu(q, k, v, "causal", D ** -0.5, None, out=out)
    assert (buf[:pad] == 12345.0).all() and (buf[pad + n:] == 12345.0).all(), "guard band written"
    want = oracle.attention(q, k, v, "causal", D ** -0.5)
    compare(to64(out), want, q.dtype, f"guarded S={S}")


# ----------------------------------------------------------------- a running max that keeps moving
# Key rows scaled by 1 + 20 j / S: scaled scores (exp2 domain) reach a spread of ~30 near the
# end, so a tile's weights against the running max keep passing the kernel's sum-check bound
# (2^15) along the sequence, and the redo with the tile's max and the rescale of O and of the
# row sum run repeatedly, on every workgroup shape.
@pytest.mark.parametrize("mode,D,dtype,B,S,Hq,Hkv,full", [
    ("none", 128, "bf16", 1, 4096, 2, 2, False),     # 256-row workgroups, V's rows
    ("causal", 128, "bf16", 1, 16384, 1, 1, False),  # 256-row causal workgroups, packed V^T
    ("none", 128, "bf16", 1, 1024, 8, 2, True),      # GQA group of 4, 256-row workgroups
    ("causal", 128, "bf16", 2, 700, 4, 4, True),     # 128-row workgroups, V's rows
    ("bitmask", 64, "f16", 2, 1000, 2, 2, True),     # 128-row workgroups, V's rows
    ("causal", 64, "f16", 1, 4500, 2, 2, False),     # 128-row workgroups, packed V^T
    ("bitmask", 128, "f16", 1, 300, 3, 1, True),     # GQA group of 3, ragged tail
    ("none", 64, "f16", 1, 333, 2, 1, True),
], ids=lambda x: str(x))
def test_growing_max(mode, D, dtype, B, S, Hq, Hkv, full):
    w = inputs.Workload("grow", dtype, mode, B, S, Hq, Hkv, D, seed=17000 + S + D)
    q, k, v = inputs.make_qkv(w)
    k = inputs.growing_keys(k, 20.0)
    m = inputs.make_bitmask(w) if mode == "bitmask" else None
    label = f"growing max {mode} d{D} {dtype} B{B} S{S} H{Hq}/{Hkv}"
    log(f"case {label}")
    if full:
        check_full(q, k, v, mode, w.scale, m, label)
    else:
        check_sampled(q, k, v, mode, w.scale, m, label, seed=w.seed)


# The running max starts at the first tile's row max.  Rows that keep no key in their first
# 64-key tile start from the -1e30 floor and take the redo on their first live tile; rows that
# keep keys only in the first tile never move it; the rest keep a random half.  With growing
# keys the max keeps moving after the first tile too.  The split-KV case starts every key range
# from its own first tile.
@pytest.mark.parametrize("D,dtype,B,S,Hq,Hkv,splits", [
    (128, "bf16", 1, 1000, 4, 2, 1),   # 256-row workgroups
    (64, "f16", 2, 700, 2, 2, 1),      # 128-row workgroups
    (128, "bf16", 1, 1500, 2, 1, 3),   # split-KV key ranges
], ids=lambda x: str(x))
def test_first_tile_without_kept_keys(D, dtype, B, S, Hq, Hkv, splits):
    from attention_forward_fwd_amd import fa_fwd
    w = inputs.Workload("first", dtype, "bitmask", B, S, Hq, Hkv, D, seed=18000 + S + D)
    q, k, v = inputs.make_qkv(w)
    k = inputs.growing_keys(k, 20.0)
    m = inputs.make_bitmask(w).clone()
    rows = torch.arange(S)
    m[:, :, rows[rows % 4 == 0], :2] = 0     # nothing kept in the first tile
    m[:, :, rows[rows % 4 == 1], 2:] = 0     # kept keys only in the first tile
    label = f"first tile without kept keys d{D} {dtype} B{B} S{S} H{Hq}/{Hkv} splits={splits}"
    log(f"case {label}")
    dev = torch.device("cuda:0")
    o = fa_fwd(q.to(dev), k.to(dev), v.to(dev), mode="bitmask", scale=w.scale, mask=m.to(dev),
               kv_splits=splits)
    want = oracle_rows(q, k, v, "bitmask", w.scale, m)
    compare(to64(o), want, q.dtype, label)


# Sharp softmax: scaled scores spread over hundreds of exp2 units, so a row's maximum jumps far
# past the running max from tile to tile (in either direction of the scale's sign; the sum
# check fails and the tile is redone) and most rows are dominated by one or two keys.
@pytest.mark.parametrize("scale", [12.0, -12.0])
@pytest.mark.parametrize("mode,D,dtype,B,S,Hq,Hkv,full", [
    ("none", 128, "bf16", 1, 4096, 2, 2, False),     # 256-row workgroups
    ("causal", 128, "bf16", 1, 1100, 4, 2, True),    # 256-row causal workgroups, V's rows
    ("bitmask", 64, "f16", 2, 700, 2, 2, True),
], ids=lambda x: str(x))
def test_sharp_softmax(scale, mode, D, dtype, B, S, Hq, Hkv, full):
    q, k, v = _qkv(B, S, Hq, Hkv, D, dtype, 9500 + S + D)
    m = _mask(B, Hq, S, 9501 + S) if mode == "bitmask" else None
    label = f"sharp softmax scale={scale} {mode} d{D} {dtype} B{B} S{S} H{Hq}/{Hkv}"
    log(f"case {label}")
    if full:
        check_full(q, k, v, mode, scale, m, label)
    else:
        check_sampled(q, k, v, mode, scale, m, label, seed=9502)


# Large and uneven GQA groups: a workgroup's rows (position-major, head-minor) then cover only a
# few positions of many heads, and the group size does not divide the 32-row wave blocks.
@pytest.mark.parametrize("Hq,Hkv,S,D,dtype", [
    (64, 1, 70, 128, "bf16"),     # G = 64: 4480 rows per KV head, 256-row workgroups (non-causal)
    (48, 2, 129, 64, "f16"),      # G = 24
    (40, 8, 513, 128, "bf16"),    # G = 5
], ids=lambda x: str(x))
@pytest.mark.parametrize("mode", ["none", "causal", "bitmask"])
def test_large_uneven_groups(Hq, Hkv, S, D, dtype, mode):
    q, k, v = _qkv(1, S, Hq, Hkv, D, dtype, 9700 + Hq + S)
    m = _mask(1, Hq, S, 9701 + S) if mode == "bitmask" else None
    label = f"groups {Hq}/{Hkv} {mode} S={S} d{D} {dtype}"
    log(f"case {label}")
    check_full(q, k, v, mode, D ** -0.5, m, label)


# ----------------------------------------------------------------- per-scenario sweep: long S
# One sequence (B = 1) at S = 16384 and 32768 for every mode, head dim and dtype, each gated on
# its own; Hq 4 over Hkv 2 gives 32768-65536 rows per KV head (256-row workgroups, packed V^T).
# Compared on sampled rows at full key length.
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mode", ["none", "causal", "bitmask"])
@pytest.mark.parametrize("S", [16384, 32768])
def test_long_single_sequence(S, mode, D, dtype):
    w = inputs.Workload("long-b1", dtype, mode, 1, S, 4, 2, D,
                        seed=19000 + S // 1024 + 7 * D + (1 if dtype == "f16" else 0)
                        + {"none": 0, "causal": 2, "bitmask": 4}[mode])
    q, k, v = inputs.make_qkv(w)
    m = inputs.make_bitmask(w) if mode == "bitmask" else None
    log(f"case {w.label}")
    check_sampled(q, k, v, mode, w.scale, m, w.label, seed=w.seed)


# fp16 at the d128 prefill shapes (the benchmark grid runs them in bf16)
@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
@pytest.mark.parametrize("B,S", inputs.PREFILL_SHAPES, ids=lambda x: str(x))
def test_mha_prefill_fp16(B, S, causal):
    w = inputs.Workload("mha-prefill-fp16", "f16", "causal" if causal else "none", B, S, 16, 16,
                        128, seed=19500 + S // 1024 + (1 if causal else 0))
    q, k, v = inputs.make_qkv(w)
    log(f"case {w.label}")
    check_sampled(q, k, v, w.mode, w.scale, None, w.label, seed=w.seed)
