"""GPU parity of fa_fwd_lse: the per-row log-sum-exp against the fp64 oracle, and O unchanged.

LSE bound (max-abs): the kernel sums the weights after rounding them to the input dtype (the
same sum that normalises O), so its relative error in the row sum is at most the dtype's unit
roundoff u (2^-8 bf16, 2^-11 fp16) and the error of ln(sum) at most about u; 1e-4 more covers
the fp32 scores, exp2 and log2.  Mean-abs bound u / 2 (the rounding errors of many weights
average out).  Fully masked rows must be exactly -inf.
"""

import numpy as np
import pytest
import torch

from attention_forward_fwd_amd import fa_fwd, fa_fwd_lse, inputs
from gpu_util import compare, log, oracle_rows, sample_rows, to64
import oracle

pytestmark = pytest.mark.gpu

U = {torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}


def _qkv(B, S, Hq, Hkv, D, dtype, seed):
    return inputs.make_qkv(inputs.Workload("edge", dtype, "none", B, S, Hq, Hkv, D, seed=seed))


def _mask(B, Hq, S, seed):
    return inputs.make_bitmask(inputs.Workload("edge", "f16", "bitmask", B, S, Hq, Hq, 64, seed=seed))


def _run(q, k, v, mode, scale, mask=None):
    dev = torch.device("cuda:0")
    o, lse = fa_fwd_lse(q.to(dev), k.to(dev), v.to(dev), mode=mode, scale=scale,
                        mask=None if mask is None else mask.to(dev))
    torch.cuda.synchronize()
    return o, lse.cpu().numpy().astype(np.float64)


def compare_lse(got, want, dtype, label):
    inf_want = np.isneginf(want)
    assert np.array_equal(np.isneginf(got), inf_want), f"{label}: -inf rows differ"
    assert np.isfinite(got[~inf_want]).all(), f"{label}: non-finite LSE"
    if (~inf_want).any():
        err = np.abs(got[~inf_want] - want[~inf_want])
        mx, mean = float(err.max()), float(err.mean())
        log(f"  {label} LSE: max_abs={mx:.3e} mean_abs={mean:.3e} ({int(inf_want.sum())} empty rows)")
        u = U[dtype]
        assert mx <= u + 1e-4 and mean <= u / 2, f"{label}: LSE max {mx:.3e} mean {mean:.3e} (u={u:.3e})"


def check_full_lse(q, k, v, mode, scale, mask, label):
    o, lse = _run(q, k, v, mode, scale, mask)
    want_o, want_lse = oracle.attention_lse(q, k, v, mode, scale, mask)
    compare(to64(o), want_o, q.dtype, label)
    compare_lse(lse, want_lse, q.dtype, label)
    return o, lse


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mode", ["none", "causal", "bitmask"])
@pytest.mark.parametrize("S", [1, 33, 129, 1000])
def test_lse_ragged(S, mode, D, dtype):
    B, Hq, Hkv = 2, 6, 2
    seed = 12000 + S * 7 + D + (1 if dtype == "f16" else 0)
    q, k, v = _qkv(B, S, Hq, Hkv, D, dtype, seed)
    m = _mask(B, Hq, S, seed) if mode == "bitmask" else None
    if m is not None and S > 2:
        m = inputs.empty_rows(m, [0, S // 2])   # fully masked rows -> -inf
    label = f"lse S={S} {mode} d={D} {dtype}"
    log(f"case {label}")
    check_full_lse(q, k, v, mode, D ** -0.5, m, label)


@pytest.mark.parametrize("scale", [0.0, -0.125, 2.5])
def test_lse_scales(scale):
    S, D = 257, 64
    q, k, v = _qkv(1, S, 4, 2, D, "f16", 12500)
    m = _mask(1, 4, S, 12501)
    for mode in ("none", "causal", "bitmask"):
        label = f"lse scale={scale} {mode}"
        log(f"case {label}")
        check_full_lse(q, k, v, mode, scale, m if mode == "bitmask" else None, label)


@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
@pytest.mark.parametrize("kind", ["mha", "gqa"])
def test_lse_prefill_sampled(kind, causal):
    # 256-row workgroups (the benchmark's launch configuration); packed V except causal MHA
    w = inputs.mha_prefill(4, 8192, causal) if kind == "mha" else inputs.gqa_prefill(2, 16384, 4, causal)
    q, k, v = inputs.make_qkv(w)
    log(f"case lse {w.label}")
    o, lse = _run(q, k, v, w.mode, w.scale)
    rows = sample_rows(w.seq_len, seed=w.seed)
    want_o, want_lse = oracle_rows(q, k, v, w.mode, w.scale, None, rows=rows, return_lse=True)
    compare(to64(o[:, torch.as_tensor(rows, device=o.device)]), want_o, q.dtype, w.label)
    compare_lse(lse[:, :, rows], want_lse.transpose(0, 2, 1), q.dtype, w.label)


@pytest.mark.parametrize("mode", ["none", "causal", "bitmask"])
def test_lse_leaves_o_unchanged(mode):
    S, Hq, Hkv, D = 700, 8, 2, 128
    q, k, v = _qkv(1, S, Hq, Hkv, D, "bf16", 12600)
    m = _mask(1, Hq, S, 12601) if mode == "bitmask" else None
    dev = torch.device("cuda:0")
    a = fa_fwd(q.to(dev), k.to(dev), v.to(dev), mode=mode, mask=None if m is None else m.to(dev))
    b, _ = fa_fwd_lse(q.to(dev), k.to(dev), v.to(dev), mode=mode,
                      mask=None if m is None else m.to(dev))
    torch.cuda.synchronize()
    assert torch.equal(a, b), "fa_fwd_lse must produce the same O as fa_fwd"


def test_lse_every_element_written():
    S, Hq, D = 100, 3, 64
    q, k, v = _qkv(1, S, Hq, 1, D, "f16", 12700)
    dev = torch.device("cuda:0")
    lse = torch.full((1, Hq, S), float("nan"), dtype=torch.float32, device=dev)
    m = inputs.empty_rows(_mask(1, Hq, S, 12701), [5])
    fa_fwd_lse(q.to(dev), k.to(dev), v.to(dev), mode="bitmask", mask=m.to(dev), lse=lse)
    torch.cuda.synchronize()
    x = lse.cpu()
    assert not torch.isnan(x).any(), "an LSE element was not written"
    assert torch.isneginf(x[0, :, 5]).all()


@pytest.mark.parametrize("D,dtype", [(128, "bf16"), (64, "f16")])
def test_lse_first_tile_without_kept_keys(D, dtype):
    # Rows that keep no key in their first tile (the running max starts at its floor and moves
    # at the first live tile) beside rows that keep keys only there, with growing keys; plus
    # rows with no kept key at all (-inf).
    S, Hq, Hkv = 700, 4, 2
    w = inputs.Workload("first", dtype, "bitmask", 1, S, Hq, Hkv, D, seed=18500 + D)
    q, k, v = inputs.make_qkv(w)
    k = inputs.growing_keys(k, 20.0)
    m = inputs.make_bitmask(w).clone()
    rows = torch.arange(S)
    m[:, :, rows[rows % 4 == 0], :2] = 0
    m[:, :, rows[rows % 4 == 1], 2:] = 0
    m = inputs.empty_rows(m, [3, 350])
    label = f"lse first tile without kept keys d={D} {dtype}"
    log(f"case {label}")
    check_full_lse(q, k, v, "bitmask", w.scale, m, label)
