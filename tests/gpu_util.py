"""Helpers for GPU parity tests: run the HIP path through the C ABI, compare with the oracle."""

from __future__ import annotations

import numpy as np
import torch

import oracle
from attention_forward_fwd_amd import fa_fwd

# Max-abs / mean-abs error bounds against the fp64 oracle, per input dtype.
TOL = {torch.bfloat16: (2e-2, 2e-3), torch.float16: (5e-3, 5e-4)}


def log(msg: str) -> None:
    print(msg, flush=True)


def run_gpu(q, k, v, mode, scale, mask=None, out=None):
    dev = torch.device("cuda:0")
    o = fa_fwd(q.to(dev), k.to(dev), v.to(dev), mode=mode, scale=scale,
               mask=None if mask is None else mask.to(dev), out=out)
    torch.cuda.synchronize()
    return o


def to64(t):
    return t.float().cpu().numpy().astype(np.float64)


def compare(got, want, dtype, label, zero_rows=None):
    err = np.abs(got - want)
    mx, mean = float(err.max()), float(err.mean())
    log(f"  {label}: max_abs={mx:.3e} mean_abs={mean:.3e}")
    assert np.isfinite(got).all(), f"{label}: non-finite output"
    tmax, tmean = TOL[dtype]
    assert mx <= tmax and mean <= tmean, f"{label}: max {mx:.3e} (<= {tmax}) mean {mean:.3e} (<= {tmean})"
    return mx, mean


def sample_rows(S, n_random=48, seed=0):
    """Rows at tile edges, the ends and the middle, plus seeded random rows."""
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 255, 256, S // 2, S - 65, S - 64, S - 2, S - 1]
    rng = np.random.default_rng(seed)
    rnd = rng.integers(0, S, size=n_random).tolist()
    return np.array(sorted({r for r in fixed + rnd if 0 <= r < S}))


def check_full(q, k, v, mode, scale, mask=None, label=""):
    o = run_gpu(q, k, v, mode, scale, mask)
    want = oracle.attention(q, k, v, mode, scale, mask)
    return compare(to64(o), want, q.dtype, label), o


def check_sampled(q, k, v, mode, scale, mask=None, label="", rows=None, seed=0):
    S = q.shape[1]
    o = run_gpu(q, k, v, mode, scale, mask)
    rows = sample_rows(S, seed=seed) if rows is None else rows
    want = oracle.attention_rows(q, k, v, mode, scale, mask, rows=rows)
    got = to64(o[:, torch.as_tensor(rows, device=o.device)])
    return compare(got, want, q.dtype, label + f" ({len(rows)} rows x all heads)"), o
