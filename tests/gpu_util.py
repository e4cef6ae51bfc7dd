"""Helpers for GPU parity tests: run the HIP path through the C ABI, compare with the oracle.

The oracle is called per (batch, query head) on that head's slice of Q, K, V (and mask), over a
pool of host threads with single-threaded BLAS: numpy releases the interpreter lock in its
matrix products and array loops, so the slices run in parallel.  Each call is the unchanged
oracle on its rows; only the split over threads is added here.  Threads, not processes: no
process is started from one that holds the GPU."""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
from attention_forward_fwd_amd import fa_fwd

# Max-abs / mean-abs error bounds against the fp64 oracle, per input dtype.
TOL = {torch.bfloat16: (2e-2, 2e-3), torch.float16: (5e-3, 5e-4)}

# Host threads for the oracle (the GPU machine's CPU share is 16).
WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))


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


def _np(t):
    """CPU numpy view of a tensor: bf16/fp16 as float32 (exact), mask words as uint32."""
    if t is None or isinstance(t, np.ndarray):
        return t
    t = t.detach().cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.float().numpy()
    return t.numpy()


def oracle_rows(q, k, v, mode, scale, mask=None, rows=None, return_lse=False):
    """oracle.attention_rows for rows `rows` (all when None) of every batch and query head,
    computed per (batch, head) slice on WORKERS threads.  Returns O [B, R, Hq, D] float64 (and
    LSE [B, R, Hq] when return_lse)."""
    from threadpoolctl import threadpool_limits
    qn, kn, vn, mn = _np(q), _np(k), _np(v), _np(mask)
    B, S, Hq, D = qn.shape
    G = Hq // kn.shape[2]
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((B, len(rows), Hq, D), dtype=np.float64)
    lse = np.empty((B, len(rows), Hq), dtype=np.float64) if return_lse else None

    def one(bh):
        b, h = divmod(bh, Hq)
        g = h // G
        r = oracle.attention_rows(qn[b:b + 1, :, h:h + 1], kn[b:b + 1, :, g:g + 1],
                                  vn[b:b + 1, :, g:g + 1], mode, scale,
                                  None if mn is None else mn[b:b + 1, h:h + 1], rows=rows,
                                  return_lse=return_lse)
        if return_lse:
            out[b, :, h, :], lse[b, :, h] = r[0][0, :, 0, :], r[1][0, :, 0]
        else:
            out[b, :, h, :] = r[0, :, 0, :]

    with threadpool_limits(1), ThreadPoolExecutor(WORKERS) as ex:
        list(ex.map(one, range(B * Hq)))
    return (out, lse) if return_lse else out


def compare(got, want, dtype, label, zero_rows=None):
    err = np.abs(got - want)
    mx, mean = float(err.max()), float(err.mean())
    log(f"  {label}: max_abs={mx:.3e} mean_abs={mean:.3e}")
    assert np.isfinite(got).all(), f"{label}: non-finite output"
    tmax, tmean = TOL[dtype]
    assert mx <= tmax and mean <= tmean, f"{label}: max {mx:.3e} (<= {tmax}) mean {mean:.3e} (<= {tmean})"
    return mx, mean


def sample_rows(S, n_random=None, seed=0):
    """Rows at tile edges, the ends and the middle, plus seeded random rows (S / 16 of them, at
    least 48)."""
    if n_random is None:
        n_random = max(48, S // 16)
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 255, 256, S // 2, S - 65, S - 64, S - 2, S - 1]
    rng = np.random.default_rng(seed)
    rnd = rng.integers(0, S, size=n_random).tolist()
    return np.array(sorted({r for r in fixed + rnd if 0 <= r < S}))


def check_full(q, k, v, mode, scale, mask=None, label=""):
    o = run_gpu(q, k, v, mode, scale, mask)
    want = oracle_rows(q, k, v, mode, scale, mask)
    return compare(to64(o), want, q.dtype, label), o


def check_sampled(q, k, v, mode, scale, mask=None, label="", rows=None, seed=0):
    S = q.shape[1]
    o = run_gpu(q, k, v, mode, scale, mask)
    rows = sample_rows(S, seed=seed) if rows is None else rows
    want = oracle_rows(q, k, v, mode, scale, mask, rows=rows)
    got = to64(o[:, torch.as_tensor(rows, device=o.device)])
    return compare(got, want, q.dtype, label + f" ({len(rows)} rows x all heads)"), o
