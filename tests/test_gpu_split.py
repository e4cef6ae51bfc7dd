"""GPU parity of split-KV (fa_fwd_ex with kv_splits): each row tile's key range cut into shares
computed by separate workgroups and merged by a second kernel.  O and the LSE are compared with
the fp64 oracle (O to the same bounds as the unsplit path, LSE to the dtype's unit roundoff +
1e-4): explicit share counts, the automatic choice on small grids, causal rows whose later
shares are empty, 256-row workgroups, masked and fully masked rows, and determinism."""

import numpy as np
import pytest
import torch

from attention_forward_fwd_amd import fa_fwd, fa_fwd_lse, inputs
from gpu_util import compare, log, oracle_rows, sample_rows, to64
import oracle
from test_gpu_lse import compare_lse

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _case(B, S, Hq, Hkv, D, dtype, mode, seed):
    w = inputs.Workload("split", dtype, mode, B, S, Hq, Hkv, D, seed=seed)
    q, k, v = inputs.make_qkv(w)
    m = inputs.make_bitmask(w) if mode == "bitmask" else None
    return w, q, k, v, m


def _run(q, k, v, mode, scale, m, splits):
    o, lse = fa_fwd_lse(q.to(DEV), k.to(DEV), v.to(DEV), mode=mode, scale=scale,
                        mask=None if m is None else m.to(DEV), kv_splits=splits)
    torch.cuda.synchronize()
    return o, lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("splits", [2, 3, 5, 16])
@pytest.mark.parametrize("mode", ["none", "causal", "bitmask"])
@pytest.mark.parametrize("D,dtype", [(128, "bf16"), (64, "f16")])
def test_split_explicit(splits, mode, D, dtype):
    w, q, k, v, m = _case(1, 1100, 4, 2, D, dtype, mode, seed=14000 + splits * 7 + D)
    if m is not None:
        m = inputs.empty_rows(m, [0, 517])
    label = f"split {splits} {mode} d{D} {dtype}"
    log(f"case {label}")
    o, lse = _run(q, k, v, mode, w.scale, m, splits)
    want_o, want_lse = oracle.attention_lse(q, k, v, mode, w.scale, m)
    compare(to64(o), want_o, q.dtype, label)
    compare_lse(lse, want_lse, q.dtype, label)


@pytest.mark.parametrize("mode", ["none", "causal"])
def test_split_auto_small_grid(mode):
    # one head, 4096 positions: 16 row tiles of 256 rows, a sixteenth of the chip's slots
    w, q, k, v, _ = _case(1, 4096, 1, 1, 128, "bf16", mode, seed=14100)
    label = f"auto split {mode} B1 H1 S4096"
    log(f"case {label}")
    o, lse = _run(q, k, v, mode, w.scale, None, 0)
    rows = sample_rows(4096, seed=14101)
    want_o, want_lse = oracle_rows(q, k, v, mode, w.scale, None, rows=rows, return_lse=True)
    compare(to64(o[:, torch.as_tensor(rows, device=o.device)]), want_o, q.dtype, label)
    compare_lse(lse[:, :, rows], want_lse.transpose(0, 2, 1), q.dtype, label)


def test_split_wide_workgroups():
    # 8800 rows per KV head: 256-row workgroups, 35 of them; automatic split
    w, q, k, v, _ = _case(1, 1100, 16, 2, 128, "bf16", "causal", seed=14200)
    log("case auto split 256-row workgroups causal")
    o, lse = _run(q, k, v, "causal", w.scale, None, 0)
    want_o, want_lse = oracle.attention_lse(q, k, v, "causal", w.scale)
    compare(to64(o), want_o, q.dtype, "wide split")
    compare_lse(lse, want_lse, q.dtype, "wide split")


def test_split_matches_unsplit_and_is_deterministic():
    w, q, k, v, m = _case(2, 700, 4, 4, 64, "f16", "bitmask", seed=14300)
    qd, kd, vd, md = q.to(DEV), k.to(DEV), v.to(DEV), m.to(DEV)
    a = fa_fwd(qd, kd, vd, mode="bitmask", mask=md, kv_splits=4)
    b = fa_fwd(qd, kd, vd, mode="bitmask", mask=md, kv_splits=4)
    c = fa_fwd(qd, kd, vd, mode="bitmask", mask=md)
    torch.cuda.synchronize()
    assert torch.equal(a, b), "split-KV must be deterministic"
    err = (a.float() - c.float()).abs().max().item()
    log(f"  split vs unsplit max_abs={err:.3e}")
    assert err <= 5e-3


def test_split_nothing_kept():
    w, q, k, v, m = _case(1, 500, 2, 2, 64, "f16", "bitmask", seed=14400)
    m = torch.zeros_like(m)
    o, lse = _run(q, k, v, "bitmask", w.scale, m, 4)
    assert (o == 0).all() and np.isneginf(lse).all()


@pytest.mark.parametrize("S,splits", [(65, 2), (65, 16), (130, 3), (200, 16)])
@pytest.mark.parametrize("mode", ["none", "causal", "bitmask"])
def test_split_short_ranges(S, splits, mode):
    # shares capped at the tile count, shares of one tile, causal shares that are empty
    w, q, k, v, m = _case(2, S, 3, 1, 64, "f16", mode, seed=14500 + S * 3 + splits)
    label = f"split {splits} short S={S} {mode}"
    log(f"case {label}")
    o, lse = _run(q, k, v, mode, w.scale, m, splits)
    want_o, want_lse = oracle.attention_lse(q, k, v, mode, w.scale, m)
    compare(to64(o), want_o, q.dtype, label)
    compare_lse(lse, want_lse, q.dtype, label)


@pytest.mark.parametrize("splits", [1, 4])
@pytest.mark.parametrize("mode", ["none", "causal", "bitmask"])
def test_growing_max_split_lse(mode, splits):
    # Key rows scaled by 1 + 20 j / S: each row's running maximum keeps rising (the sum check
    # fails and tiles are redone), so every share ends on its own (lagging) maximum and the merge
    # and the LSE must still reproduce the oracle.
    w, q, k, v, m = _case(1, 1100, 4, 2, 128, "bf16", mode, seed=14600 + splits)
    k = inputs.growing_keys(k, 20.0)
    label = f"growing max split {splits} {mode}"
    log(f"case {label}")
    o, lse = _run(q, k, v, mode, w.scale, m, splits)
    want_o, want_lse = oracle.attention_lse(q, k, v, mode, w.scale, m)
    compare(to64(o), want_o, q.dtype, label)
    compare_lse(lse, want_lse, q.dtype, label)
