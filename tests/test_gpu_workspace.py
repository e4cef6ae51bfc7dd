"""Caller-owned workspace (fa_fwd_ex's workspace argument): the call then uses the caller's
buffer instead of the library's pool, and its results are bitwise those of the pool path."""

import pytest
import torch

from attention_forward_fwd_amd import fa_fwd, fa_fwd_lse, inputs, workspace_bytes
from gpu_util import log

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.mark.parametrize("B,S,Hq,Hkv,D,mode,splits", [
    (1, 8192, 16, 16, 128, "none", 1),      # packed V (256-row workgroups)
    (1, 4000, 4, 4, 64, "causal", 1),       # packed V (128-row workgroups, d64)
    (1, 8192, 2, 2, 64, "bitmask", 1),      # packed V (256-row workgroups, d64 bitmask)
    (1, 4096, 1, 1, 128, "causal", 0),      # automatic split-KV: partials
    (1, 1100, 16, 2, 128, "none", 3),       # explicit split
])
def test_caller_workspace_equals_pool(B, S, Hq, Hkv, D, mode, splits):
    dtype = "f16" if D == 64 else "bf16"
    w = inputs.Workload("workspace", dtype, mode, B, S, Hq, Hkv, D, seed=15000 + S + Hkv)
    q, k, v = (t.to(DEV) for t in inputs.make_qkv(w))
    m = inputs.make_bitmask(w).to(DEV) if mode == "bitmask" else None
    need = workspace_bytes(q, k, mode, kv_splits=splits)
    log(f"case caller workspace {w.label} splits={splits}: {need} bytes")
    assert need > 0
    ref, ref_lse = fa_fwd_lse(q, k, v, mode=mode, mask=m, kv_splits=splits)
    for fill in (0, 0xFF):   # whatever the buffer holds on entry
        ws = torch.full((need,), fill, dtype=torch.uint8, device=DEV)
        o, lse = fa_fwd_lse(q, k, v, mode=mode, mask=m, kv_splits=splits, workspace=ws)
        o2 = fa_fwd(q, k, v, mode=mode, mask=m, kv_splits=splits, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o, ref) and torch.equal(o2, ref)
        assert torch.equal(lse, ref_lse)


def test_workspace_not_needed_is_ignored():
    # A short sequence plans no workspace: any buffer (here one byte) is accepted and unused.
    w = inputs.short_masked(512)
    q, k, v = (t.to(DEV) for t in inputs.make_qkv(w))
    m = inputs.make_bitmask(w).to(DEV)
    assert workspace_bytes(q, k, "bitmask") == 0
    ref = fa_fwd(q, k, v, mode="bitmask", mask=m)
    o = fa_fwd(q, k, v, mode="bitmask", mask=m, workspace=torch.zeros(1, dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(o, ref)


def test_workspace_too_small_rejected():
    from attention_forward_fwd_amd import FaError
    w = inputs.mha_prefill(1, 8192, False)   # packed V: a workspace is needed
    q, k, v = (t.to(DEV) for t in inputs.make_qkv_device(w, DEV))
    need = workspace_bytes(q, k, "none")
    assert need > 256
    o = torch.full_like(q, 7.0)
    with pytest.raises(FaError) as ei:
        fa_fwd(q, k, v, out=o, workspace=torch.empty(need - 256, dtype=torch.uint8, device=DEV))
    assert ei.value.status == 7
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()), "a rejected call must leave o untouched"
