"""fa_fwd_noalloc: the no-allocation entry point (device scratch in a static array of the
library) against fa_fwd_ex with the library's pool, through the C ABI, on two calls in a row per
case, the second with a smaller input (the array keeps the first call's contents)."""

import pytest
import torch

from attention_forward_fwd_amd import fa_fwd_lse, fa_fwd_noalloc, fa_fwd_plan, inputs
from attention_forward_fwd_amd.fa import DTYPES, MODES
from gpu_util import log

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
LIMIT = 256 << 20


def _case(B, S, Hq, Hkv, D, mode, seed):
    w = inputs.Workload("noalloc", "f16" if D == 64 else "bf16", mode, B, S, Hq, Hkv, D, seed=seed)
    q, k, v = inputs.make_qkv_device(w, DEV)
    m = inputs.make_bitmask_device(w, DEV) if mode == "bitmask" else None
    return w, q, k, v, m


@pytest.mark.parametrize("first,second,splits", [
    ((1, 8192, 16, 16, 128, "none"), (1, 8192, 4, 4, 128, "none"), 1),         # packed V^T
    ((1, 8192, 16, 2, 128, "causal"), (1, 6000, 8, 2, 128, "causal"), 1),      # GQA, causal
    ((1, 8192, 4, 4, 64, "bitmask"), (1, 8000, 2, 2, 64, "bitmask"), 1),      # d64 masked, packed V^T
    ((1, 8192, 1, 1, 128, "none"), (1, 4096, 1, 1, 128, "none"), 0),           # auto split-KV
    ((1, 2000, 4, 4, 128, "bitmask"), (1, 1500, 2, 2, 128, "bitmask"), 4),     # explicit split
], ids=["packed-v", "gqa-causal", "d64-masked", "auto-split", "split4"])
def test_noalloc_equals_pool_path(first, second, splits):
    for n, shape in enumerate((first, second)):
        B, S, Hq, Hkv, D, mode = shape
        w, q, k, v, m = _case(B, S, Hq, Hkv, D, mode, seed=16000 + 10 * n + S)
        plan = fa_fwd_plan(DTYPES[q.dtype], MODES[mode], B, Hq, Hkv, S, D, False, splits)
        log(f"case noalloc call {n + 1} {w.label} splits={splits}: scratch {plan['workspace_bytes']} B")
        assert 0 < plan["workspace_bytes"] <= LIMIT
        ref, ref_lse = fa_fwd_lse(q, k, v, mode=mode, mask=m, kv_splits=splits)
        out = torch.empty_like(q)
        lse = torch.empty_like(ref_lse)
        fa_fwd_noalloc(q, k, v, out, mode=mode, mask=m, lse=lse, kv_splits=splits)
        out2 = torch.empty_like(q)
        fa_fwd_noalloc(q, k, v, out2, mode=mode, mask=m, kv_splits=splits)   # without lse
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "fa_fwd_noalloc O differs from fa_fwd_ex's"
        assert torch.equal(out2, ref)
        assert torch.equal(lse, ref_lse), "fa_fwd_noalloc LSE differs from fa_fwd_ex's"


def test_noalloc_over_limit_leaves_output_untouched():
    from attention_forward_fwd_amd import FaError
    w, q, k, v, _ = _case(1, 4096, 2, 2, 128, "none", seed=16900)
    # 16 shares of a 2-head S4096 row range fit; the rejection case is checked on the CPU with a
    # larger plan, so here only: a valid call after a rejected one still works.
    out = torch.full_like(q, 3.0)
    big = torch.empty((9, 8192, 16, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(FaError) as ei:
        fa_fwd_noalloc(big, big, big, torch.empty_like(big))
    assert ei.value.status == 8
    fa_fwd_noalloc(q, k, v, out)
    ref = fa_fwd_lse(q, k, v)[0]
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
