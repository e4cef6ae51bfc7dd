"""fa_set_kernel_events: the next call on this thread records the two events around its attention
kernel only (after the V pre-pass, before the split-KV merge), on the call's stream; the hook
serves one call, whatever its outcome, and does not change the result."""

import pytest
import torch

from attention_forward_fwd_amd import fa_fwd, fa_fwd_raw, inputs, set_kernel_events
from gpu_util import log

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _events(n):
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:  # (torch creates an event when it is first recorded)
        e.record()
    torch.cuda.synchronize()
    return evs


@pytest.mark.parametrize("S,H,splits,what", [
    (8192, 2, 1, "packed V: pre-pass outside the pair"),
    (1000, 4, 1, "attention kernel alone"),
    (4096, 1, 3, "split-KV: merge outside the pair"),
])
def test_kernel_events_bracket_the_attention_kernel(S, H, splits, what):
    w = inputs.Workload("events", "bf16", "none", 1, S, H, H, 128, seed=23000 + S)
    q, k, v = (t.to(DEV) for t in inputs.make_qkv(w))
    log(f"case kernel events S{S} H{H} splits={splits} ({what})")
    o_ref = fa_fwd(q, k, v, scale=w.scale, kv_splits=splits)
    ka, kb, a, b = _events(4)
    a.record()
    set_kernel_events(ka, kb)
    o = fa_fwd(q, k, v, scale=w.scale, kv_splits=splits)
    b.record()
    torch.cuda.synchronize()
    t_kernel, t_call = ka.elapsed_time(kb), a.elapsed_time(b)
    log(f"  kernel {t_kernel * 1e3:.1f} us, call {t_call * 1e3:.1f} us")
    assert torch.equal(o, o_ref)
    assert 0.0 < t_kernel <= t_call
    # (a re-recorded stop event would move by at least a whole later call; readings of one
    # pair can differ in the last nanosecond)
    t_end = a.elapsed_time(kb)

    # One call only: the next call, without the hook, leaves the pair as it was.
    fa_fwd(q, k, v, scale=w.scale, kv_splits=splits)
    torch.cuda.synchronize()
    assert abs(a.elapsed_time(kb) - t_end) < 1e-3

    # A call that fails validation consumes the pair and records nothing.
    set_kernel_events(ka, kb)
    assert fa_fwd_raw(1, 0, 1, H, H, S, 128, w.scale, 0, k.data_ptr(), v.data_ptr(), 0,
                      o.data_ptr(), torch.cuda.current_stream().cuda_stream) == 1
    fa_fwd(q, k, v, scale=w.scale, kv_splits=splits)
    torch.cuda.synchronize()
    assert abs(a.elapsed_time(kb) - t_end) < 1e-3


@pytest.mark.parametrize("entry", ["fa_fwd_lse", "fa_fwd_noalloc"])
def test_kernel_events_other_entry_points(entry):
    # The other entry points record the pair the same way (packed V: the pre-pass stays outside).
    from attention_forward_fwd_amd import fa_fwd_lse, fa_fwd_noalloc
    w = inputs.Workload("events", "bf16", "causal", 1, 16384, 1, 1, 128, seed=23500)
    q, k, v = (t.to(DEV) for t in inputs.make_qkv(w))
    log(f"case kernel events via {entry}")
    o_ref = fa_fwd(q, k, v, mode="causal", scale=w.scale)
    out = torch.empty_like(q)
    call = {"fa_fwd_lse": lambda: fa_fwd_lse(q, k, v, mode="causal", scale=w.scale, out=out),
            "fa_fwd_noalloc": lambda: fa_fwd_noalloc(q, k, v, out, mode="causal", scale=w.scale)}[entry]
    ka, kb, a, b = _events(4)
    a.record()
    set_kernel_events(ka, kb)
    call()
    b.record()
    torch.cuda.synchronize()
    t_kernel, t_call = ka.elapsed_time(kb), a.elapsed_time(b)
    log(f"  kernel {t_kernel * 1e3:.1f} us, call {t_call * 1e3:.1f} us")
    assert torch.equal(out, o_ref)
    assert 0.0 < t_kernel < t_call
