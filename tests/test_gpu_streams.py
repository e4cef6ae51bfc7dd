"""The library enqueues on the caller's stream (torch's current stream through the binding):
calls on non-default streams, including the packed-V and split-KV workspaces taken
stream-ordered from the library's pool, give the same results as on the default stream, and
calls on two streams running at once do not disturb each other."""

import pytest
import torch

from attention_forward_fwd_amd import fa_fwd, fa_fwd_lse, inputs
from gpu_util import log

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _inputs(B, S, Hq, Hkv, D, dtype, mode, seed):
    w = inputs.Workload("streams", dtype, mode, B, S, Hq, Hkv, D, seed=seed)
    q, k, v = (t.to(DEV) for t in inputs.make_qkv(w))
    m = inputs.make_bitmask(w).to(DEV) if mode == "bitmask" else None
    return w, q, k, v, m


@pytest.mark.parametrize("mode", ["none", "causal", "bitmask"])
def test_side_stream_matches_default_stream(mode):
    # 8192 positions x 2 heads: 32 row tiles per KV head, so V is packed by the pre-pass into a
    # workspace from the pool (not for causal, which packs from 64); split-KV takes its partials
    # from the same pool.
    w, q, k, v, m = _inputs(1, 8192, 2, 2, 128, "bf16", mode, seed=21000)
    log(f"case side stream {mode}")
    o_ref = fa_fwd(q, k, v, mode=mode, scale=w.scale, mask=m)
    o_ref_split = fa_fwd(q, k, v, mode=mode, scale=w.scale, mask=m, kv_splits=3)
    o_ref_lse, lse_ref = fa_fwd_lse(q, k, v, mode=mode, scale=w.scale, mask=m)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o = fa_fwd(q, k, v, mode=mode, scale=w.scale, mask=m)
        o_split = fa_fwd(q, k, v, mode=mode, scale=w.scale, mask=m, kv_splits=3)
        o_lse, lse = fa_fwd_lse(q, k, v, mode=mode, scale=w.scale, mask=m)
    side.synchronize()
    assert torch.equal(o, o_ref), "side-stream O differs from the default stream's"
    assert torch.equal(o_split, o_ref_split), "side-stream split-KV O differs"
    assert torch.equal(o_lse, o_ref_lse) and torch.equal(lse, lse_ref), "side-stream LSE differs"


def test_two_streams_at_once():
    # Two calls with different inputs and shapes in flight together on two streams, each with
    # its own packed-V workspace, then each checked bitwise against the same call made alone.
    a = _inputs(2, 4096, 8, 2, 128, "bf16", "none", seed=21100)
    b = _inputs(1, 4096, 4, 4, 64, "f16", "causal", seed=21200)
    log("case two streams at once")
    ref = []
    for w, q, k, v, m in (a, b):
        ref.append(fa_fwd(q, k, v, mode=w.mode, scale=w.scale, mask=m))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(device=DEV), torch.cuda.Stream(device=DEV)]
    outs = []
    for s, (w, q, k, v, m) in zip(streams, (a, b)):
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            outs.append([fa_fwd(q, k, v, mode=w.mode, scale=w.scale, mask=m) for _ in range(3)])
    for s in streams:
        s.synchronize()
    for r, os_ in zip(ref, outs):
        for o in os_:
            assert torch.equal(o, r), "a call running beside another stream's call changed"


def test_calls_from_several_host_threads():
    # Four host threads, each with its own stream and inputs, call the library at the same time
    # (ctypes releases the GIL during the call); each result must equal the same call made alone.
    import threading
    cases = [_inputs(1, 2048 + 128 * i, 4, 2, 128 if i % 2 == 0 else 64, "bf16" if i % 2 == 0 else "f16",
                     ("none", "causal", "bitmask", "none")[i], seed=21300 + i) for i in range(4)]
    log("case four host threads")
    ref = [fa_fwd(q, k, v, mode=w.mode, scale=w.scale, mask=m) for w, q, k, v, m in cases]
    torch.cuda.synchronize()
    outs = [None] * len(cases)
    errors = []

    def worker(i):
        try:
            w, q, k, v, m = cases[i]
            s = torch.cuda.Stream(device=DEV)
            s.wait_stream(torch.cuda.default_stream(DEV))
            with torch.cuda.stream(s):
                res = [fa_fwd(q, k, v, mode=w.mode, scale=w.scale, mask=m) for _ in range(3)]
            s.synchronize()
            outs[i] = res
        except Exception as e:  # reported in the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not errors, errors
    for r, res in zip(ref, outs):
        assert res is not None
        for o in res:
            assert torch.equal(o, r), "a call made beside calls from other host threads changed"
