"""Full-tensor gate (opt-in: FA_FULL_GATE=1): every element of a full-size prefill output
against the fp64 oracle, the oracle spread over the host cores in worker processes.

The regular parity tests compare full-size prefill workloads on sampled rows at full key
length; this gate compares all B*S*Hq rows once.  It takes minutes of CPU time, so the default
test run skips it."""

import multiprocessing as mp
import os
import time

import numpy as np
import pytest
import torch

from attention_forward_fwd_amd import fa_fwd, inputs
from gpu_util import TOL, log
import oracle_pool

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(os.environ.get("FA_FULL_GATE") != "1",
                                 reason="full-tensor gate runs only with FA_FULL_GATE=1")]


@pytest.mark.timeout(1100)
@pytest.mark.parametrize("workload", [
    lambda: inputs.mha_prefill(4, 8192, False),
    lambda: inputs.mha_prefill(4, 8192, True),
    lambda: inputs.gqa_prefill(4, 8192, 8, True),
    lambda: inputs.gqa_prefill(4, 8192, 4, False),
], ids=["mha-none-B4S8192", "mha-causal-B4S8192", "gqa32_8-causal-B4S8192", "gqa32_4-none-B4S8192"])
def test_full_tensor(workload):
    w = workload()
    q, k, v = inputs.make_qkv(w)
    dev = torch.device("cuda:0")
    o = fa_fwd(q.to(dev), k.to(dev), v.to(dev), mode=w.mode, scale=w.scale)
    torch.cuda.synchronize()
    got = o.float().cpu().numpy()
    G = w.n_q_heads // w.n_kv_heads
    qf, kf, vf = (t.float().numpy() for t in (q, k, v))   # bf16 values, exact in float32
    tasks = [(qf[b:b + 1, :, h:h + 1], kf[b:b + 1, :, h // G:h // G + 1], vf[b:b + 1, :, h // G:h // G + 1],
              w.mode, w.scale) for b in range(w.batch) for h in range(w.n_q_heads)]
    n_proc = min(16, os.cpu_count() or 1)
    log(f"case full tensor {w.label}: {len(tasks)} (batch, head) pairs over {n_proc} processes")
    tmax, tmean = TOL[q.dtype]
    mx, total, n = 0.0, 0.0, 0
    t0 = time.time()
    with mp.get_context("spawn").Pool(n_proc, initializer=oracle_pool.init_worker) as pool:
        for idx, want in enumerate(pool.imap(oracle_pool.oracle_pair, tasks)):
            b, h = divmod(idx, w.n_q_heads)
            err = np.abs(got[b, :, h, :].astype(np.float64) - want)
            mx = max(mx, float(err.max()))
            total += float(err.sum())
            n += err.size
            if idx % 8 == 7:
                log(f"  {idx + 1}/{len(tasks)} pairs, {time.time() - t0:.0f} s, max_abs so far {mx:.3e}")
    mean = total / n
    log(f"  {w.label} full tensor ({n} elements): max_abs={mx:.3e} mean_abs={mean:.3e}")
    assert np.isfinite(got).all()
    assert mx <= tmax and mean <= tmean, f"max {mx:.3e} (<= {tmax}) mean {mean:.3e} (<= {tmean})"
