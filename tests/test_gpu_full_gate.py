"""Full-tensor gate: every element of full-size prefill outputs (non-causal and causal MHA,
causal GQA 32/8 and non-causal GQA 32/4, all at B4 S8192 H16/32 d128 bf16) against the fp64
oracle, in the launch configuration the benchmark times.

The oracle runs per (batch, query head) on host threads (gpu_util.oracle_rows); about 10-20 s
of host time per case on a 16-core share.  The other prefill tests compare sampled rows at full
key length."""

import time

import numpy as np
import pytest
import torch

from attention_forward_fwd_amd import fa_fwd, inputs
from gpu_util import TOL, WORKERS, log, oracle_rows

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(400)
@pytest.mark.parametrize("workload", [
    lambda: inputs.mha_prefill(4, 8192, False),
    lambda: inputs.mha_prefill(4, 8192, True),
    lambda: inputs.gqa_prefill(4, 8192, 8, True),
    lambda: inputs.gqa_prefill(4, 8192, 4, False),
], ids=["mha-none-B4S8192", "mha-causal-B4S8192", "gqa32_8-causal-B4S8192", "gqa32_4-none-B4S8192"])
def test_full_tensor(workload):
    w = workload()
    log(f"case full tensor {w.label}: {w.batch * w.n_q_heads} (batch, head) pairs on {WORKERS} threads")
    q, k, v = inputs.make_qkv(w)
    dev = torch.device("cuda:0")
    o = fa_fwd(q.to(dev), k.to(dev), v.to(dev), mode=w.mode, scale=w.scale)
    torch.cuda.synchronize()
    got = o.float().cpu().numpy()
    del o
    t0 = time.time()
    want = oracle_rows(q, k, v, w.mode, w.scale)
    log(f"  oracle {time.time() - t0:.1f} s")
    assert np.isfinite(got).all()
    err = np.abs(got.astype(np.float64) - want)
    mx, mean = float(err.max()), float(err.mean())
    log(f"  {w.label} full tensor ({err.size} elements): max_abs={mx:.3e} mean_abs={mean:.3e}")
    tmax, tmean = TOL[q.dtype]
    assert mx <= tmax and mean <= tmean, f"max {mx:.3e} (<= {tmax}) mean {mean:.3e} (<= {tmean})"
