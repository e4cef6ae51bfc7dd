"""GPU parity at the size limits of the C ABI (sampled rows against the fp64 oracle).

  * MHA with seq_len x n_q_heads x head_dim just under 2^31 elements per batch (S = 131072,
    127 heads, d = 128): the largest offsets the kernel computes, K/V buffer resources just under
    2^32 bytes, and a 4.3 GB packed-V workspace;
  * a bitmask at S = 131072 (2048 row blocks: the largest tile summary a workgroup can list,
    all 64 summary words of a block used), with a sliding-window band so most tiles are dead:
    the tile walk must equal the dense walk bitwise and the oracle within the fp16 bounds.
Inputs are drawn on the device (seeded); only the sampled rows and their heads' K/V are copied
to the host for the oracle."""

import numpy as np
import pytest
import torch

from attention_forward_fwd_amd import fa_fwd, inputs, mask_tiles
from gpu_util import compare, log
import oracle

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _sampled(q, k, v, o, mode, scale, mask, rows, heads):
    """Oracle rows for the given (rows, heads), from host copies of just those slices."""
    qh = q[:, rows][:, :, heads].cpu()
    Hq, Hkv = q.shape[2], k.shape[2]
    G = Hq // Hkv
    kv_heads = sorted({h // G for h in heads})
    kh, vh = k[:, :, kv_heads].cpu(), v[:, :, kv_heads].cpu()
    want = np.zeros((1, len(rows), len(heads), q.shape[3]))
    for hi, h in enumerate(heads):
        g = kv_heads.index(h // G)
        mrow = None if mask is None else mask[:, h:h + 1][:, :, rows].cpu()
        # one query head against its KV head: a 1-head problem over the sampled rows
        res = oracle.attention_rows(_expand(qh[:, :, hi:hi + 1], rows, q.shape[1]),
                                    kh[:, :, g:g + 1], vh[:, :, g:g + 1], mode, scale,
                                    None if mrow is None else _expand_mask(mrow, rows, q.shape[1]),
                                    rows=np.asarray(rows))
        want[:, :, hi] = res[:, :, 0]
    got = o[:, rows][:, :, heads].float().cpu().numpy().astype(np.float64)
    return got, want


def _expand(qrows, rows, S):
    """A [1, S, 1, D] query tensor holding the sampled rows at their positions (others 0)."""
    full = torch.zeros((1, S, 1, qrows.shape[3]), dtype=qrows.dtype)
    full[:, rows] = qrows
    return full


def _expand_mask(mrows, rows, S):
    full = torch.zeros((1, 1, S, mrows.shape[3]), dtype=mrows.dtype)
    full[:, :, rows] = mrows
    return full


def test_max_offsets_mha():
    S, H, D = 131072, 127, 128
    assert S * H * D < 2 ** 31 and S * H * D * 2 > 2 ** 31   # just under the per-batch limit
    w = inputs.Workload("limits", "bf16", "none", 1, S, H, H, D, seed=15000)
    q, k, v = inputs.make_qkv_device(w, DEV)
    log("case max offsets MHA S=131072 H=127 d=128")
    o = fa_fwd(q, k, v, mode="none", scale=w.scale)
    torch.cuda.synchronize()
    rows = [0, 1, 63, 64, 65535, 65536, S - 65, S - 2, S - 1]
    heads = [0, 1, 63, 126]
    got, want = _sampled(q, k, v, o, "none", w.scale, None, rows, heads)
    compare(got, want, q.dtype, "max offsets MHA (9 rows x 4 heads)")


def test_max_tile_summary_band_mask():
    S, D = 131072, 64
    w = inputs.Workload("limits", "f16", "bitmask", 1, S, 1, 1, D, seed=15100)
    q, k, v = inputs.make_qkv_device(w, DEV)
    m = inputs.band_mask(inputs.make_bitmask_device(w, DEV), 1000)
    tiles = mask_tiles(m)
    assert tiles.shape == (1, 1, 2048, 64)
    log("case max tile summary S=131072 band 1000")
    a = fa_fwd(q, k, v, mode="bitmask", scale=w.scale, mask=m)
    b = fa_fwd(q, k, v, mode="bitmask", scale=w.scale, mask=m, tiles=tiles)
    torch.cuda.synchronize()
    assert torch.equal(a, b), "tile walk differs from the dense walk at 2048 row blocks"
    rows = [0, 1, 999, 1000, 1001, 65535, 65536, S - 1001, S - 1]
    got, want = _sampled(q, k, v, b, "bitmask", w.scale, m, rows, [0])
    compare(got, want, q.dtype, "max tile summary (9 rows)")
