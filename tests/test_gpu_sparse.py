"""GPU parity of the tile-summary walk (fa_fwd_ex with `tiles`): with the summary of the mask
(mask_tiles), the result must equal the dense walk's bit for bit (O and LSE) and the oracle
within the bitmask bounds, on structured masks (packed documents, cleared 64x64 blocks, a
single live block, nothing kept), on each workgroup shape (128 rows, 256 rows, GQA groups,
two summary words per block), with a superset summary (every bit set), and with an automatic
split-KV request (which a tile walk never splits)."""

import numpy as np
import pytest
import torch

from attention_forward_fwd_amd import fa_fwd, fa_fwd_lse, inputs, mask_tiles
from gpu_util import compare, log, to64
import oracle

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _case(S, Hq, Hkv, D, dtype, seed):
    w = inputs.Workload("sparse", dtype, "bitmask", 2, S, Hq, Hkv, D, seed=seed)
    q, k, v = inputs.make_qkv(w)
    return w, q, k, v, inputs.make_bitmask(w)


def _both(q, k, v, m, tiles):
    qd, kd, vd, md = q.to(DEV), k.to(DEV), v.to(DEV), m.to(DEV)
    o_d, l_d = fa_fwd_lse(qd, kd, vd, mode="bitmask", mask=md)
    o_s, l_s = fa_fwd_lse(qd, kd, vd, mode="bitmask", mask=md, tiles=tiles)
    o_s2 = fa_fwd(qd, kd, vd, mode="bitmask", mask=md, tiles=tiles)
    torch.cuda.synchronize()
    return o_d, l_d, o_s, l_s, o_s2


@pytest.mark.parametrize("S,Hq,Hkv,D,dtype,kind", [
    (1000, 4, 4, 64, "f16", "docs4"),       # 128-row workgroups, packed documents
    (333, 8, 2, 128, "bf16", "blocks"),     # GQA group of 4: the summary is ORed over heads
    (1030, 8, 1, 64, "f16", "docs3"),       # 8240 rows per KV head: 256-row workgroups
    (2100, 2, 2, 128, "bf16", "docs8"),     # 33 row blocks: two summary words per block
    (65, 3, 3, 64, "f16", "blocks"),
    (1, 2, 1, 64, "bf16", "docs1"),
])
def test_sparse_walk_equals_dense(S, Hq, Hkv, D, dtype, kind):
    w, q, k, v, m = _case(S, Hq, Hkv, D, dtype, seed=13000 + S + Hq)
    if kind.startswith("docs"):
        m = inputs.document_mask(m, min(int(kind[4:]), S), seed=w.seed + 1)
    else:
        m = inputs.empty_tiles(m, 64, 0.7, seed=w.seed + 2)
    tiles = mask_tiles(m.to(DEV))
    label = f"sparse {kind} S={S} H{Hq}/{Hkv} d{D} {dtype}"
    log(f"case {label}")
    o_d, l_d, o_s, l_s, o_s2 = _both(q, k, v, m, tiles)
    assert torch.equal(o_s, o_d), "tile walk changed O"
    assert torch.equal(o_s2, o_d), "tile walk (no LSE) changed O"
    assert torch.equal(l_s, l_d), "tile walk changed the LSE"
    compare(to64(o_s), oracle.attention(q, k, v, "bitmask", w.scale, m), q.dtype, label)


def test_sparse_nothing_kept():
    w, q, k, v, m = _case(700, 4, 2, 128, "bf16", seed=13100)
    m = torch.zeros_like(m)
    tiles = mask_tiles(m.to(DEV))
    _, _, o_s, l_s, _ = _both(q, k, v, m, tiles)
    assert (o_s == 0).all() and torch.isneginf(l_s).all()


def test_sparse_one_live_block():
    w, q, k, v, m = _case(600, 2, 2, 64, "f16", seed=13200)
    keep = torch.zeros_like(m)
    keep[:, :, 128:192, 6:8] = m[:, :, 128:192, 6:8]      # rows 128..191 x keys 192..255
    tiles = mask_tiles(keep.to(DEV))
    o_d, l_d, o_s, l_s, _ = _both(q, k, v, keep, tiles)
    assert torch.equal(o_s, o_d) and torch.equal(l_s, l_d)
    compare(to64(o_s), oracle.attention(q, k, v, "bitmask", w.scale, keep), q.dtype, "one block")


def test_sparse_superset_summary():
    # every summary bit set (also past the last tile): the walk visits every tile, nothing changes
    w, q, k, v, m = _case(500, 4, 4, 64, "f16", seed=13300)
    R = (500 + 63) // 64
    tiles = torch.full((2, 4, R, (R + 31) // 32), -1, dtype=torch.int32, device=DEV)
    o_d, l_d, o_s, l_s, _ = _both(q, k, v, m, tiles)
    assert torch.equal(o_s, o_d) and torch.equal(l_s, l_d)


def test_sparse_walk_with_automatic_split_request():
    # kv_splits=0 (automatic) never splits a tile-summary walk: same result as the walk alone
    w, q, k, v, m = _case(1000, 2, 2, 64, "f16", seed=13400)
    m = inputs.document_mask(m, 3, seed=13401)
    tiles = mask_tiles(m.to(DEV))
    qd, kd, vd, md = q.to(DEV), k.to(DEV), v.to(DEV), m.to(DEV)
    a = fa_fwd(qd, kd, vd, mode="bitmask", mask=md, tiles=tiles)
    b = fa_fwd(qd, kd, vd, mode="bitmask", mask=md, tiles=tiles, kv_splits=0)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
