"""GPU parity of the mask kernels (fa_pack_mask, fa_mask_tiles) against the CPU oracle: bit-exact
on every output word, for ragged lengths, every load width the packer picks (16-, 8-, 4- and
1-byte pieces, from the row length and the base alignment), value spreads, structured masks,
the short random-mask benchmark size, and guard bands around the outputs."""

import numpy as np
import pytest
import torch

from attention_forward_fwd_amd import fa_fwd, inputs, mask_tiles, pack_mask
from gpu_util import log
import oracle

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _bytes(seed, shape, p=0.5, values=(1, 2, 255)):
    r = np.random.default_rng(seed)
    keep = r.random(shape) < p
    vals = r.choice(np.array(values, dtype=np.uint8), size=shape)
    return np.where(keep, vals, 0).astype(np.uint8)


def _gpu_pack(b_np, offset=0):
    """Pack on the GPU; `offset` bytes of misalignment for the input base."""
    n = b_np.size
    buf = torch.zeros(n + 64, dtype=torch.uint8, device=DEV)
    buf[offset:offset + n] = torch.from_numpy(b_np.ravel()).to(DEV)
    src = buf[offset:offset + n].view(b_np.shape)
    w = pack_mask(src)
    torch.cuda.synchronize()
    return w.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("offset", [0, 8, 4, 1])
@pytest.mark.parametrize("S", [1, 7, 31, 32, 33, 100, 128, 136, 1000, 1025])
def test_pack_ragged_and_alignment(S, offset):
    b = _bytes(400 + S + offset, (2, 3, S, S))
    log(f"case pack S={S} offset={offset}")
    np.testing.assert_array_equal(_gpu_pack(b, offset), oracle.pack_mask(b))


@pytest.mark.parametrize("dtype", [torch.bool, torch.int8])
def test_pack_bool_and_int8(dtype):
    S = 96
    b = _bytes(450, (1, 2, S, S), values=(1,))
    t = torch.from_numpy(b).to(DEV).to(dtype)
    w = pack_mask(t)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(w.cpu().numpy().view(np.uint32), oracle.pack_mask(b))


@pytest.mark.parametrize("p", [0.0, 0.003, 1.0])
def test_pack_sparse_and_dense(p):
    S = 300
    b = _bytes(460, (2, 2, S, S), p=p)
    log(f"case pack p={p}")
    np.testing.assert_array_equal(_gpu_pack(b), oracle.pack_mask(b))


def test_pack_short_masked_size():
    # the short random-mask benchmark shape: B16 H16 S1000 (256 MB of bytes)
    w_ = inputs.short_masked(1000)
    b = np.concatenate([_bytes(w_.seed + 70 + i, (1, 16, 1000, 1000)) for i in range(16)])
    log("case pack B16 H16 S1000")
    got = _gpu_pack(b)
    for i in range(16):   # the oracle one batch at a time (bounded host memory)
        np.testing.assert_array_equal(got[i:i + 1], oracle.pack_mask(b[i:i + 1]), err_msg=f"batch {i}")


def _tiles_want(words_np, S):
    keep = oracle.bit_of(words_np, S)
    return oracle.tile_summary(keep.astype(np.uint8))


@pytest.mark.parametrize("S", [1, 63, 64, 65, 129, 1000, 2065])
def test_tiles_random_words(S):
    # random words, padding bits random too (ignored by the summary)
    r = np.random.default_rng(500 + S)
    W = (S + 31) // 32
    words = r.integers(0, 2 ** 32, size=(2, 3, S, W), dtype=np.uint64).astype(np.uint32)
    # sparse: most blocks empty so both outcomes of every bit occur
    words &= (r.random(words.shape) < 0.02).astype(np.uint32) * np.uint32(0xFFFFFFFF)
    t = mask_tiles(torch.from_numpy(words.view(np.int32)).to(DEV))
    torch.cuda.synchronize()
    log(f"case tiles S={S}")
    np.testing.assert_array_equal(t.cpu().numpy().view(np.uint32), _tiles_want(words, S))


def test_tiles_block_structured():
    S = 1000
    b = np.zeros((2, 2, S, S), dtype=np.uint8)
    r = np.random.default_rng(510)
    for _ in range(40):
        bb, h, i, j = r.integers(0, 2), r.integers(0, 2), r.integers(0, S), r.integers(0, S)
        b[bb, h, i, j] = 1
    b[0, 0, :, :64] = 1     # a whole column of tiles
    w = pack_mask(torch.from_numpy(b).to(DEV))
    t = mask_tiles(w)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(t.cpu().numpy().view(np.uint32), oracle.tile_summary(b))


def test_pack_then_attention():
    # pack_mask's words drive fa_fwd exactly as the oracle's packing of the same bytes does
    B, H, S, D = 2, 4, 333, 64
    b = _bytes(520, (B, H, S, S), p=0.4)
    q, k, v = inputs.make_qkv(inputs.Workload("edge", "f16", "none", B, S, H, H, D, seed=521))
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    w_gpu = pack_mask(torch.from_numpy(b).to(DEV))
    w_cpu = torch.from_numpy(oracle.pack_mask(b).view(np.int32)).to(DEV)
    a = fa_fwd(qd, kd, vd, mode="bitmask", mask=w_gpu)
    c = fa_fwd(qd, kd, vd, mode="bitmask", mask=w_cpu)
    torch.cuda.synchronize()
    assert torch.equal(a, c)


def test_guard_bands():
    S, B, H = 77, 1, 2
    b = _bytes(530, (B, H, S, S))
    W, R = (S + 31) // 32, (S + 63) // 64
    n, pad = B * H * S * W, 1024
    buf = torch.full((n + 2 * pad,), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    out = buf[pad:pad + n].view(B, H, S, W)
    pack_mask(torch.from_numpy(b).to(DEV), out=out)
    nt = B * H * R * ((R + 31) // 32)
    tbuf = torch.full((nt + 2 * pad,), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    tout = tbuf[pad:pad + nt].view(B, H, R, (R + 31) // 32)
    mask_tiles(out, out=tout)
    torch.cuda.synchronize()
    for g in (buf, tbuf):
        assert (g[:pad] == 0x5A5A5A5A).all() and (g[-pad:] == 0x5A5A5A5A).all(), "guard band written"
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), oracle.pack_mask(b))
    np.testing.assert_array_equal(tout.cpu().numpy().view(np.uint32), oracle.tile_summary(b))
