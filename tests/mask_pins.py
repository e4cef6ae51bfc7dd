"""Pins for the mask-packing oracle (oracle/mask_pack.py): checks against facts fixed outside it.

  * the hand example (tests/golden/hand_example.json): its byte rows pack to its words, any
    nonzero byte keeps, and its one 64 x 64 block holds kept bits;
  * a library routine: numpy.packbits with little bit order, read as little-endian uint32;
  * round trip through the attention oracle's unpacking (bit_of);
  * closed forms of the summary: an empty mask has no bit set; a single kept (i, j) sets
    exactly bit (i // 64, j // 64); a full mask sets the bits of every tile < ceil(S/64) and no
    other; and a loop-by-loop brute force on small shapes.
Plain functions, so tests/test_oracle_mutations.py can plant mistakes and check they fail.
"""

from __future__ import annotations

import json
import os

import numpy as np

import oracle
from oracle import mask_pack

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_example.json")


def _bytes(seed, shape, p=0.5, values=(1,)):
    r = np.random.default_rng(seed)
    keep = r.random(shape) < p
    vals = r.choice(np.array(values, dtype=np.uint8), size=shape)
    return np.where(keep, vals, 0).astype(np.uint8)


def pin_pack_hand_example():
    g = json.load(open(GOLDEN))
    for key in ("mask_bytes", "mask_bytes_other_values"):
        b = np.array(g[key], dtype=np.uint8)[None, None]
        np.testing.assert_array_equal(oracle.pack_mask(b).ravel(),
                                      np.array(g["mask_words"], dtype=np.uint32), err_msg=key)
        assert int(oracle.tile_summary(b).ravel()[0]) == g["expected_tile_summary"]


def pin_pack_numpy_packbits():
    for S in (32, 64, 96, 1, 31, 33, 100):
        b = _bytes(300 + S, (2, 3, S, S), values=(1, 2, 255))
        W = (S + 31) // 32
        padded = np.zeros((2, 3, S, W * 32), dtype=bool)
        padded[..., :S] = b != 0
        by = np.packbits(padded, axis=-1, bitorder="little")          # [.., W*4] bytes
        want = np.ascontiguousarray(by).view("<u4").astype(np.uint32)
        np.testing.assert_array_equal(oracle.pack_mask(b), want, err_msg=f"S={S}")


def pin_pack_round_trip():
    for S in (5, 40, 77):
        b = _bytes(310 + S, (1, 2, S, S), p=0.3, values=(1, 9))
        np.testing.assert_array_equal(oracle.bit_of(oracle.pack_mask(b), S), b != 0)
        w = oracle.pack_mask(b)
        if S % 32:
            assert (w[..., -1] >> np.uint32(S % 32) == 0).all(), "padding bits must be 0"


def pin_summary_closed_forms():
    for S in (1, 64, 65, 130, 300):
        n_kt = (S + 63) // 64
        z = np.zeros((1, 1, S, S), dtype=np.uint8)
        assert (oracle.tile_summary(z) == 0).all()
        full = np.ones((1, 1, S, S), dtype=np.uint8)
        want = np.zeros(oracle.tile_words(S), dtype=np.uint32)
        for t in range(n_kt):
            want[t // 32] |= np.uint32(1) << np.uint32(t % 32)
        for r in range(n_kt):
            np.testing.assert_array_equal(oracle.tile_summary(full)[0, 0, r], want)
        rng = np.random.default_rng(320 + S)
        for _ in range(5):
            i, j = rng.integers(0, S, size=2)
            one = np.zeros((1, 1, S, S), dtype=np.uint8)
            one[0, 0, i, j] = 3
            s = oracle.tile_summary(one)[0, 0]
            nz = [(r, t) for r in range(s.shape[0]) for t in range(32 * s.shape[1])
                  if (int(s[r, t // 32]) >> (t % 32)) & 1]
            assert nz == [(i // 64, j // 64)], (S, i, j, nz)


def pin_summary_brute_force():
    for S in (70, 200):
        b = _bytes(330 + S, (2, 2, S, S), p=0.002)
        s = oracle.tile_summary(b)
        for bb in range(2):
            for h in range(2):
                for r in range((S + 63) // 64):
                    for t in range((S + 63) // 64):
                        anyk = False
                        for i in range(64 * r, min(S, 64 * r + 64)):
                            for j in range(64 * t, min(S, 64 * t + 64)):
                                anyk = anyk or bool(b[bb, h, i, j])
                        got = (int(s[bb, h, r, t // 32]) >> (t % 32)) & 1
                        assert got == int(anyk), (S, bb, h, r, t)


ALL_PINS = [f for n, f in sorted(globals().items()) if n.startswith("pin_") and callable(f)]
