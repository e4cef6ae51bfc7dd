"""CPU oracle for masked softmax attention -- TEST INFRASTRUCTURE, NOT PRODUCT CODE.

Only the test suite, the package smoke check and the benchmark's CPU-baseline leg may import
anything from here.  The HIP library never links, calls or imports it, and it imports
nothing from the HIP path.  `attention` is the plain fp64 definition (`attention_lse` adds each
row's log-sum-exp); `attention_brute` is a 50-digit `decimal` brute force used to pin them
on tiny inputs.  `pack_mask` and `tile_summary` define the packing of a byte mask into that
layout and its per-64x64-block summary.
"""

from .masked_attention import (MODES, attention, attention_flops, attention_lse, attention_rows,
                               bit_of, keep_rows, kv_head_index, mask_words, masked_logsumexp,
                               masked_softmax)
from .brute import attention_brute
from .mask_pack import pack_mask, packed_words, tile_summary, tile_words

__all__ = ["MODES", "attention", "attention_lse", "attention_rows", "attention_flops",
           "attention_brute", "bit_of", "keep_rows", "kv_head_index", "mask_words",
           "masked_logsumexp", "masked_softmax", "pack_mask", "packed_words", "tile_summary",
           "tile_words"]
