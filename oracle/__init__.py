"""CPU oracle for masked softmax attention -- TEST INFRASTRUCTURE, NOT PRODUCT CODE.

Only the test suite, the package smoke check and the benchmark's CPU-baseline leg may import
anything from here.  The HIP library never links, calls or imports it, and it imports
nothing from the HIP path.  `attention` is the plain fp64 definition (`attention_lse` adds each
row's log-sum-exp); `attention_brute` is a 50-digit `decimal` brute force used to pin them
on tiny inputs.
"""

from .masked_attention import (MODES, attention, attention_flops, attention_lse, attention_rows,
                               bit_of, keep_rows, kv_head_index, mask_words, masked_logsumexp,
                               masked_softmax)
from .brute import attention_brute

__all__ = ["MODES", "attention", "attention_lse", "attention_rows", "attention_flops",
           "attention_brute", "bit_of", "keep_rows", "kv_head_index", "mask_words",
           "masked_logsumexp", "masked_softmax"]
