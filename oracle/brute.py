"""Arbitrary-precision brute force of masked softmax attention, for tiny inputs only.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  It exists to pin the fp64 oracle in
oracle/masked_attention.py: it is a second, loop-by-loop statement of the same definition in
Python's `decimal` arithmetic (50 significant digits), written without numpy, so a slip in
the vectorised oracle (a transposed operand, a wrong broadcast, a wrong head index) shows up
as a disagreement far above fp64 rounding.

Definition followed (the FlashAttention forward result; pages: https://yetianai.com/news/16520
section "传统进化搜索的天花板" for the tiled computation whose result this is, and
https://yunpan.plus/t/19526-1-1 section "AI生成的代码质量如何？" excerpt 2 for the bitmask
rule): O[b,i,h] = sum_j softmax_j(scale * <Q[b,i,h], K[b,j,h//G]> over kept j) * V[b,j,h//G],
and 0 for a row with no kept key; and LSE[b,h,i] = ln sum_{kept j} exp(scale * <Q, K_j>),
-inf for a row with no kept key.
"""

from __future__ import annotations

from decimal import Decimal, getcontext

getcontext().prec = 50


def _d(x: float) -> Decimal:
    return Decimal(float(x))  # exact: every binary float is a finite decimal


def attention_brute(q, k, v, mode: str, scale: float, mask=None, with_lse: bool = False):
    """q: nested lists [B][S][Hq][D] of floats; k, v: [B][S][Hkv][D]; mask: [B][Hq][S][W] ints.

    Returns nested lists [B][S][Hq][D] of Decimal; with_lse=True also returns the
    log-sum-exp as nested lists [B][Hq][S] of Decimal (Decimal('-Infinity') for a row with
    no kept key)."""
    B, S, Hq, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv = len(k[0][0])
    G = Hq // Hkv
    sc = _d(scale)
    out = []
    lse = [[[Decimal("-Infinity")] * S for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        ob = []
        for i in range(S):
            oi = []
            for h in range(Hq):
                g = h // G
                kept = []
                for j in range(S):
                    if mode == "none":
                        ok = True
                    elif mode == "causal":
                        ok = j <= i
                    else:
                        word = int(mask[b][h][i][j // 32])
                        ok = (word >> (j % 32)) & 1 == 1
                    if ok:
                        dot = sum(_d(q[b][i][h][t]) * _d(k[b][j][g][t]) for t in range(D))
                        kept.append((j, sc * dot))
                if not kept:
                    oi.append([Decimal(0)] * D)
                    continue
                m = max(s for _, s in kept)
                w = [(j, (s - m).exp()) for j, s in kept]
                den = sum(x for _, x in w)
                lse[b][h][i] = m + den.ln()
                row = []
                for t in range(D):
                    num = sum(x * _d(v[b][j][g][t]) for j, x in w)
                    row.append(num / den)
                oi.append(row)
            ob.append(oi)
        out.append(ob)
    return (out, lse) if with_lse else out
