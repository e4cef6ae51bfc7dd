"""Worker side of the full-tensor gate: the fp64 oracle of one (batch, query head) in a worker
process.  Imports only numpy and the oracle (no torch, no GPU library), so spawned workers never
touch the GPU."""

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def init_worker():
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)


def oracle_pair(args):
    """Oracle output of one (batch, query head): q, k, v are [1, S, 1, D] slices; returns [S, D]
    float64."""
    import oracle
    q, k, v, mode, scale = args
    return oracle.attention(q, k, v, mode, scale)[0, :, 0, :]
