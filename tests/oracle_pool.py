"""Runs the fp64 oracle over many heads at once, for full-size comparisons.

Each (batch, head) is an independent call of ``oracle.attention_forward`` on
that head's slice; the calls run on a pool of threads (numpy releases the
interpreter lock inside its array loops and BLAS products, so the heads really
run in parallel), with one BLAS thread per worker.  No process is forked, so
nothing here touches the GPU state of the calling process.  The arithmetic is
the oracle's, unchanged: a head's result does not depend on the others.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle


def host_cores() -> int:
    """Cores this process may run on (the box's share, not the machine's)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        return os.cpu_count() or 1


def forward_by_heads(q, k, v, scale, causal, rows=None, workers=None, progress=None):
    """(O, LSE) of ``oracle.attention_forward`` for all heads of [B, H, N, d]
    inputs; ``rows`` as there ([R] or [B, H, R]).  ``progress(done, total)`` is
    called after each head."""
    from threadpoolctl import threadpool_limits
    B, H = q.shape[:2]
    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64)
        if rows.ndim == 1:
            rows = np.broadcast_to(rows, (B, H, rows.shape[0]))
    R = q.shape[2] if rows is None else rows.shape[-1]
    O = np.empty((B, H, R, q.shape[3]))
    L = np.empty((B, H, R))
    workers = min(workers or host_cores(), 16, B * H)
    done = [0]

    def one(bh):
        b, h = divmod(bh, H)
        r = None if rows is None else rows[b, h][None, None]
        o, lse = oracle.attention_forward(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1],
                                          v[b:b + 1, h:h + 1], scale, causal, rows=r)
        O[b, h], L[b, h] = o[0, 0], lse[0, 0]
        done[0] += 1
        if progress is not None:
            progress(done[0], B * H)

    with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
        for f in [ex.submit(one, bh) for bh in range(B * H)]:
            f.result()
    return O, L
