"""Test helper: the oracle's attention over many (head, row range) pieces
on a thread pool, for full-size checks.  Each piece is one call of
oracle.attention restricted to a head and a row range; numpy releases the
GIL in its array kernels, and BLAS is held to one thread per piece so that
the pool, not BLAS, spreads the work over the host cores."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle as O


def host_workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def attention_heads(w, heads, rows_per_piece=2048, workers=None):
    """out [N, len(heads), D] and lse [len(heads), N] in fp64 for the given
    heads of workload w, every row."""
    from threadpoolctl import threadpool_limits
    q = np.asarray(w.q, np.float64)
    k = np.asarray(w.k, np.float64)
    v = np.asarray(w.v, np.float64)
    N, D = w.N, w.D
    out = np.zeros((N, len(heads), D), np.float64)
    lse = np.full((len(heads), N), -np.inf, np.float64)
    cu = w.cu_seqlens.astype(np.int64)
    pieces = []
    for b in range(w.B):   # row ranges inside one sequence, so pieces are balanced by their key count
        s, e = int(cu[b]), int(cu[b + 1])
        for r0 in range(s, e, rows_per_piece):
            for t, h in enumerate(heads):
                pieces.append((t, h, r0, min(r0 + rows_per_piece, e), e - s))
    pieces.sort(key=lambda p: -(p[3] - p[2]) * p[4])

    def one(p):
        t, h, r0, r1, _ = p
        o, l = O.attention(q, k, v, w.cu_seqlens, w.startend, w.n_vec, w.causal, w.scale, heads=[h], rows=(r0, r1))
        out[r0:r1, t] = o[r0:r1, h]
        lse[t, r0:r1] = l[h, r0:r1]

    with threadpool_limits(limits=1, user_api="blas"):
        with ThreadPoolExecutor(max_workers=workers or host_workers()) as ex:
            list(ex.map(one, pieces))
    return out, lse
