"""The float64 oracle over a whole full-size workload, in parallel worker processes
(test infrastructure only: it calls oracle.ref and nothing of the HIP path).

One job is one (batch, query head): the worker upcasts that head's q and its kv
head's k and v, and evaluates every query row in blocks of 1024 rows, each row
still seeing its full score row (oracle.ref.attention with ``rows``).  Workers
are spawned with one BLAS thread each; their number is the CPU affinity of the
process, at most 16 (the host share of one GPU).
"""

from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np

ROW_BLOCK = 1024


def workers() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _head_job(args):
    from oracle import ref
    b, h, qh, kh, vh, opts, slope = args
    S = qh.shape[0]
    out = np.empty((S, qh.shape[1]), dtype=np.float64)
    lse = np.empty((S,), dtype=np.float64)
    kw = dict(opts)
    if slope is not None:
        kw["alibi_slopes"] = np.asarray([slope], dtype=np.float64)
    for r0 in range(0, S, ROW_BLOCK):
        rows = np.arange(r0, min(S, r0 + ROW_BLOCK))
        o, ls = ref.attention(qh[None, :, None], kh[None, :, None], vh[None, :, None], rows=rows, **kw)
        out[rows] = o[0, :, 0]
        lse[rows] = ls[0, 0]
    return b, h, out, lse


def dense_full(q, k, v, softmax_scale=None, causal=False, window=(-1, -1), softcap=0.0, alibi_slopes=None):
    """Oracle (out [B,S,Hq,D], lse [B,Hq,S]) float64 of a dense workload, over all rows.

    q, k, v: CPU tensors (any float dtype, upcast exactly; float8 through float32).
    """
    import torch
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    group = Hq // Hkv
    up = lambda t: t.float().numpy() if t.dtype != torch.float64 else t.numpy()
    qn, kn, vn = up(q), up(k), up(v)
    slopes = None if alibi_slopes is None else [float(x) for x in alibi_slopes.reshape(-1)]
    opts = dict(softmax_scale=softmax_scale, causal=causal, window=window, softcap=softcap)
    jobs = [(b, h, qn[b, :, h], kn[b, :, h // group], vn[b, :, h // group], opts,
             None if slopes is None else slopes[h]) for b in range(B) for h in range(Hq)]
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    out = np.zeros((B, S, Hq, D), dtype=np.float64)
    lse = np.zeros((B, Hq, S), dtype=np.float64)
    with mp.get_context("spawn").Pool(workers()) as pool:
        for b, h, o, ls in pool.imap_unordered(_head_job, jobs, chunksize=1):
            out[b, :, h] = o
            lse[b, h] = ls
    return out, lse
