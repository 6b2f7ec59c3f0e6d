"""Runs the CPU oracle's encoder and dequantizer on large weights in worker
processes (test infrastructure).

The oracle functions themselves are unchanged: a weight [rows, cols] is cut
into row slabs whose element counts are multiples of 16384 (one second-level
group of 256 blocks of 64), so that every block and every group lies wholly in
one slab; each slab goes through oracle.nf4_quantize, nf4_double_quant and
nf4_dequantize, and the pieces are concatenated in order.  Because no group
straddles a slab, the result is exactly the whole-matrix call's.
"""
from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os

import numpy as np

GROUP_ELEMS = 64 * 256


def _workers():
    n = len(os.sched_getaffinity(0))
    return max(1, min(16, n))


def _slab_job(args):
    import oracle as O
    w, bf16, cols, dequant = args
    rows = w.shape[0]
    Wf = O.bf16_value(w).astype(np.float32) if bf16 else w
    codes, absmax = O.nf4_quantize(Wf)
    c2, c1 = O.nf4_double_quant(absmax)
    Wq = O.nf4_dequantize(codes, c2, c1, rows, cols) if dequant else None
    return codes, absmax, c2, c1, Wq


def slab_rows(rows, cols, parts):
    """Row boundaries of at most `parts` slabs, each a whole number of groups."""
    step = GROUP_ELEMS // np.gcd(GROUP_ELEMS, cols)        # rows per whole number of groups
    units = -(-rows // step)
    per = max(1, -(-units // parts))
    bounds = list(range(0, rows, per * step)) + [rows]
    return list(zip(bounds[:-1], bounds[1:]))


def quantize(W, dequant=True, workers=None):
    """Oracle (codes, absmax, c2, c1, Wq or None) of W [rows, cols].

    W: float32 array, or uint16 array of bf16 bit patterns.  Only the last slab
    may end inside a group (the matrix's own last, partial group)."""
    W = np.ascontiguousarray(W)
    bf16 = W.dtype == np.uint16
    rows, cols = W.shape
    parts = (workers or _workers()) * 2
    jobs = [(W[a:b], bf16, cols, dequant) for a, b in slab_rows(rows, cols, parts)]
    if len(jobs) == 1:
        outs = [_slab_job(jobs[0])]
    else:
        with cf.ProcessPoolExecutor(max_workers=workers or _workers(), mp_context=mp.get_context("spawn")) as ex:
            outs = list(ex.map(_slab_job, jobs))
    codes = np.concatenate([o[0] for o in outs])
    absmax = np.concatenate([o[1] for o in outs])
    c2 = np.concatenate([o[2] for o in outs])
    c1 = np.concatenate([o[3] for o in outs])
    Wq = np.concatenate([o[4] for o in outs]) if dequant else None
    return codes, absmax, c2, c1, Wq
