"""Row-parallel drivers of the fp64 oracle (test infrastructure only).

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the tests, the smoke
check and the CPU-baseline leg of the benchmark use it.

The oracle computes every query row over its complete key row, so its rows are
independent: O, LSE and dQ of a row depend on that row alone, and dK, dV are sums
over rows of per-row terms (the loss sum_i dO_i . O_i is a sum over the rank's
rows).  These drivers cut a rank's rows into contiguous groups of about equal cost,
run ``attention_fwd`` / ``attention_bwd`` on each group (one batch element and one
query head at a time) in a pool of worker threads, and then place (O, LSE, dQ) or
add (dK, dV) the groups' results.  Nothing else changes: the arithmetic is the
oracle's own, only the order of the fp64 additions that form dK and dV differs.

Workers are threads, not processes: NumPy's loops and the BLAS calls release the
interpreter lock, so the threads run in parallel, and no worker process inherits
the state of a caller that already holds a GPU.  BLAS is held to one thread per
worker while a pool runs, so the workers do not oversubscribe the cores.
"""
from __future__ import annotations

import contextlib
import os
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .attention import _default_scale, _kv_head, attention_bwd, attention_fwd

MAX_WORKERS = 16


def default_workers() -> int:
    """Threads for a pool: the host cores this process may use, at most MAX_WORKERS."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux hosts
        n = os.cpu_count() or 1
    return max(1, min(MAX_WORKERS, n))


@contextlib.contextmanager
def _one_blas_thread():
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover - then BLAS keeps its own setting
        yield
        return
    with threadpool_limits(1):
        yield


def _row_groups(rows: np.ndarray, causal: bool, seq_total: int, n_groups: int):
    """Contiguous index ranges of `rows` of about equal cost.  A row's cost is the
    number of keys the oracle multiplies it with: its position + 1 when causal (the
    visible prefix), every key otherwise."""
    n = rows.size
    if n == 0:
        return []
    cost = (rows + 1).astype(np.float64) if causal else np.full(n, float(seq_total))
    edges = np.searchsorted(np.cumsum(cost), np.linspace(0.0, cost.sum(), n_groups + 1)[1:-1])
    bounds = np.unique(np.concatenate(([0], edges, [n])))
    return [(int(a), int(b)) for a, b in zip(bounds[:-1], bounds[1:]) if b > a]


def attention_fwd_rows(Qg, Kg, Vg, rows, causal: bool, scale: float | None = None,
                       heads=None, bounds=None, workers: int | None = None):
    """``attention_fwd`` with its rows split over a pool of `workers` threads.

    Same arguments and results: O [B, len(heads) or Hq, len(rows), d] and LSE.
    """
    B, Hq, S, d = Qg.shape
    Hkv = Kg.shape[1]
    scale = _default_scale(d) if scale is None else scale
    rows = np.asarray(rows, dtype=np.int64)
    heads = list(range(Hq)) if heads is None else list(heads)
    workers = default_workers() if workers is None else max(1, int(workers))
    O = np.zeros((B, len(heads), rows.size, Vg.shape[3]), dtype=np.float64)
    LSE = np.full((B, len(heads), rows.size), -np.inf, dtype=np.float64)
    groups = _row_groups(rows, causal, S, workers)

    def job(bi, hi, h, a, e):  # each job writes its own rows
        g = _kv_head(h, Hq, Hkv)
        bl = None if bounds is None else [bounds[bi]]
        o, lse = attention_fwd(Qg[bi:bi + 1, h:h + 1], Kg[bi:bi + 1, g:g + 1],
                               Vg[bi:bi + 1, g:g + 1], rows[a:e], causal, scale, bounds=bl)
        O[bi, hi, a:e] = o[0, 0]
        LSE[bi, hi, a:e] = lse[0, 0]

    _run(workers, job, [(bi, hi, h, a, e) for bi in range(B) for hi, h in enumerate(heads)
                        for a, e in groups])
    return O, LSE


def attention_bwd_rows(Qg, Kg, Vg, dO_rows, rows, causal: bool, scale: float | None = None,
                       heads=None, bounds=None, workers: int | None = None):
    """``attention_bwd`` with its rows split over a pool of `workers` threads.

    Same arguments and results: dQ [B, len(heads) or Hq, len(rows), d] in local row
    order, dK and dV [B, Hkv, S, d] in global order (each KV head summed over the
    query heads in `heads` that read it).
    """
    B, Hq, S, d = Qg.shape
    Hkv = Kg.shape[1]
    scale = _default_scale(d) if scale is None else scale
    rows = np.asarray(rows, dtype=np.int64)
    heads = list(range(Hq)) if heads is None else list(heads)
    workers = default_workers() if workers is None else max(1, int(workers))
    dQ = np.zeros((B, len(heads), rows.size, d), dtype=np.float64)
    dK = np.zeros((B, Hkv, S, d), dtype=np.float64)
    dV = np.zeros((B, Hkv, S, Vg.shape[3]), dtype=np.float64)
    groups = _row_groups(rows, causal, S, workers)

    lock = threading.Lock()

    def job(bi, hi, h, a, e):  # own dQ rows; dK, dV added under the lock
        g = _kv_head(h, Hq, Hkv)
        bl = None if bounds is None else [bounds[bi]]
        dq, dk, dv = attention_bwd(Qg[bi:bi + 1, h:h + 1], Kg[bi:bi + 1, g:g + 1],
                                   Vg[bi:bi + 1, g:g + 1], dO_rows[bi:bi + 1, hi:hi + 1, a:e],
                                   rows[a:e], causal, scale, bounds=bl)
        dQ[bi, hi, a:e] = dq[0, 0]
        # keys after the group's last row received nothing when causal: add the prefix
        lim = int(rows[a:e].max()) + 1 if causal else S
        with lock:
            dK[bi, g, :lim] += dk[0, 0, :lim]
            dV[bi, g, :lim] += dv[0, 0, :lim]

    _run(workers, job, [(bi, hi, h, a, e) for bi in range(B) for hi, h in enumerate(heads)
                        for a, e in groups])
    return dQ, dK, dV


def _run(workers, job, tasks):
    """Runs job(*t) for every task on `workers` threads; re-raises the first failure."""
    with _one_blas_thread(), ThreadPoolExecutor(workers) as ex:
        for f in [ex.submit(job, *t) for t in tasks]:
            f.result()
