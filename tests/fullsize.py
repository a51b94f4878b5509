"""Every head of a full-size workload against the fp64 oracle.

The GPU computes the whole workload in one launch; the oracle then runs head
by head (or a few heads at a time, vectorised) on the host, in a thread pool
(numpy's BLAS and ufuncs release the GIL), so host memory stays bounded by a
few heads' fp64 features at once.  Each job copies its own heads off the
device.  Returns the per-head errors so that a test can assert the bar on the
worst head and print it.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np


def workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:   # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def per_head(n_heads: int, chunk: int, job) -> np.ndarray:
    """job(h0, h1) -> errors of heads [h0, h1) (array-like of length h1 - h0)."""
    errs = per_head_rows(n_heads, chunk, job)
    assert errs.ndim == 1, errs.shape
    return errs


def head_slices(tensors, n_heads: int):
    """[B, H, ...] device tensors viewed as [B*H, ...]."""
    return [t.reshape((n_heads,) + tuple(t.shape[2:])) for t in tensors]


def host64(t, h0: int, h1: int) -> np.ndarray:
    return t[h0:h1].detach().cpu().double().numpy()


def report(label: str, errs: np.ndarray) -> tuple[int, float]:
    worst = int(np.argmax(errs))
    print(f"{label}: {errs.size} heads, worst head {worst} err {errs[worst]:.3e}, "
          f"median {np.median(errs):.3e}", flush=True)
    return worst, float(errs[worst])


def per_head_rows(n_heads: int, chunk: int, job) -> np.ndarray:
    """job(h0, h1) -> errors of heads [h0, h1), one row (or value) per head."""
    starts = list(range(0, n_heads, chunk))
    with ThreadPoolExecutor(workers()) as ex:
        parts = list(ex.map(lambda h0: np.asarray(job(h0, min(n_heads, h0 + chunk)), np.float64),
                            starts))
    rows = np.concatenate(parts, axis=0)
    assert rows.shape[0] == n_heads, rows.shape
    return rows
