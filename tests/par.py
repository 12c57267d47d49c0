"""Run an oracle call over a batch in chunks on host threads.

The oracle's per-matrix loops (star reverse mode, star solve / sample) are
single-threaded; its C entry points release the GIL (ctypes), so chunks of
the batch run side by side on a thread pool.  Only the batching changes: each
chunk goes through the oracle exactly as a smaller batch would.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np


def workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def chunked(fn, B, batched, scalars=(), n_workers=None):
    """fn(*[a[lo:hi] for a in batched], *scalars-sliced) for chunks of the
    leading axis; every output of fn (a tuple of arrays with a leading batch
    axis) is concatenated back in order.  `scalars` are per-matrix arrays of
    shape [B] passed after the batched ones."""
    n_workers = n_workers or workers()
    step = max(1, -(-B // n_workers))
    bounds = [(lo, min(B, lo + step)) for lo in range(0, B, step)]

    def one(lh):
        lo, hi = lh
        return fn(*[a[lo:hi] for a in batched], *[s[lo:hi] for s in scalars])

    with ThreadPoolExecutor(max_workers=n_workers) as ex:
        parts = list(ex.map(one, bounds))
    if not isinstance(parts[0], tuple):
        return np.concatenate(parts)
    return tuple(np.concatenate([p[k] for p in parts]) for k in range(len(parts[0])))
