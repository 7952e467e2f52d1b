"""Runs the oracle over independent pieces of a workload on a pool of threads.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pieces are the ones the definitions make independent: logits rows (H is a
per-row quantity), hidden-state rows of a layer (D is per token), and layers
(window attention, fusion and selection of layer l use only layer l's tensors
plus H and D).  Each piece is computed by the oracle function unchanged, on its
own slice of the input; the pool only decides which thread runs which piece,
and results are put back in piece order, so the output is the same as one call
over the whole input.

numpy releases the interpreter lock inside its array loops, sorts, partitions
and BLAS calls, so threads run the pieces in parallel.  BLAS is held to one
thread per call while the pool runs, so the thread count reported is the number
of threads doing the work.
"""
from __future__ import annotations

import concurrent.futures as cf
import contextlib
import os


def host_threads(limit: int | None = 16) -> int:
    """Threads this process may run on (its CPU affinity), at most ``limit``."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, limit) if limit else n)


@contextlib.contextmanager
def _one_blas_thread():
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:
        yield
        return
    with threadpool_limits(limits=1):
        yield


def map_pieces(fn, pieces, threads: int | None = None) -> list:
    """[fn(p) for p in pieces], run on ``threads`` threads (default: the
    affinity count, at most 16), in piece order."""
    pieces = list(pieces)
    threads = threads or host_threads()
    if threads <= 1 or len(pieces) <= 1:
        return [fn(p) for p in pieces]
    with _one_blas_thread(), cf.ThreadPoolExecutor(threads) as ex:
        return list(ex.map(fn, pieces))


def row_chunks(n: int, rows: int):
    """(start, stop) pairs that cover [0, n) in chunks of ``rows``."""
    return [(r0, min(n, r0 + rows)) for r0 in range(0, n, rows)]
