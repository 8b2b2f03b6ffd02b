"""Process pool over channel shards for the oracle (test infrastructure only).

The long convolutions, gates and skips act channel by channel, so the oracle
can split the channels into contiguous shards and run each shard's recurrence
in its own process ("spawn" start: the workers import numpy and this package
only). Each worker does exactly the arithmetic the single-process call does on
its channels; the shards are concatenated back in channel order.
"""
from __future__ import annotations

import multiprocessing
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np


def default_workers() -> int:
    """Cores this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _one_thread():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:
        pass


def channel_shards(fn, channels: int, workers: int, args_of, axis: int = 1) -> np.ndarray:
    """Runs fn(*args_of(slice)) for contiguous channel slices in `workers`
    processes and concatenates the results along `axis`."""
    workers = max(1, min(workers, channels))
    bounds = np.linspace(0, channels, workers + 1).astype(int)
    slices = [slice(int(a), int(b)) for a, b in zip(bounds[:-1], bounds[1:]) if b > a]
    if len(slices) == 1:
        return fn(*args_of(slices[0]))
    # a worker that cannot start (or dies) fails the call instead of being respawned
    with ProcessPoolExecutor(len(slices), mp_context=multiprocessing.get_context("spawn"),
                             initializer=_one_thread) as pool:
        futures = [pool.submit(fn, *args_of(sl)) for sl in slices]
        parts = [f.result() for f in futures]
    return np.concatenate(parts, axis=axis)
