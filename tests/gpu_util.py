"""Shared helpers for the GPU tests (device handling and case printing)."""
from __future__ import annotations

import sys

import pytest


def device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_51_amd as fa
    fa.load()  # raises when the HIP library is missing: no fallback
    return torch.device("cuda:0")


def announce(*parts):
    """Name the case before any GPU work, so a failing run says what it was doing."""
    print("CASE", *parts, file=sys.stderr, flush=True)


def to_dev(ts, dev):
    return tuple(t.to(dev) for t in ts)


def host_workers():
    """Worker threads for oracle work on the host: the cores this process may
    run on, at most 16 (a GPU machine's CPU share per GPU)."""
    import os
    return max(1, min(16, len(os.sched_getaffinity(0))))


def par_map(fn, items):
    """[fn(x) for x in items] on host_workers() threads, one BLAS thread each
    (numpy releases the interpreter lock inside its array loops)."""
    import concurrent.futures

    from threadpoolctl import threadpool_limits
    items = list(items)
    with threadpool_limits(limits=1, user_api="blas"):
        with concurrent.futures.ThreadPoolExecutor(max_workers=host_workers()) as ex:
            return list(ex.map(fn, items))
