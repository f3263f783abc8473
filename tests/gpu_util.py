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
