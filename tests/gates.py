"""Parity gates between the HIP path and the fp64 oracle.

Stated gates: max abs error 1e-4 for fp32 I/O; |x - r| <= 2e-2 + 1e-2 |r|
elementwise for bf16/fp16 outputs and gradients.  Because attention outputs are
small at long sequence lengths (|O| ~ sigma_V * sqrt(e^{sigma_s^2} / n)), an
all-zero output would pass the 16-bit elementwise gate, so two supplemental
gates are always applied as well: the relative Frobenius error ||x - r|| / ||r||
and a max-abs bound on the log-sum-exp.
"""
from __future__ import annotations

import numpy as np

FWD_REL = {"f32": 1e-5, "f16": 3e-3, "bf16": 1e-2}
GRAD_REL = {"f32": 1e-5, "f16": 1e-2, "bf16": 2e-2}
LSE_ABS = {"f32": 1e-5, "f16": 1e-3, "bf16": 1e-3}


def to_np(x):
    import torch
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def check(x, ref, dtype, what, rel_gate=None):
    """Assert the stated gate and the relative Frobenius gate; return the error stats."""
    x, ref = to_np(x), to_np(ref)
    assert x.shape == ref.shape, f"{what}: shape {x.shape} vs {ref.shape}"
    assert np.all(np.isfinite(x)), f"{what}: non-finite values"
    diff = np.abs(x - ref)
    max_abs = float(diff.max()) if diff.size else 0.0
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(x - ref) / nref) if nref > 0 else float(np.linalg.norm(x - ref))
    if dtype == "f32":
        assert max_abs <= 1e-4, f"{what}: max abs err {max_abs:.3e} > 1e-4"
    else:
        bound = 2e-2 + 1e-2 * np.abs(ref)
        worst = float((diff - bound).max()) if diff.size else -1.0
        assert worst <= 0.0, f"{what}: elementwise gate exceeded by {worst:.3e} (max abs err {max_abs:.3e})"
    gate = rel_gate if rel_gate is not None else FWD_REL[dtype]
    assert rel <= gate, f"{what}: relative Frobenius error {rel:.3e} > {gate:.1e}"
    return {"max_abs": max_abs, "rel_fro": rel}


def check_lse(x, ref, dtype, what):
    x, ref = to_np(x), to_np(ref)
    err = float(np.max(np.abs(x - ref))) if x.size else 0.0
    assert np.all(np.isfinite(x)), f"{what}: non-finite LSE"
    assert err <= LSE_ABS[dtype], f"{what}: LSE max abs err {err:.3e} > {LSE_ABS[dtype]:.0e}"
    return err
