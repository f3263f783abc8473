"""Backward parity: dQ, dK, dV from the HIP path against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_51_amd import workloads as W
from gates import GRAD_REL, bwd_rounding_bound, check, to_np
from gpu_util import announce, device, to_dev

pytestmark = pytest.mark.gpu


def _fwd_bwd(q, k, v, do, scale, causal):
    import exact_io_aware_51_amd as fa
    o, lse = fa.forward(q, k, v, scale=scale, causal=causal)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def _check_grads(got, ref, dtype, tag):
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        check(g, r, dtype, f"{name} {tag}", rel_gate=GRAD_REL[dtype])


SHAPES = [(1, 2, n, d) for n in (1, 7, 63, 65, 129, 257, 1000) for d in (64, 128)]
SHAPES += [(2, 3, 191, 64)]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bwd_small_shapes(shape, causal, dtype):
    dev = device()
    B, H, N, d = shape
    w = W.shape_case(B, H, N, d, dtype, causal, seed=31 + N + d)
    announce("bwd", w.name)
    q, k, v, do = W.make_inputs(w)
    _, _, dq, dk, dv = _fwd_bwd(*to_dev((q, k, v, do), dev), w.scale, causal)
    ref = oracle.attention_backward(q, k, v, do, w.scale, causal)
    _check_grads((dq, dk, dv), ref, dtype, w.name)


def test_bwd_zero_dout_and_determinism():
    dev = device()
    w = W.shape_case(2, 2, 777, 128, "bf16", True, seed=41)
    announce("bwd determinism", w.name)
    q, k, v, do = to_dev(W.make_inputs(w), dev)
    a = _fwd_bwd(q, k, v, do, w.scale, True)
    b = _fwd_bwd(q, k, v, do, w.scale, True)
    for x, y in zip(a, b):
        assert torch.equal(x, y), "backward must be bit-reproducible"
    z = _fwd_bwd(q, k, v, torch.zeros_like(do), w.scale, True)
    for g in z[2:]:
        assert torch.count_nonzero(g).item() == 0, "dO = 0 must give zero gradients"


def test_bwd_negative_scale():
    """A negative scale (same magnitude as 1/sqrt(64)) flips every score's sign."""
    dev = device()
    w = W.shape_case(1, 2, 300, 64, "bf16", True, seed=43)
    announce("bwd negative scale")
    q, k, v, do = W.make_inputs(w)
    _, _, dq, dk, dv = _fwd_bwd(*to_dev((q, k, v, do), dev), -0.125, True)
    ref = oracle.attention_backward(q, k, v, do, np.float32(-0.125), True)
    _check_grads((dq, dk, dv), ref, "bf16", "scale=-0.125")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("scale", [0.2, 0.25, 0.5, -0.5])
def test_bwd_large_scale_within_rounding_model(scale, dtype):
    """Large |scale|: the error is the rounding the recompute scheme performs.

    P and dS are rounded to the I/O type before their products, and D comes
    from the rounded O.  With u the unit roundoff (2^-8 for bf16), the dS
    rounding alone moves dK_jc by up to u |scale| sum_i |dS_ij| |q_ic|.  That
    grows with the gradients, so past |scale| ~ 0.2 the absolute part of the
    stated elementwise gate (2e-2) no longer holds for elements that cancel
    to near zero.  What must hold at any scale: every element within the
    first-order bound of those roundings (gates.bwd_rounding_bound, computed
    from the oracle's exact P and dS), and the relative Frobenius gate.
    """
    dev = device()
    w = W.shape_case(1, 2, 400, 128, dtype, True, seed=47)
    announce("bwd large scale", scale, dtype)
    q, k, v, do = W.make_inputs(w)
    sc = np.float32(scale)
    _, _, dq, dk, dv = _fwd_bwd(*to_dev((q, k, v, do), dev), float(sc), True)
    ref = oracle.attention_backward(q, k, v, do, sc, True)
    ro, _ = oracle.attention_forward(q, k, v, sc, True)
    got = [to_np(g) for g in (dq, dk, dv)]
    for h in range(w.H):
        terms = oracle.attention_backward_terms(q, k, v, do, sc, True, 0, h)
        hq, hk, hv, hdo = (to_np(x)[0, h] for x in (q, k, v, do))
        bounds = bwd_rounding_bound(hq, hk, hv, hdo, ro[0, h], terms, float(sc), dtype)
        for name, g, r, bd in zip(("dQ", "dK", "dV"), got, ref, bounds):
            err = np.abs(g[0, h] - r[0, h])
            worst = np.unravel_index(int(np.argmax(err - bd)), err.shape)
            assert err[worst] <= bd[worst], (f"{name} head {h}: error {err[worst]:.3e} above the rounding bound "
                                             f"{bd[worst]:.3e} at {worst}")
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        rel = np.linalg.norm(g - r) / np.linalg.norm(r)
        assert rel <= GRAD_REL[dtype], f"{name}: relative Frobenius error {rel:.3e} > {GRAD_REL[dtype]:.0e}"
