"""Backward parity: dQ, dK, dV from the HIP path against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_51_amd import workloads as W
from gates import GRAD_REL, check, to_np
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


def test_bwd_workload_c5():
    """The fwd+bwd workload at full size: whole heads against the oracle, plus invariants."""
    dev = device()
    w = W.WORKLOADS["c5"]
    announce("bwd workload c5")
    q, k, v, do = W.make_inputs(w)
    o, lse, dq, dk, dv = _fwd_bwd(*to_dev((q, k, v, do), dev), w.scale, w.causal)
    heads = [(0, 0), (1, 15), (1, 6)]
    ref = oracle.attention_backward(q, k, v, do, w.scale, w.causal, heads=heads)
    for (b, h) in heads:
        _check_grads((dq[b, h].cpu(), dk[b, h].cpu(), dv[b, h].cpu()), ref[(b, h)], w.dtype, f"c5 head {b},{h}")
    # invariants over every head: sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i
    dk64, dv64, do64 = (x.double() for x in (dk, dv, do.to(dev)))
    sk = dk64.sum(dim=2).abs().max().item()
    sv = (dv64.sum(dim=2) - do64.sum(dim=2)).abs().max().item()
    scale_k = dk64.abs().sum(dim=2).max().item()
    scale_v = dv64.abs().sum(dim=2).max().item()
    assert sk <= 1e-2 * scale_k, f"sum_j dK_j not ~0: {sk:.3e} vs {scale_k:.3e}"
    assert sv <= 1e-2 * scale_v, f"sum_j dV_j != sum_i dO_i: {sv:.3e} vs {scale_v:.3e}"


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
    """A negative scale (same magnitude as 1/sqrt(64)) flips every score's sign.

    At larger |scale| the gradients grow and the bf16 rounding of dS before the
    dK/dQ products dominates the absolute error (a CPU simulation of that
    rounding alone reaches 2.0e-2 at scale -0.2); the sign handling is what is
    checked here.
    """
    dev = device()
    w = W.shape_case(1, 2, 300, 64, "bf16", True, seed=43)
    announce("bwd negative scale")
    q, k, v, do = W.make_inputs(w)
    _, _, dq, dk, dv = _fwd_bwd(*to_dev((q, k, v, do), dev), -0.125, True)
    ref = oracle.attention_backward(q, k, v, do, np.float32(-0.125), True)
    _check_grads((dq, dk, dv), ref, "bf16", "scale=-0.125")
