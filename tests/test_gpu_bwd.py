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


def _stage_call(fa, name, args):
    st = getattr(fa, name)(*args)
    assert st == fa.FA_OK, f"{name}: {fa.fa_status_string(st)}"


@pytest.mark.parametrize("dtype,causal,shape", [("bf16", True, (1, 2, 300, 128)), ("f16", False, (2, 1, 257, 64)),
                                                ("bf16", False, (1, 3, 1000, 128)), ("f32", True, (1, 2, 129, 64))],
                         ids=["bf16-causal-300x128", "f16-full-257x64", "bf16-full-1000x128", "f32-causal-129x64"])
def test_bwd_stage_entry_points(dtype, causal, shape):
    """fa_bwd is fa_bwd_dq_rowsum then fa_bwd_dkdv (bit for bit); the three-launch
    sequence fa_bwd_rowsum, fa_bwd_dkdv, fa_bwd_dq gives the same gradients up to
    D's summation order and passes the oracle's gates; both row sums match
    sum_c dO_ic O_ic of the stored O within fp32 rounding."""
    import exact_io_aware_51_amd as fa
    dev = device()
    B, H, N, d = shape
    w = W.shape_case(B, H, N, d, dtype, causal, seed=53 + N + d)
    announce("bwd stages", w.name)
    q, k, v, do = to_dev(W.make_inputs(w), dev)
    o, lse = fa.forward(q, k, v, scale=w.scale, causal=causal)
    ref_dq, ref_dk, ref_dv = fa.backward(q, k, v, o, lse, do, scale=w.scale, causal=causal)
    code = {"bf16": fa.FA_BF16, "f16": fa.FA_F16, "f32": fa.FA_F32}[dtype]
    wsb = fa.fa_bwd_workspace_bytes(B, H, N, d, code)
    stream = torch.cuda.current_stream().cuda_stream
    sd = (B, H, N, d, w.scale, int(causal), code, stream)
    p = lambda t: t.data_ptr()  # noqa: E731

    ws1 = torch.full((wsb,), 0xFF, dtype=torch.uint8, device=dev)  # garbage D: the stage must overwrite it
    dq1, dk1, dv1 = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    _stage_call(fa, "fa_bwd_dq_rowsum", (p(q), p(k), p(v), p(o), p(do), p(lse), p(ws1), wsb, p(dq1), *sd))
    _stage_call(fa, "fa_bwd_dkdv", (p(q), p(k), p(v), p(do), p(lse), p(ws1), wsb, p(dk1), p(dv1), *sd))

    ws2 = torch.empty((wsb,), dtype=torch.uint8, device=dev)
    dq2, dk2, dv2 = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    _stage_call(fa, "fa_bwd_rowsum", (p(o), p(do), p(ws2), wsb, B, H, N, d, code, stream))
    _stage_call(fa, "fa_bwd_dkdv", (p(q), p(k), p(v), p(do), p(lse), p(ws2), wsb, p(dk2), p(dv2), *sd))
    _stage_call(fa, "fa_bwd_dq", (p(q), p(k), p(v), p(do), p(lse), p(ws2), wsb, p(dq2), *sd))
    torch.cuda.synchronize()

    for a, b, what in zip((dq1, dk1, dv1), (ref_dq, ref_dk, ref_dv), ("dQ", "dK", "dV")):
        assert torch.equal(a, b), f"{what}: fa_bwd_dq_rowsum + fa_bwd_dkdv differ from fa_bwd"
    rows = B * H * N
    d1 = ws1[:rows * 4].view(torch.float32).double().cpu().numpy()
    d2 = ws2[:rows * 4].view(torch.float32).double().cpu().numpy()
    prod = (to_np(do) * to_np(o)).reshape(rows, d)
    exact, mag = prod.sum(axis=1), np.abs(prod).sum(axis=1)
    tol = d * 2.0 ** -24 * mag + 1e-30   # fp32 sums of d exact products, any order
    assert np.all(np.abs(d1 - exact) <= tol), "row sums from the dQ stage"
    assert np.all(np.abs(d2 - exact) <= tol), "row sums from fa_bwd_rowsum"
    ref = oracle.attention_backward(*(t.cpu() for t in (q, k, v, do)), w.scale, causal)
    for got, what in (((dq1, dk1, dv1), "two-stage"), ((dq2, dk2, dv2), "three-stage")):
        _check_grads(got, ref, dtype, f"{w.name} {what}")
