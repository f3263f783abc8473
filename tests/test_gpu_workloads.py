"""The five workloads at full size, every output element against the oracle.

The method's claim is exactness over the whole output ("How Flash Attention
Works: Tiling, Softmax, GPU I/O", section "How Flash Attention Works: The
Exact-Attention Idea"; "attn-flash-equivalence", its summary: the same output
as naive attention up to the order of floating-point reductions).  Each test
launches the workload exactly as bench.py does (one call over all heads) and
compares every row of O and LSE (and of dQ, dK, dV for the fwd+bwd workload)
with the fp64 oracle, which runs a row panel or a head per host thread.  A
failure names the head and 128-row block of the worst element.
"""
import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_51_amd import workloads as W
from gates import GRAD_REL, check_blocks, check_lse_blocks
from gpu_util import announce, device, par_map, to_dev

pytestmark = pytest.mark.gpu

PANEL = 1024


def _oracle_forward(q, k, v, w):
    """The oracle's O and LSE for every head, a row panel per task."""
    tasks = [(b, h, r0) for b in range(w.B) for h in range(w.H) for r0 in range(0, w.N, PANEL)]
    res = par_map(lambda t: oracle.attention_forward_panel(q, k, v, w.scale, w.causal, t[0], t[1], t[2],
                                                           min(w.N, t[2] + PANEL)), tasks)
    o = np.empty((w.B, w.H, w.N, w.d))
    lse = np.empty((w.B, w.H, w.N))
    for (b, h, r0), (po, pl) in zip(tasks, res):
        o[b, h, r0:r0 + len(pl)] = po
        lse[b, h, r0:r0 + len(pl)] = pl
    return o, lse


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_fwd_workload_whole(name):
    import exact_io_aware_51_amd as fa
    dev = device()
    w = W.WORKLOADS[name]
    announce("fwd workload (whole output)", name)
    q, k, v = W.make_inputs(w, with_grad=False)
    o, lse = fa.forward(*to_dev((q, k, v), dev), scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    ro, rl = _oracle_forward(q, k, v, w)
    check_blocks(o, ro, w.dtype, f"O {name}")
    check_lse_blocks(lse, rl, w.dtype, f"LSE {name}")


def test_fwd_bwd_workload_c5_whole():
    """Workload c5: O, LSE, dQ, dK and dV of all 32 heads, plus the gradient identities."""
    import exact_io_aware_51_amd as fa
    dev = device()
    w = W.WORKLOADS["c5"]
    announce("fwd+bwd workload (whole output) c5")
    q, k, v, do = W.make_inputs(w)
    qd, kd, vd, dod = to_dev((q, k, v, do), dev)
    o, lse = fa.forward(qd, kd, vd, scale=w.scale, causal=w.causal)
    dq, dk, dv = fa.backward(qd, kd, vd, o, lse, dod, scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    ref = par_map(lambda bh: oracle.attention_backward(q, k, v, do, w.scale, w.causal, heads=[bh])[bh], heads)
    rq, rk, rv = (np.empty((w.B, w.H, w.N, w.d)) for _ in range(3))
    for (b, h), (a, bb, cc) in zip(heads, ref):
        rq[b, h], rk[b, h], rv[b, h] = a, bb, cc
    ro, rl = _oracle_forward(q, k, v, w)
    check_blocks(o.cpu(), ro, w.dtype, "O c5")
    check_lse_blocks(lse.cpu(), rl, w.dtype, "LSE c5")
    for nm, g, r in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        check_blocks(g.cpu(), r, w.dtype, f"{nm} c5", rel_gate=GRAD_REL[w.dtype])
    # identities of the definition, on the device's own results: every dS row
    # sums to zero, so sum_j dK_j = 0; sum_j dV_j = sum_j P^T dO = sum_i dO_i
    dk64, dv64, do64 = (x.double() for x in (dk, dv, dod))
    sk = dk64.sum(dim=2).abs().max().item()
    sv = (dv64.sum(dim=2) - do64.sum(dim=2)).abs().max().item()
    assert sk <= 1e-2 * dk64.abs().sum(dim=2).max().item(), f"sum_j dK_j not ~0: {sk:.3e}"
    assert sv <= 1e-2 * dv64.abs().sum(dim=2).max().item(), f"sum_j dV_j != sum_i dO_i: {sv:.3e}"
