"""GPU parity for block-sparse attention (fa_fwd_sparse, fa_bwd_sparse).

The HIP path is compared with oracle.attention_forward_sparse /
attention_backward_sparse on the same seeded inputs and masks.  Reading under
test (the pages name the extension, not a format): a uint8 mask over
(128-query block, 128-key block) pairs removes those scores on top of the
causal mask; rows that see no key output O = 0 and LSE = -inf.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_51_amd as fa
import oracle
from exact_io_aware_51_amd import workloads as W
from gates import GRAD_REL, check, check_lse, to_np
from gpu_util import announce, device, to_dev

pytestmark = pytest.mark.gpu

DTYPES = ["f32", "f16", "bf16"]
SHAPES = [(1, 2, 300, 64), (2, 1, 512, 128), (1, 2, 1000, 128), (1, 1, 1000, 64)]
SIDS = [f"B{b}H{h}N{n}d{d}" for b, h, n, d in SHAPES]
MASKS = ["random", "empty-row", "diagonal"]


def _mask(kind, B, H, N, seed):
    m = W.block_mask(B, H, N, 0.5, seed)
    if kind == "empty-row":
        m[:, :, min(1, m.shape[2] - 1), :] = 0   # a query block that sees nothing
        m[0, 0, 0, 0] = 1
    elif kind == "diagonal":
        m = torch.eye(m.shape[2], dtype=torch.uint8).expand(B, H, -1, -1).contiguous()
    return m


def _check_fwd(o, lse, ro, rl, dtype, what):
    rl = np.asarray(rl)
    empty = np.isinf(rl)
    lse_np = to_np(lse)
    assert np.array_equal(np.isinf(lse_np) & (lse_np < 0), empty), f"{what}: rows with LSE = -inf differ"
    assert np.all(to_np(o)[empty] == 0.0), f"{what}: rows that see no key are not exactly 0"
    check(o, ro, dtype, f"{what} O")
    if (~empty).any():
        check_lse(lse_np[~empty], rl[~empty], dtype, f"{what} LSE")


@pytest.mark.parametrize("kind", MASKS)
@pytest.mark.parametrize("shape", SHAPES, ids=SIDS)
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_fwd_sparse_matches_oracle(dtype, causal, shape, kind):
    dev = device()
    B, H, N, d = shape
    seed = 11000 + N + d
    announce("fwd_sparse", dtype, causal, shape, kind, seed)
    q, k, v = W.kv_inputs(B, H, N, N, d, dtype, seed, with_grad=False)
    m = _mask(kind, B, H, N, seed + 1)
    scale = 1.0 / float(np.sqrt(d))
    o, lse = fa.forward_sparse(*to_dev((q, k, v), dev), m.to(dev), scale=scale, causal=causal)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_forward_sparse(q, k, v, scale, causal, m.numpy())
    _check_fwd(o, lse, ro, rl, dtype, f"fwd_sparse {dtype} causal={causal} {shape} {kind}")


@pytest.mark.parametrize("kind", MASKS)
@pytest.mark.parametrize("shape", SHAPES[:3], ids=SIDS[:3])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_bwd_sparse_matches_oracle(dtype, causal, shape, kind):
    dev = device()
    B, H, N, d = shape
    seed = 12000 + N + d
    announce("bwd_sparse", dtype, causal, shape, kind, seed)
    q, k, v, do = W.kv_inputs(B, H, N, N, d, dtype, seed)
    m = _mask(kind, B, H, N, seed + 1)
    scale = 1.0 / float(np.sqrt(d))
    qd, kd, vd, dod = to_dev((q, k, v, do), dev)
    md = m.to(dev)
    o, lse = fa.forward_sparse(qd, kd, vd, md, scale=scale, causal=causal)
    dq, dk, dv = fa.backward_sparse(qd, kd, vd, o, lse, dod, md, scale=scale, causal=causal)
    torch.cuda.synchronize()
    rdq, rdk, rdv = oracle.attention_backward_sparse(q, k, v, do, scale, causal, m.numpy())
    tag = f"bwd_sparse {dtype} causal={causal} {shape} {kind}"
    gate = GRAD_REL[dtype]
    check(dq, rdq, dtype, f"{tag} dQ", rel_gate=gate)
    check(dk, rdk, dtype, f"{tag} dK", rel_gate=gate)
    check(dv, rdv, dtype, f"{tag} dV", rel_gate=gate)


@pytest.mark.parametrize("dtype", DTYPES)
def test_all_ones_mask_is_the_dense_path(dtype):
    """Every block kept: the same arithmetic as fa_fwd / fa_bwd, bit for bit,
    except dK/dV at d = 128 with 16-bit I/O, where the dense path runs a kernel
    of its own (K and V resident in LDS, 32 keys per wave) and the block-sparse
    path the 16-key kernel, which add the same products in another order:
    there the two may differ by one rounding of the output type plus fp32
    reordering noise."""
    dev = device()
    announce("sparse all-ones", dtype)
    q, k, v, do = to_dev(W.kv_inputs(2, 2, 700, 700, 128, dtype, 13001), dev)
    ones = torch.ones((2, 2, 6, 6), dtype=torch.uint8, device=dev)
    for causal in (False, True):
        o1, l1 = fa.forward(q, k, v, causal=causal)
        o2, l2 = fa.forward_sparse(q, k, v, ones, causal=causal)
        g1 = fa.backward(q, k, v, o1, l1, do, causal=causal)
        g2 = fa.backward_sparse(q, k, v, o2, l2, do, ones, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        assert torch.equal(g1[0], g2[0]), "dQ"
        for a, b, what in zip(g1[1:], g2[1:], ("dK", "dV")):
            if dtype == "f32":
                assert torch.equal(a, b), what
            else:
                ulp = 2.0 ** -7 if dtype == "bf16" else 2.0 ** -10   # one step of the output type, relative
                af, bf = a.float(), b.float()
                assert torch.all((af - bf).abs() <= ulp * bf.abs() + 1e-4 * bf.abs().max()), what


def test_all_zero_mask():
    dev = device()
    announce("sparse all-zero")
    q, k, v, do = to_dev(W.kv_inputs(1, 2, 333, 333, 64, "bf16", 13002), dev)
    zero = torch.zeros((1, 2, 3, 3), dtype=torch.uint8, device=dev)
    o, lse = fa.forward_sparse(q, k, v, zero, causal=False)
    dq, dk, dv = fa.backward_sparse(q, k, v, o, lse, do, zero)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    assert torch.all(dq == 0) and torch.all(dk == 0) and torch.all(dv == 0)


def test_sparse_4096():
    """A causal half-density mask at N = 4096 (bf16, d = 128), forward and backward."""
    dev = device()
    announce("sparse N=4096")
    q, k, v, do = W.kv_inputs(1, 2, 4096, 4096, 128, "bf16", 13003)
    m = W.block_mask(1, 2, 4096, 0.5, 13004)
    qd, kd, vd, dod = to_dev((q, k, v, do), dev)
    md = m.to(dev)
    o, lse = fa.forward_sparse(qd, kd, vd, md, scale=0.08838835, causal=True)
    dq, dk, dv = fa.backward_sparse(qd, kd, vd, o, lse, dod, md, scale=0.08838835, causal=True)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_forward_sparse(q, k, v, 0.08838835, True, m.numpy())
    _check_fwd(o, lse, ro, rl, "bf16", "sparse 4096")
    rdq, rdk, rdv = oracle.attention_backward_sparse(q, k, v, do, 0.08838835, True, m.numpy())
    for x, r, n in ((dq, rdq, "dQ"), (dk, rdk, "dK"), (dv, rdv, "dV")):
        check(x, r, "bf16", f"sparse 4096 {n}", rel_gate=GRAD_REL["bf16"])
