"""GPU parity for attention dropout (fa_fwd_dropout, fa_bwd_dropout).

The HIP path is compared with oracle.attention_forward_dropout /
attention_backward_dropout on the same seeded inputs.  Reading under test (the
pages put dropout inside the fused kernel and fix no generator): the weight of
query i and key j in slice b * H + h is kept iff word (j & 3) of
Philox4x32-10(counter (j >> 2, i, b * H + h, offset), key (seed lo, seed hi))
is >= floor(p * 2^32); kept weights are scaled by 1 / (1 - p); the LSE is that
of the undropped softmax.  The keep decision is integer work, so the mask
itself is compared bit for bit (value matrix = identity makes O = P o Z).
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
SHAPES = [(1, 2, 300, 64), (2, 1, 512, 128), (1, 1, 1000, 128), (2, 2, 129, 64)]
SIDS = [f"B{b}H{h}N{n}d{d}" for b, h, n, d in SHAPES]
SEED = 0x9E3779B97F4A7C15  # exercises both 32-bit halves of the key


def _p32(p):
    """The probability as the library receives it (a C float)."""
    return float(np.float32(p))


@pytest.mark.parametrize("p", [0.1, 0.5])
@pytest.mark.parametrize("shape", SHAPES, ids=SIDS)
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_fwd_dropout_matches_oracle(dtype, causal, shape, p):
    dev = device()
    B, H, N, d = shape
    seed = 21000 + N + d
    announce("fwd_dropout", dtype, causal, shape, p, seed)
    q, k, v = W.kv_inputs(B, H, N, N, d, dtype, seed, with_grad=False)
    scale = 1.0 / float(np.sqrt(d))
    o, lse = fa.forward_dropout(*to_dev((q, k, v), dev), p, SEED, offset=5, scale=scale, causal=causal)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_forward_dropout(q, k, v, scale, causal, _p32(p), SEED, 5)
    tag = f"fwd_dropout {dtype} causal={causal} {shape} p={p}"
    check(o, ro, dtype, f"{tag} O")
    check_lse(lse, rl, dtype, f"{tag} LSE")


@pytest.mark.parametrize("p", [0.1, 0.5])
@pytest.mark.parametrize("shape", SHAPES[:3], ids=SIDS[:3])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_bwd_dropout_matches_oracle(dtype, causal, shape, p):
    dev = device()
    B, H, N, d = shape
    seed = 22000 + N + d
    announce("bwd_dropout", dtype, causal, shape, p, seed)
    q, k, v, do = W.kv_inputs(B, H, N, N, d, dtype, seed)
    scale = 1.0 / float(np.sqrt(d))
    qd, kd, vd, dod = to_dev((q, k, v, do), dev)
    o, lse = fa.forward_dropout(qd, kd, vd, p, SEED, offset=9, scale=scale, causal=causal)
    dq, dk, dv = fa.backward_dropout(qd, kd, vd, o, lse, dod, p, SEED, offset=9, scale=scale, causal=causal)
    torch.cuda.synchronize()
    rdq, rdk, rdv = oracle.attention_backward_dropout(q, k, v, do, scale, causal, _p32(p), SEED, 9)
    tag = f"bwd_dropout {dtype} causal={causal} {shape} p={p}"
    gate = GRAD_REL[dtype]
    check(dq, rdq, dtype, f"{tag} dQ", rel_gate=gate)
    check(dk, rdk, dtype, f"{tag} dK", rel_gate=gate)
    check(dv, rdv, dtype, f"{tag} dV", rel_gate=gate)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("d", [64, 128])
def test_keep_mask_is_bit_exact(dtype, d):
    """With v = identity (N = d) the output row i is P_i o Z_i: its zeros are exactly the dropped keys."""
    dev = device()
    announce("dropout mask", dtype, d)
    B, H, N = 2, 3, d
    q, k, _ = W.kv_inputs(B, H, N, N, d, dtype, 23000 + d, with_grad=False)
    q, k = q * 0.25, k * 0.25                     # scores near 0: every weight near 1/N, far from underflow
    v = torch.eye(N, dtype=q.dtype).expand(B, H, N, N).contiguous()
    for causal in (False, True):
        o, _ = fa.forward_dropout(*to_dev((q, k, v), dev), 0.3, 12345, offset=77, causal=causal)
        torch.cuda.synchronize()
        got = to_np(o) != 0.0
        for b in range(B):
            for h in range(H):
                keep = oracle.dropout_keep(N, N, b * H + h, _p32(0.3), 12345, 77)
                if causal:
                    keep = keep & np.tril(np.ones((N, N), dtype=bool))
                assert np.array_equal(got[b, h], keep), f"mask differs at b={b} h={h} causal={causal}"


@pytest.mark.parametrize("dtype", DTYPES)
def test_p_zero_is_the_dense_path(dtype):
    dev = device()
    announce("dropout p=0", dtype)
    q, k, v, do = to_dev(W.kv_inputs(1, 2, 700, 700, 128, dtype, 23101), dev)
    for causal in (False, True):
        o1, l1 = fa.forward(q, k, v, causal=causal)
        o2, l2 = fa.forward_dropout(q, k, v, 0.0, 99, causal=causal)
        g1 = fa.backward(q, k, v, o1, l1, do, causal=causal)
        g2 = fa.backward_dropout(q, k, v, o2, l2, do, 0.0, 99, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        for a, b in zip(g1, g2):
            assert torch.equal(a, b)


def test_seed_and_offset_select_the_mask():
    """Same (seed, offset): identical bits; another offset or seed: another mask; LSE never changes."""
    dev = device()
    announce("dropout seed/offset")
    q, k, v = to_dev(W.kv_inputs(1, 2, 640, 640, 64, "bf16", 23102, with_grad=False), dev)
    o1, l1 = fa.forward_dropout(q, k, v, 0.2, 1, offset=0)
    o2, l2 = fa.forward_dropout(q, k, v, 0.2, 1, offset=0)
    o3, l3 = fa.forward_dropout(q, k, v, 0.2, 1, offset=1)
    o4, l4 = fa.forward_dropout(q, k, v, 0.2, 1 << 32, offset=0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert not torch.equal(o1, o3) and not torch.equal(o1, o4) and not torch.equal(o3, o4)
    assert torch.equal(l1, l3) and torch.equal(l1, l4)


def test_dropout_4096():
    """Causal bf16 at N = 4096, d = 128, p = 0.1: forward and backward against the oracle."""
    dev = device()
    announce("dropout N=4096")
    q, k, v, do = W.kv_inputs(1, 1, 4096, 4096, 128, "bf16", 23103)
    qd, kd, vd, dod = to_dev((q, k, v, do), dev)
    sc = 0.08838835
    o, lse = fa.forward_dropout(qd, kd, vd, 0.1, SEED, offset=3, scale=sc, causal=True)
    dq, dk, dv = fa.backward_dropout(qd, kd, vd, o, lse, dod, 0.1, SEED, offset=3, scale=sc, causal=True)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_forward_dropout(q, k, v, sc, True, _p32(0.1), SEED, 3)
    check(o, ro, "bf16", "dropout 4096 O")
    check_lse(lse, rl, "bf16", "dropout 4096 LSE")
    rdq, rdk, rdv = oracle.attention_backward_dropout(q, k, v, do, sc, True, _p32(0.1), SEED, 3)
    for x, r, n in ((dq, rdq, "dQ"), (dk, rdk, "dK"), (dv, rdv, "dV")):
        check(x, r, "bf16", f"dropout 4096 {n}", rel_gate=GRAD_REL["bf16"])
