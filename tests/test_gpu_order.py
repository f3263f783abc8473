"""The order in which workgroups take (head, block) pairs changes no result.

Causal grids are issued by block rank within groups of heads; the group size
depends on the head count, the blocks per head and the kernel.  Head counts
that are not a multiple of the group size leave a partial last group.  Every
block's arithmetic is independent of when it runs (no atomics), so all heads
in one launch must equal the same heads launched one at a time, bit for bit,
for the forward and each backward stage.  The shapes below give partial
groups in the forward and dQ (12 heads of 64 blocks, groups of 8), in the
d = 64 dK/dV and dQ kernels (13 heads of 64 blocks, groups of 8), in the
d = 128 dK/dV kernel, whose groups are four times wider (20 heads of 64
128-key blocks, groups of 16), and head counts that are no multiple of 8 in
one group (10 heads at N = 2048).
"""
import pytest
import torch

import exact_io_aware_51_amd as fa
from exact_io_aware_51_amd import workloads as W
from gpu_util import announce, device, to_dev

pytestmark = pytest.mark.gpu

CASES = [(3, 4, 8192, 128, "bf16"), (1, 13, 8192, 64, "f16"), (2, 5, 2048, 128, "bf16"), (1, 20, 8192, 128, "bf16")]


@pytest.mark.parametrize("B,H,N,d,dtype", CASES, ids=lambda x: str(x))
def test_causal_grid_equals_per_head_launches(B, H, N, d, dtype):
    dev = device()
    announce("grid order", B, H, N, d, dtype)
    w = W.shape_case(B, H, N, d, dtype, True, seed=61000 + H)
    q, k, v, do = to_dev(W.make_inputs(w), dev)
    o, lse = fa.forward(q, k, v, scale=w.scale, causal=True)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            sl = (slice(b, b + 1), slice(h, h + 1))
            q1, k1, v1, do1 = (t[sl].contiguous() for t in (q, k, v, do))
            o1, lse1 = fa.forward(q1, k1, v1, scale=w.scale, causal=True)
            dq1, dk1, dv1 = fa.backward(q1, k1, v1, o1, lse1, do1, scale=w.scale, causal=True)
            torch.cuda.synchronize()
            for name, full, one in (("O", o, o1), ("LSE", lse, lse1), ("dQ", dq, dq1), ("dK", dk, dk1),
                                    ("dV", dv, dv1)):
                assert torch.equal(full[sl], one), f"{name} of head ({b}, {h}) differs from its own launch"
