"""Seeded random shapes through the dense, padded-batch, block-sparse and
dropout entry points, forward and backward, against the oracle at the stated
gates.

The cases are drawn once from a fixed generator: batch and head counts 1-3,
sequence lengths 1-700 (so most end in a ragged tile), d in {64, 128}, every
I/O type, with and without the causal mask, random per-sequence lengths
(including empty sequences) for the padded batches, and random keep rates for
the block masks.  Key counts of the padded batches stay at 32 or more: with a
handful of keys against many queries the bf16 gradients leave the absolute part
of the elementwise gate through the rounding of dS, a case
test_gpu_kv.test_bwd_kv_few_keys_within_rounding_model holds to its own bound.
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


def _draw_cases(n=32):
    g = np.random.default_rng(20261203)
    cases = []
    for t in range(n):
        kind = ("dense", "kv", "sparse", "dropout")[t % 4]
        dtype = str(g.choice(["f32", "f16", "bf16"])) if kind != "dropout" else str(g.choice(["f16", "bf16"]))
        B, H = int(g.integers(1, 4)), int(g.integers(1, 4))
        Nq = int(g.integers(1, 701))
        Nk = int(g.integers(32, 701)) if kind == "kv" else Nq
        d = int(g.choice([64, 128]))
        causal = bool(g.integers(0, 2))
        extra = None
        if kind == "kv" and g.integers(0, 2):
            extra = ([int(g.integers(0, Nq + 1)) for _ in range(B)], [int(g.integers(32, Nk + 1)) for _ in range(B)])
        elif kind == "sparse":
            extra = float(g.uniform(0.2, 1.0))
        elif kind == "dropout":
            extra = float(g.choice([0.1, 0.3, 0.5]))
        cases.append((kind, dtype, B, H, Nq, Nk, d, causal, extra, 97000 + t))
    return cases


CASES = _draw_cases()
IDS = [f"{c[0]}-{c[1]}-B{c[2]}H{c[3]}q{c[4]}k{c[5]}d{c[6]}{'-causal' if c[7] else ''}" for c in CASES]


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_random_shape_matches_oracle(case):
    kind, dtype, B, H, Nq, Nk, d, causal, extra, seed = case
    dev = device()
    announce("random", *case)
    q, k, v, do = W.kv_inputs(B, H, Nq, Nk, d, dtype, seed)
    scale = 1.0 / float(np.sqrt(d))
    qd, kd, vd, dod = to_dev((q, k, v, do), dev)
    if kind == "dense":
        o, lse = fa.forward(qd, kd, vd, scale=scale, causal=causal)
        grads = fa.backward(qd, kd, vd, o, lse, dod, scale=scale, causal=causal)
        ro, rl = oracle.attention_forward(q, k, v, scale, causal)
        ref = oracle.attention_backward(q, k, v, do, scale, causal)
    elif kind == "kv":
        lq, lk = extra if extra is not None else (None, None)
        tq = None if lq is None else torch.tensor(lq, dtype=torch.int32, device=dev)
        tk = None if lk is None else torch.tensor(lk, dtype=torch.int32, device=dev)
        o, lse = fa.forward_kv(qd, kd, vd, seqlens_q=tq, seqlens_k=tk, scale=scale, causal=causal)
        grads = fa.backward_kv(qd, kd, vd, o, lse, dod, seqlens_q=tq, seqlens_k=tk, scale=scale, causal=causal)
        ro, rl = oracle.attention_forward_kv(q, k, v, scale, causal, lq, lk)
        ref = oracle.attention_backward_kv(q, k, v, do, scale, causal, lq, lk)
    elif kind == "sparse":
        m = W.block_mask(B, H, Nq, extra, seed + 1)
        md = m.to(dev)
        o, lse = fa.forward_sparse(qd, kd, vd, md, scale=scale, causal=causal)
        grads = fa.backward_sparse(qd, kd, vd, o, lse, dod, md, scale=scale, causal=causal)
        ro, rl = oracle.attention_forward_sparse(q, k, v, scale, causal, m.numpy())
        ref = oracle.attention_backward_sparse(q, k, v, do, scale, causal, m.numpy())
    else:
        p32 = float(np.float32(extra))
        o, lse = fa.forward_dropout(qd, kd, vd, extra, 777, offset=2, scale=scale, causal=causal)
        grads = fa.backward_dropout(qd, kd, vd, o, lse, dod, extra, 777, offset=2, scale=scale, causal=causal)
        ro, rl = oracle.attention_forward_dropout(q, k, v, scale, causal, p32, 777, 2)
        ref = oracle.attention_backward_dropout(q, k, v, do, scale, causal, p32, 777, 2)
    torch.cuda.synchronize()
    tag = "random " + " ".join(str(x) for x in case)
    rl = np.asarray(rl)
    empty = np.isinf(rl)
    lse_np = to_np(lse)
    assert np.array_equal(np.isinf(lse_np) & (lse_np < 0), empty), f"{tag}: rows with LSE = -inf differ"
    check(o, ro, dtype, f"{tag} O")
    if (~empty).any():
        check_lse(lse_np[~empty], rl[~empty], dtype, f"{tag} LSE")
    for name, g, r in zip(("dQ", "dK", "dV"), grads, ref):
        check(g, r, dtype, f"{tag} {name}", rel_gate=GRAD_REL[dtype])
