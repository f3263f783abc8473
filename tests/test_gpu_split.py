"""GPU parity for the split-key forward (fa_fwd_kv_split).

Each key range writes an fp32 partial output and LSE, and a merge pass combines
them with the online-softmax rescale, so the result is the attention of
oracle.attention_forward_kv up to rounding order: the same 16-bit gates apply.
Readings under test are those of fa_fwd_kv (bottom-right causal alignment,
padding rows and rows that see no key give O = 0 and LSE = -inf).
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

DTYPES = ["f16", "bf16"]

# (B, H, Nq, Nk, d, seqlens_q, seqlens_k, splits)
CASES = [
    (2, 4, 1, 4096, 128, None, None, 16),             # decoding: one query against a key cache
    (1, 2, 1, 1000, 64, None, None, 3),               # ragged last tile, uneven ranges
    (3, 2, 4, 3001, 128, None, [3001, 640, 0], 7),    # lengths ending inside and before split ranges, an empty cache
    (1, 2, 77, 2048, 64, [50], [1500], 5),            # a prefill chunk: several queries, padded rows
    (1, 1, 200, 200, 128, None, None, 16),            # more splits than key tiles: empty ranges
    (2, 2, 129, 700, 64, None, None, 2),              # two query blocks per head
]
IDS = [f"B{c[0]}H{c[1]}q{c[2]}k{c[3]}d{c[4]}s{c[7]}{'-ragged' if c[6] or c[5] else ''}" for c in CASES]


def _lens(x, dev):
    return None if x is None else torch.tensor(x, dtype=torch.int32, device=dev)


def _check_fwd(o, lse, ro, rl, dtype, what):
    rl = np.asarray(rl)
    empty = np.isinf(rl)
    lse_np = to_np(lse)
    assert np.array_equal(np.isinf(lse_np) & (lse_np < 0), empty), f"{what}: rows with LSE = -inf differ"
    assert np.all(to_np(o)[empty] == 0.0), f"{what}: padding / empty rows are not exactly 0"
    check(o, ro, dtype, f"{what} O")
    if (~empty).any():
        check_lse(lse_np[~empty], rl[~empty], dtype, f"{what} LSE")


@pytest.mark.parametrize("case", CASES, ids=IDS)
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_split_matches_oracle(dtype, causal, case):
    dev = device()
    B, H, Nq, Nk, d, lq, lk, splits = case
    seed = 41000 + 17 * Nq + Nk + d
    announce("fwd_kv_split", dtype, causal, case, seed)
    q, k, v = W.kv_inputs(B, H, Nq, Nk, d, dtype, seed, with_grad=False)
    scale = 1.0 / float(np.sqrt(d))
    o, lse = fa.forward_kv_split(*to_dev((q, k, v), dev), seqlens_q=_lens(lq, dev), seqlens_k=_lens(lk, dev),
                                 scale=scale, causal=causal, num_splits=splits)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_forward_kv(q, k, v, scale, causal, lq, lk)
    _check_fwd(o, lse, ro, rl, dtype, f"split {dtype} causal={causal} {case}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_split_agrees_with_unsplit(dtype):
    """Every split count gives the unsplit result up to rounding order; one split is the unsplit kernel itself."""
    dev = device()
    announce("split vs unsplit", dtype)
    q, k, v = to_dev(W.kv_inputs(2, 8, 3, 8192, 128, dtype, 41900, with_grad=False), dev)
    o1, l1 = fa.forward_kv(q, k, v, causal=True)
    for splits in (1, 2, 5, 32, 128, 256):
        o2, l2 = fa.forward_kv_split(q, k, v, causal=True, num_splits=splits)
        torch.cuda.synchronize()
        if splits == 1:
            assert torch.equal(o1, o2) and torch.equal(l1, l2)
        assert float((l1 - l2).abs().max()) <= 2e-5, f"{splits} splits: LSE"
        assert float((o1.float() - o2.float()).abs().max()) <= 8e-3, f"{splits} splits: O"


def test_backward_accepts_split_forward():
    """fa_bwd_kv on the split forward's O and LSE gives the oracle's gradients."""
    dev = device()
    announce("bwd from split forward")
    B, H, Nq, Nk, d = 1, 2, 64, 2000, 128
    q, k, v, do = W.kv_inputs(B, H, Nq, Nk, d, "bf16", 41950)
    qd, kd, vd, dod = to_dev((q, k, v, do), dev)
    o, lse = fa.forward_kv_split(qd, kd, vd, causal=True, num_splits=6)
    dq, dk, dv = fa.backward_kv(qd, kd, vd, o, lse, dod, causal=True)
    torch.cuda.synchronize()
    rdq, rdk, rdv = oracle.attention_backward_kv(q, k, v, do, 1.0 / np.sqrt(d), True)
    for x, r, n in ((dq, rdq, "dQ"), (dk, rdk, "dK"), (dv, rdv, "dV")):
        check(x, r, "bf16", f"bwd after split forward {n}", rel_gate=GRAD_REL["bf16"])


def test_split_hint_decode_long_cache():
    """The suggested split count on a 32768-key decode, checked on every row against the oracle."""
    dev = device()
    announce("split hint decode")
    B, H, Nq, Nk, d = 1, 8, 1, 32768, 128
    q, k, v = W.kv_inputs(B, H, Nq, Nk, d, "bf16", 41990, with_grad=False)
    o, lse = fa.forward_kv_split(*to_dev((q, k, v), dev), causal=True)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_forward_kv(q, k, v, 1.0 / np.sqrt(d), True)
    _check_fwd(o, lse, ro, rl, "bf16", "split hint decode")
