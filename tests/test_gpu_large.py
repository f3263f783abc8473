"""Maximum sizes: long sequences through every path, checked on sampled outputs.

At these sizes the oracle cannot form whole heads, so the forward is checked
row by row (oracle.attention_forward_rows, attention_forward_sparse_rows) and
the backward on sampled dQ rows (attention_backward_rows) plus two identities
that hold at any size because every softmax row sums to one:
sum_j dK_j = scale * sum_i (sum_j dS_ij) q_i = 0 and sum_j dV_j = sum_i dO_i.
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


def _rows(n):
    return sorted({0, 1, 127, 128, n // 3 + 5, n // 2 + 63, n - 129, n - 2, n - 1})


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_dense_forward_n262144(causal):
    dev = device()
    N, d = 262144, 64
    announce("large dense fwd", N, causal)
    q, k, v = W.kv_inputs(1, 1, N, N, d, "bf16", 61000, with_grad=False)
    o, lse = fa.forward(*to_dev((q, k, v), dev), scale=0.125, causal=causal)
    torch.cuda.synchronize()
    rows = _rows(N)
    ro, rl = oracle.attention_forward_rows(q, k, v, 0.125, causal, 0, 0, rows)
    check(o[0, 0, rows], ro, "bf16", f"N={N} O rows")
    check_lse(lse[0, 0, rows], rl, "bf16", f"N={N} LSE rows")


def test_sparse_forward_at_the_mask_limit():
    """N = 524288 (4096 mask blocks per side, the largest the kernels accept) at 2% density, causal."""
    dev = device()
    N, d = 524288, 64
    announce("large sparse fwd", N)
    q, k, v = W.kv_inputs(1, 1, N, N, d, "bf16", 61100, with_grad=False)
    m = W.block_mask(1, 1, N, 0.02, 61101)
    m[0, 0, :, 0] = 1  # every query block keeps the first key block: no empty causal rows
    o, lse = fa.forward_sparse(*to_dev((q, k, v), dev), m.to(dev), scale=0.125, causal=True)
    torch.cuda.synchronize()
    rows = _rows(N)
    ro, rl = oracle.attention_forward_sparse_rows(q, k, v, 0.125, True, m.numpy(), 0, 0, rows)
    check(o[0, 0, rows], ro, "bf16", "sparse N=524288 O rows")
    check_lse(lse[0, 0, rows], rl, "bf16", "sparse N=524288 LSE rows")


def test_split_decode_against_a_million_keys():
    """One query per head against 2^20 keys through the split-key forward; every row checked."""
    dev = device()
    B, H, Nk, d = 1, 2, 1 << 20, 128
    announce("decode 2^20 keys")
    q, k, v = W.kv_inputs(B, H, 1, Nk, d, "bf16", 61200, with_grad=False)
    o, lse = fa.forward_kv_split(*to_dev((q, k, v), dev), causal=True)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_forward_kv(q, k, v, 1.0 / np.sqrt(d), True)
    check(o, ro, "bf16", "decode 2^20 O")
    check_lse(lse, rl, "bf16", "decode 2^20 LSE")


def test_backward_n65536():
    dev = device()
    N, d = 65536, 128
    sc = 0.08838835
    announce("large bwd", N)
    q, k, v, do = W.kv_inputs(1, 1, N, N, d, "bf16", 61300)
    qd, kd, vd, dod = to_dev((q, k, v, do), dev)
    o, lse = fa.forward(qd, kd, vd, scale=sc, causal=True)
    dq, dk, dv = fa.backward(qd, kd, vd, o, lse, dod, scale=sc, causal=True)
    torch.cuda.synchronize()
    rows = _rows(N)
    rdq = oracle.attention_backward_rows(q, k, v, do, sc, True, 0, 0, rows)
    check(dq[0, 0, rows], rdq, "bf16", "N=65536 dQ rows", rel_gate=GRAD_REL["bf16"])
    # identities over all keys (fp64 sums of the bf16 outputs)
    dk64, dv64, do64 = to_np(dk[0, 0]), to_np(dv[0, 0]), to_np(dod[0, 0])
    dk_sum, dk_abs = np.abs(dk64.sum(axis=0)), np.abs(dk64).sum(axis=0)
    assert np.all(dk_sum <= 1e-3 * dk_abs + 1e-3), f"sum_j dK_j not 0: worst {np.max(dk_sum / (dk_abs + 1e-30)):.2e}"
    dv_err = np.abs(dv64.sum(axis=0) - do64.sum(axis=0))
    assert np.all(dv_err <= 1e-3 * np.abs(dv64).sum(axis=0) + 1e-2), f"sum_j dV_j != sum_i dO_i: {dv_err.max():.3e}"


# ------------------------------------------------------------------ addressing past 2^32 bytes per head
# With Q = K = 0 every score is 0, so each row's softmax is uniform: O = (sum of the V
# rows) / Nk and LSE = ln Nk exactly, whatever the length.  V (or dO) is zero except
# "probe" rows set to 1, placed around the row counts where a 32-bit byte count or
# offset per head would wrap (2^24 rows of 256 bytes, 2^23 rows of 512 bytes); a
# tile that is read short, or from the wrong place, changes the result.

def _probe_rows(n, wrap):
    rows = {0, 1, n - 1, wrap - 1, wrap, wrap + 1}
    rows |= set(range(n - wrap - 64, n - wrap + 64))  # the tile whose remaining byte count wraps to a few KiB
    return sorted(r for r in rows if 0 <= r < n)


@pytest.mark.parametrize("path", ["kv", "split", "fp32"])
def test_key_addressing_beyond_4gib_per_head(path):
    dev = device()
    dtype = torch.float32 if path == "fp32" else torch.bfloat16
    d = 128
    wrap = (1 << 32) // (d * (4 if path == "fp32" else 2))  # rows per 4 GiB
    nk = wrap + 1000
    announce("long keys", path, nk)
    q = torch.zeros((1, 1, 1, d), dtype=dtype, device=dev)
    k = torch.zeros((1, 1, nk, d), dtype=dtype, device=dev)
    v = torch.zeros((1, 1, nk, d), dtype=dtype, device=dev)
    probes = _probe_rows(nk, wrap)
    v[0, 0, probes] = 1.0
    if path == "split":
        o, lse = fa.forward_kv_split(q, k, v, num_splits=64)
    else:
        o, lse = fa.forward_kv(q, k, v)
    torch.cuda.synchronize()
    want = len(probes) / nk
    got = o.double().cpu().numpy()
    assert np.allclose(got, want, rtol=1e-2, atol=0), f"{path}: O {got.min():.6e}..{got.max():.6e}, want {want:.6e}"
    assert abs(float(lse) - np.log(nk)) <= 1e-4, f"{path}: LSE {float(lse)} vs {np.log(nk)}"
    del k, v


def test_query_addressing_beyond_4gib_per_head():
    """The backward streams Q and dO tiles past 2^24 rows of 256 bytes: dV_j = (sum_i dO_i) / Nk exactly."""
    dev = device()
    d, nk = 128, 64
    wrap = (1 << 32) // (d * 2)
    nq = wrap + 1000
    announce("long queries", nq)
    q = torch.zeros((1, 1, nq, d), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((1, 1, nk, d), dtype=torch.bfloat16, device=dev)
    v = torch.randn((1, 1, nk, d), generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).to(dev)
    do = torch.zeros_like(q)
    probes = _probe_rows(nq, wrap)
    do[0, 0, probes] = 1.0
    o, lse = fa.forward_kv(q, k, v)
    dq, dk, dv = fa.backward_kv(q, k, v, o, lse, do)
    torch.cuda.synchronize()
    want = len(probes) / nk
    got = dv.double().cpu().numpy()
    assert np.allclose(got, want, rtol=1e-2, atol=0), f"dV {got.min():.6e}..{got.max():.6e}, want {want:.6e}"
    assert float(dq.abs().max()) == 0.0 and float(dk.abs().max()) == 0.0
    o_want = v.double().mean(dim=2, keepdim=True).cpu().numpy()
    o_rows = o[0, 0, probes].double().cpu().numpy()
    assert np.allclose(o_rows, o_want[0, 0], rtol=1e-2, atol=1e-3), "O of probe rows is not mean(V)"
