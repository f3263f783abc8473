"""Parity gates between the HIP path and the fp64 oracle.

Stated gates: max abs error 1e-4 for fp32 I/O; |x - r| <= 2e-2 + 1e-2 |r|
elementwise for bf16/fp16 outputs and gradients.  Because attention outputs are
small at long sequence lengths (|O| ~ sigma_V * sqrt(e^{sigma_s^2} / n)), an
all-zero output would pass the 16-bit elementwise gate, so two supplemental
gates are always applied as well: the relative Frobenius error ||x - r|| / ||r||
and a max-abs bound on the log-sum-exp.
"""
from __future__ import annotations

import numpy as np

FWD_REL = {"f32": 1e-5, "f16": 3e-3, "bf16": 1e-2}
GRAD_REL = {"f32": 1e-5, "f16": 1e-2, "bf16": 2e-2}
LSE_ABS = {"f32": 1e-5, "f16": 1e-3, "bf16": 1e-3}


def to_np(x):
    import torch
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def check(x, ref, dtype, what, rel_gate=None):
    """Assert the stated gate and the relative Frobenius gate; return the error stats."""
    x, ref = to_np(x), to_np(ref)
    assert x.shape == ref.shape, f"{what}: shape {x.shape} vs {ref.shape}"
    assert np.all(np.isfinite(x)), f"{what}: non-finite values"
    diff = np.abs(x - ref)
    max_abs = float(diff.max()) if diff.size else 0.0
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(x - ref) / nref) if nref > 0 else float(np.linalg.norm(x - ref))
    if dtype == "f32":
        assert max_abs <= 1e-4, f"{what}: max abs err {max_abs:.3e} > 1e-4"
    else:
        bound = 2e-2 + 1e-2 * np.abs(ref)
        worst = float((diff - bound).max()) if diff.size else -1.0
        assert worst <= 0.0, f"{what}: elementwise gate exceeded by {worst:.3e} (max abs err {max_abs:.3e})"
    gate = rel_gate if rel_gate is not None else FWD_REL[dtype]
    assert rel <= gate, f"{what}: relative Frobenius error {rel:.3e} > {gate:.1e}"
    return {"max_abs": max_abs, "rel_fro": rel}


def check_lse(x, ref, dtype, what):
    x, ref = to_np(x), to_np(ref)
    err = float(np.max(np.abs(x - ref))) if x.size else 0.0
    assert np.all(np.isfinite(x)), f"{what}: non-finite LSE"
    assert err <= LSE_ABS[dtype], f"{what}: LSE max abs err {err:.3e} > {LSE_ABS[dtype]:.0e}"
    return err


def check_blocks(x, ref, dtype, what, rel_gate=None, block=128):
    """check() over a whole [B, H, N, d] tensor, also per (b, h) head: the
    relative Frobenius gate holds for every head on its own, and a failure
    names the (b, h, 128-row block) where the worst element sits."""
    x, ref = to_np(x), to_np(ref)
    assert x.shape == ref.shape, f"{what}: shape {x.shape} vs {ref.shape}"
    assert np.all(np.isfinite(x)), f"{what}: non-finite values at {np.argwhere(~np.isfinite(x))[0].tolist()}"
    diff = np.abs(x - ref)
    if dtype == "f32":
        excess = diff - 1e-4
    else:
        excess = diff - (2e-2 + 1e-2 * np.abs(ref))
    b, h, i, c = np.unravel_index(int(np.argmax(excess)), excess.shape)
    assert excess[b, h, i, c] <= 0.0, (f"{what}: gate exceeded by {excess[b, h, i, c]:.3e} at head ({b}, {h}), "
                                       f"row {i} (block {i // block}), column {c}")
    gate = rel_gate if rel_gate is not None else FWD_REL[dtype]
    num = np.sqrt(np.sum((x - ref) ** 2, axis=(2, 3)))
    den = np.sqrt(np.sum(ref ** 2, axis=(2, 3)))
    rel = num / np.where(den > 0, den, 1.0)
    b, h = np.unravel_index(int(np.argmax(rel)), rel.shape)
    assert rel[b, h] <= gate, f"{what}: relative Frobenius error {rel[b, h]:.3e} > {gate:.1e} in head ({b}, {h})"
    return {"max_abs": float(diff.max()), "rel_fro_worst_head": float(rel.max())}


def check_lse_blocks(x, ref, dtype, what, block=128):
    """check_lse() over [B, H, N], naming the (b, h, 128-row block) of the worst row."""
    x, ref = to_np(x), to_np(ref)
    assert np.all(np.isfinite(x)), f"{what}: non-finite LSE"
    err = np.abs(x - ref)
    b, h, i = np.unravel_index(int(np.argmax(err)), err.shape)
    assert err[b, h, i] <= LSE_ABS[dtype], (f"{what}: LSE max abs err {err[b, h, i]:.3e} > {LSE_ABS[dtype]:.0e} at "
                                            f"head ({b}, {h}), row {i} (block {i // block})")
    return float(err.max())


# Unit roundoff u and half the smallest subnormal spacing eta of the 16-bit I/O types:
# a rounded value x' satisfies |x' - x| <= u |x| + eta.
ROUNDING = {"bf16": (2.0 ** -8, 2.0 ** -134), "f16": (2.0 ** -11, 2.0 ** -25)}


def bwd_rounding_bound(q, k, v, do, o, terms, scale, dtype):
    """First-order bound on the gradient error of a 16-bit backward pass that
    follows the recompute scheme, for one head ([N, d] float64 q, k, v, do,
    the exact output o, and terms = (P, dP, D, dS) from the oracle).

    Roundings to the I/O type (unit roundoff u, subnormal half-spacing eta):
      * the forward rounds P before P V and rounds O at the store, and
        D_i = sum_c dO_ic O_ic is formed from that O;
      * P is rounded before dV = P^T dO, and dS = P (dP - D) before
        dQ = scale dS K and dK = scale dS^T Q;
      * dQ, dK, dV are rounded once more at the store.
    fp32 work, with worst-case accumulation factors g_n = n 2^-24: the scores
    (d products, error g_d sum_c |q_ic k_jc| before the scale), the
    exponentials (2^-22 relative), the log-sum-exp (the scores' error plus the
    forward's sum of N weights), dP (g_d sum_c |dO_ic v_jc|), D, and every
    sum of N products.  Returns bounds shaped like (dQ, dK, dV)."""
    u, eta = ROUNDING[dtype]
    n, d = q.shape[0], q.shape[1]
    g_d, g_n = d * 2.0 ** -24, n * 2.0 ** -24
    p, dp, dd, ds = terms
    aq, ak, av, ado = np.abs(q), np.abs(k), np.abs(v), np.abs(do)
    a_s = aq @ ak.T                                      # sum_c |q_ic k_jc|
    sc = abs(scale)
    # relative error of the fp32 weights exp(scale s_ij - LSE_i)
    eps = sc * g_d * a_s + (sc * g_d * np.max(a_s, axis=1, keepdims=True) + g_n) + 2.0 ** -22
    # forward output: P rounded and in error by eps, a sum of N products, O rounded
    pv = p @ av
    o_err = (u + g_n) * pv + (eps * p) @ av + eta * av.sum(axis=0)[None, :] + u * np.abs(o)
    d_err = np.sum(ado * o_err, axis=1) + g_d * np.sum(ado * np.abs(o), axis=1)      # |D_gpu - D|
    dp_err = g_d * (ado @ av.T)
    e = (eps * p * np.abs(dp - dd[:, None]) + p * (dp_err + d_err[:, None])        # dS before rounding
         + u * np.abs(ds) + eta)                                                     # and its rounding
    gq = sc * (e @ ak + g_n * (np.abs(ds) @ ak))
    gk = sc * (e.T @ aq + g_n * (np.abs(ds).T @ aq))
    gv = ((u + eps + g_n) * p + eta).T @ ado
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    dv = p.T @ do
    return (gq + u * np.abs(dq) + eta, gk + u * np.abs(dk) + eta, gv + u * np.abs(dv) + eta)


# ---------------------------------------------------------------- 8-bit forward
# Error of one 64-product 8-bit matrix instruction relative to its largest
# product: measured on gfx950 over 2^20 products of random full-range codes,
# 2^-10.75 (E4M3 x E4M3), 2^-11.44 (E5M2 x E5M2) and 2^-11.32 (E5M2 x E4M3,
# the P V product on E5M2 values); the gate takes 2^-10 for both formats.
ACC_ERR = {"e4m3": 2.0 ** -10, "e5m2": 2.0 ** -10}


def score_error_bound(q, k, scale, acc, rows=None):
    """delta_i = acc |scale| max_j sum_c |q_ic| |k_jc| per row (over all keys: a valid, looser bound)."""
    if rows is not None:
        b, h, idx = rows
        return acc * abs(scale) * np.max(np.abs(q[b, h, idx]) @ np.abs(k[b, h]).T, axis=1)
    out = np.empty(q.shape[:3])
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            out[b, h] = acc * abs(scale) * np.max(np.abs(q[b, h]) @ np.abs(k[b, h]).T, axis=1)
    return out


def max_weight(q, k, scale, causal, lse, rows=None):
    """max_j P_ij = exp(max over visible j of scale q_i . k_j - lse_i), from the oracle's LSE."""
    def one(qb, kb, idx):
        s = scale * (qb @ kb.T)
        if causal:
            s = np.where(np.arange(kb.shape[0])[None, :] <= np.asarray(idx)[:, None], s, -np.inf)
        return np.max(s, axis=1)
    if rows is not None:
        b, h, idx = rows
        return np.exp(one(q[b, h, idx], k[b, h], idx) - lse)
    out = np.empty(q.shape[:3])
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            out[b, h] = np.exp(one(q[b, h], k[b, h], np.arange(q.shape[2])) - lse[b, h])
    return out


def fp8_output_bound(q, k, v, scale, causal, acc, rows=None):
    """Oracle O, LSE and the elementwise bound on |o - O| of the 8-bit forward
    on the dequantised q, k, v (float64 [B, H, N, d]), plus delta (per row).

    Roundings bounded: the score error delta_i of the 8-bit product (moves each
    weight by a relative 2 delta_i); the E4M3 rounding of each weight before
    P V, relative 2^-4 at and above 2^-6, absolute 2^-10 below, which on the
    normalised weight is at most 2^-10 max_j P_ij since the kernel's row sum
    is >= 1 / max_j P_ij (its running maximum never exceeds the true one);
    fp32 accumulation (2^-16 relative); the bf16 store (2^-8 relative):

        |o - O| <= (2^-4 + 2 delta_i + 2^-16) (P |V|)_ic
                   + 2^-10 max_j P_ij sum_j |v_jc| + 2^-8 |O_ic|.
    """
    import oracle
    if rows is None:
        ro, rl = oracle.attention_forward(q, k, v, scale, causal)
        pv, _ = oracle.attention_forward(q, k, np.abs(v), scale, causal)
        vsum = np.sum(np.abs(v), axis=-2, keepdims=True)
    else:
        b, h, idx = rows
        ro, rl = oracle.attention_forward_rows(q, k, v, scale, causal, b, h, idx)
        pv, _ = oracle.attention_forward_rows(q, k, np.abs(v), scale, causal, b, h, idx)
        vsum = np.sum(np.abs(v[b, h]), axis=0, keepdims=True)
    delta = score_error_bound(q, k, scale, acc, rows)
    pmax = max_weight(q, k, scale, causal, rl, rows)
    bound = (2.0 ** -4 + 2.0 * delta[..., None] + 2.0 ** -16) * pv + 2.0 ** -10 * pmax[..., None] * vsum \
        + 2.0 ** -8 * np.abs(ro)
    return ro, rl, bound, delta
