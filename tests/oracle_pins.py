"""Pins that tie the CPU oracle to facts outside itself.

Each pin takes an oracle-like object `orc` (attributes attention_forward,
attention_backward, attention_probs) and raises AssertionError on failure, so
the same pins run against the real oracle (test_oracle_pins.py) and against
copies of it with planted mistakes (test_oracle_mutants.py).

What each pin rests on:
  * brute force: scalar loops with math.exp / math.fsum straight from the
    definition softmax(QK^T/sqrt(d))V ("How Flash Attention Works: Tiling,
    Softmax, GPU I/O", section "How Flash Attention Works: The Exact-Attention
    Idea");
  * a worked example derived by hand (tests/golden/worked_example.json);
  * closed forms: constant V, Q = 0 (uniform weights, prefix means under the
    causal mask), causal row 0, N = 1, shift of every key by one vector;
  * invariants: probability rows sum to one, permutation equivariance;
  * the online recurrence: the running max / running normaliser update with
    rescaling of the partial output "converges to the identical value"
    as the full-row softmax ("How Flash Attention Works", section "Online
    Softmax Without the Full Score Matrix"), written here independently;
  * library special cases: scipy.special.logsumexp for the LSE, and torch CPU
    float64 autograd of the naive expression for the outputs and gradients;
  * central finite differences for the gradients, and the gradient
    invariants that follow from softmax rows summing to one.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _qkv(seed, B, H, N, d, dv=None, scale_q=1.0):
    r = _rng(seed)
    dv = d if dv is None else dv
    q = r.standard_normal((B, H, N, d)) * scale_q
    k = r.standard_normal((B, H, N, d))
    v = r.standard_normal((B, H, N, dv))
    return q, k, v


def _close(a, b, tol, what):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


# ---------------------------------------------------------------- brute force
def _brute_head(q, k, v, scale, causal):
    n, dv = len(q), len(v[0])
    o = [[0.0] * dv for _ in range(n)]
    lse = [0.0] * n
    for i in range(n):
        keys = [j for j in range(len(k)) if not (causal and j > i)]
        s = {j: scale * math.fsum(q[i][c] * k[j][c] for c in range(len(q[i]))) for j in keys}
        z = math.fsum(math.exp(s[j]) for j in keys)
        lse[i] = math.log(z)
        for c in range(dv):
            o[i][c] = math.fsum(math.exp(s[j]) / z * v[j][c] for j in keys)
    return o, lse


def pin_bruteforce_forward(orc):
    for seed, (N, d, causal) in enumerate([(1, 1, False), (3, 2, True), (5, 3, False),
                                           (8, 4, True), (8, 4, False), (7, 2, True)]):
        q, k, v = _qkv(100 + seed, 1, 2, N, d)
        scale = 1.0 / math.sqrt(d)
        # whole rows at once, and in panels of 3 rows (a memory device only)
        for o, lse in (orc.attention_forward(q, k, v, scale, causal),
                       orc.attention_forward(q, k, v, scale, causal, panel_rows=3)):
            for h in range(2):
                bo, bl = _brute_head(q[0, h].tolist(), k[0, h].tolist(), v[0, h].tolist(), scale, causal)
                _close(o[0, h], bo, 1e-12, f"brute O N={N} causal={causal}")
                _close(lse[0, h], bl, 1e-12, f"brute LSE N={N} causal={causal}")


# ------------------------------------------------------------ worked example
def _ev(x):
    return eval(x, {"__builtins__": {}}, {"ln": math.log})  # noqa: S307 - our own fixture


def _mat(rows):
    return np.array([[_ev(x) for x in r] for r in rows], dtype=np.float64)


def pin_worked_example(orc):
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        g = json.load(f)
    q, k, v, do = (_mat(g[n])[None, None] for n in ("q", "k", "v", "do"))
    for mode, causal in (("noncausal", False), ("causal", True)):
        e = g[mode]
        o, lse = orc.attention_forward(q, k, v, g["scale"], causal)
        _close(o[0, 0], _mat(e["o"]), 1e-14, f"worked O {mode}")
        _close(lse[0, 0], [_ev(x) for x in e["lse"]], 1e-14, f"worked LSE {mode}")
        _close(orc.attention_probs(q[0, 0], k[0, 0], g["scale"], causal), _mat(e["p"]), 1e-14, f"worked P {mode}")
        dq, dk, dv = orc.attention_backward(q, k, v, do, g["scale"], causal)
        _close(dq[0, 0], _mat(e["dq"]), 1e-14, f"worked dQ {mode}")
        _close(dk[0, 0], _mat(e["dk"]), 1e-14, f"worked dK {mode}")
        _close(dv[0, 0], _mat(e["dv"]), 1e-14, f"worked dV {mode}")


# ---------------------------------------------------------------- invariants
def pin_probability_rows(orc):
    for causal in (False, True):
        q, k, _ = _qkv(7, 1, 1, 37, 8, scale_q=3.0)
        p = orc.attention_probs(q[0, 0], k[0, 0], 0.3, causal)
        assert np.all(p >= 0.0), "negative probability"
        _close(p.sum(axis=1), np.ones(37), 1e-12, "row sums")
        if causal:
            assert np.all(np.triu(p, 1) == 0.0), "causal mask leaks future keys"
            assert np.all(np.diag(p) > 0.0), "causal mask hides the diagonal"


def pin_constant_v(orc):
    for causal in (False, True):
        q, k, _ = _qkv(8, 2, 2, 29, 16)
        row = _rng(9).standard_normal(16)
        v = np.broadcast_to(row, q.shape).copy()
        o, _ = orc.attention_forward(q, k, v, 0.25, causal)
        _close(o, v, 1e-12, f"constant V causal={causal}")


def pin_q_zero(orc):
    """Q = 0: all allowed keys get weight 1/count, LSE = ln(count)."""
    _, k, v = _qkv(10, 1, 2, 33, 8)
    q = np.zeros_like(k)
    n = 33
    for causal in (False, True):
        o, lse = orc.attention_forward(q, k, v, 0.125, causal)
        if causal:
            cnt = np.arange(1, n + 1, dtype=np.float64)
            ref_o = np.cumsum(v, axis=2) / cnt[:, None]
        else:
            cnt = np.full(n, float(n))
            ref_o = np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
        _close(o, ref_o, 1e-12, f"Q=0 O causal={causal}")
        _close(lse, np.broadcast_to(np.log(cnt), lse.shape), 1e-12, f"Q=0 LSE causal={causal}")


def pin_causal_row0_and_n1(orc):
    q, k, v = _qkv(11, 2, 3, 19, 8)
    scale = 0.35
    o, lse = orc.attention_forward(q, k, v, scale, True)
    _close(o[:, :, 0], v[:, :, 0], 0.0, "causal row 0 equals V_0")
    _close(lse[:, :, 0], scale * np.sum(q[:, :, 0] * k[:, :, 0], axis=-1), 1e-14, "causal LSE_0")
    for causal in (False, True):
        o1, l1 = orc.attention_forward(q[:, :, :1], k[:, :, :1], v[:, :, :1], scale, causal)
        _close(o1, v[:, :, :1], 0.0, "N=1 O")
        _close(l1[..., 0], scale * np.sum(q[:, :, 0] * k[:, :, 0], axis=-1), 1e-14, "N=1 LSE")


def pin_shift_invariance(orc):
    """K + u: every score of row i moves by scale*q_i.u, so O is unchanged and LSE shifts."""
    q, k, v = _qkv(12, 1, 2, 31, 8)
    u = _rng(13).standard_normal(8)
    scale = 0.3
    for causal in (False, True):
        o, lse = orc.attention_forward(q, k, v, scale, causal)
        o2, lse2 = orc.attention_forward(q, k + u, v, scale, causal)
        _close(o2, o, 1e-12, "shift O")
        _close(lse2 - lse, scale * (q @ u), 1e-12, "shift LSE")


def pin_permutation(orc):
    """Non-causal: permuting queries permutes outputs; permuting keys with values changes nothing."""
    q, k, v = _qkv(14, 1, 2, 40, 8)
    r = _rng(15)
    pq, pk = r.permutation(40), r.permutation(40)
    o, lse = orc.attention_forward(q, k, v, 0.4, False)
    o2, lse2 = orc.attention_forward(q[:, :, pq], k, v, 0.4, False)
    _close(o2, o[:, :, pq], 1e-12, "query permutation O")
    _close(lse2, lse[:, :, pq], 1e-12, "query permutation LSE")
    o3, lse3 = orc.attention_forward(q, k[:, :, pk], v[:, :, pk], 0.4, False)
    _close(o3, o, 1e-12, "key/value permutation O")
    _close(lse3, lse, 1e-12, "key/value permutation LSE")


def pin_online_recurrence(orc):
    """An independent online-softmax pass over key blocks equals the oracle."""
    q, k, v = _qkv(16, 1, 2, 70, 8, scale_q=2.0)
    scale = 0.5
    for causal in (False, True):
        o, lse = orc.attention_forward(q, k, v, scale, causal)
        for blk in (1, 3, 64, 70):
            for h in range(2):
                qh, kh, vh = q[0, h], k[0, h], v[0, h]
                n = len(qh)
                m = np.full(n, -np.inf)
                l = np.zeros(n)
                acc = np.zeros((n, vh.shape[1]))
                for j0 in range(0, n, blk):
                    s = scale * qh @ kh[j0:j0 + blk].T
                    if causal:
                        s[np.arange(j0, j0 + s.shape[1])[None, :] > np.arange(n)[:, None]] = -np.inf
                    mn = np.maximum(m, s.max(axis=1))
                    alive = np.isfinite(mn)
                    ratio = np.where(alive, np.exp(np.where(alive, m - mn, 0.0)), 1.0)
                    w = np.where(alive[:, None], np.exp(s - np.where(alive, mn, 0.0)[:, None]), 0.0)
                    l = ratio * l + w.sum(axis=1)
                    acc = ratio[:, None] * acc + w @ vh[j0:j0 + blk]
                    m = mn
                _close(o[0, h], acc / l[:, None], 1e-12, f"online O blk={blk} causal={causal}")
                _close(lse[0, h], m + np.log(l), 1e-12, f"online LSE blk={blk} causal={causal}")


def pin_scipy_logsumexp(orc):
    from scipy.special import logsumexp, softmax
    q, k, v = _qkv(17, 1, 1, 45, 16)
    s = 0.25 * q[0, 0] @ k[0, 0].T
    o, lse = orc.attention_forward(q, k, v, 0.25, False)
    _close(lse[0, 0], logsumexp(s, axis=1), 1e-12, "scipy logsumexp")
    _close(o[0, 0], softmax(s, axis=1) @ v[0, 0], 1e-12, "scipy softmax")


# ----------------------------------------------------------------- backward
def pin_torch_autograd(orc):
    import torch
    for causal in (False, True):
        q, k, v = _qkv(18, 2, 2, 23, 8)
        do = _rng(19).standard_normal(q.shape)
        scale = 0.3
        tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
        s = scale * torch.matmul(tq, tk.transpose(-1, -2).contiguous())
        if causal:
            mask = torch.ones(23, 23, dtype=torch.bool).triu(1)
            s = s.masked_fill(mask, float("-inf"))
        out = torch.matmul(torch.softmax(s, dim=-1), tv)
        tl = torch.logsumexp(s, dim=-1)
        (out * torch.tensor(do)).sum().backward()
        o, lse = orc.attention_forward(q, k, v, scale, causal)
        _close(o, out.detach().numpy(), 1e-12, f"autograd O causal={causal}")
        _close(lse, tl.detach().numpy(), 1e-12, f"autograd LSE causal={causal}")
        dq, dk, dv = orc.attention_backward(q, k, v, do, scale, causal)
        _close(dq, tq.grad.numpy(), 1e-10, f"autograd dQ causal={causal}")
        _close(dk, tk.grad.numpy(), 1e-10, f"autograd dK causal={causal}")
        _close(dv, tv.grad.numpy(), 1e-10, f"autograd dV causal={causal}")


def pin_finite_differences(orc):
    for causal in (False, True):
        q, k, v = _qkv(20, 1, 1, 6, 4)
        do = _rng(21).standard_normal(q.shape)
        scale = 0.45
        grads = orc.attention_backward(q, k, v, do, scale, causal)
        base = [q, k, v]
        h = 1e-6
        for which in range(3):
            num = np.zeros_like(base[which])
            for idx in np.ndindex(base[which].shape):
                loss = []
                for sgn in (1.0, -1.0):
                    xs = [x.copy() for x in base]
                    xs[which][idx] += sgn * h
                    o, _ = orc.attention_forward(*xs, scale, causal)
                    loss.append(np.sum(o * do))
                num[idx] = (loss[0] - loss[1]) / (2 * h)
            err = np.max(np.abs(num - grads[which])) / max(1.0, np.max(np.abs(num)))
            assert err < 1e-7, f"finite differences grad {which} causal={causal}: {err:.2e}"


def pin_backward_invariants(orc):
    q, k, v = _qkv(22, 2, 2, 27, 8)
    do = _rng(23).standard_normal(q.shape)
    for causal in (False, True):
        dq, dk, dv = orc.attention_backward(q, k, v, do, 0.3, causal)
        # every dS row sums to zero, so the key gradients sum to zero
        _close(dk.sum(axis=2), np.zeros((2, 2, 8)), 1e-10, "sum_j dK_j = 0")
        # every P row sums to one, so the value gradients sum to sum_i dO_i
        _close(dv.sum(axis=2), do.sum(axis=2), 1e-10, "sum_j dV_j = sum_i dO_i")
        if causal:
            _close(dq[:, :, 0], np.zeros((2, 2, 8)), 1e-14, "causal dQ_0 = 0")
        z = orc.attention_backward(q, k, v, np.zeros_like(do), 0.3, causal)
        for g in z:
            _close(g, np.zeros_like(g), 0.0, "dO = 0 gives zero gradients")


ALL_PINS = [pin_bruteforce_forward, pin_worked_example, pin_probability_rows, pin_constant_v,
            pin_q_zero, pin_causal_row0_and_n1, pin_shift_invariance, pin_permutation,
            pin_online_recurrence, pin_scipy_logsumexp, pin_torch_autograd,
            pin_finite_differences, pin_backward_invariants]
