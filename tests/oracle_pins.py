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
    rescaling of the partial output ends at the same value as the full-row
    softmax ("How Flash Attention Works", section "Online
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


# ------------------------------------------- unequal counts, padded batches
# Readings (the pages fix neither): the lq queries of a sequence are the last
# lq positions of its lk keys, so under the causal mask query i sees key j iff
# j <= i + (lk - lq); rows past a length, and rows that see no key, output
# O = 0 and LSE = -inf and take no part in any gradient.
def _visible(i, j, lq, lk, causal):
    return i < lq and j < lk and (not causal or j <= i + (lk - lq))


def _brute_kv(q, k, v, scale, causal, lq, lk):
    """One (b, h) slice by scalar loops: O [Nq][dv] and LSE [Nq]."""
    nq, dv = len(q), len(v[0])
    o = [[0.0] * dv for _ in range(nq)]
    lse = [-math.inf] * nq
    for i in range(nq):
        js = [j for j in range(len(k)) if _visible(i, j, lq, lk, causal)]
        if not js:
            continue
        s = {j: scale * math.fsum(a * b for a, b in zip(q[i], k[j])) for j in js}
        m = max(s.values())
        w = {j: math.exp(s[j] - m) for j in js}
        z = math.fsum(w.values())
        lse[i] = m + math.log(z)
        for c in range(dv):
            o[i][c] = math.fsum(w[j] * v[j][c] for j in js) / z
    return o, lse


def _qkv_kv(seed, B, H, Nq, Nk, d):
    r = _rng(seed)
    return r.standard_normal((B, H, Nq, d)), r.standard_normal((B, H, Nk, d)), r.standard_normal((B, H, Nk, d))


def pin_kv_reduces_to_square(orc):
    """Equal counts and no lengths give the square definition exactly."""
    q, k, v = _qkv(30, 2, 2, 19, 8)
    do = _rng(31).standard_normal(q.shape)
    for causal in (False, True):
        o, lse = orc.attention_forward(q, k, v, 0.3, causal)
        o2, lse2 = orc.attention_forward_kv(q, k, v, 0.3, causal, [19, 19], None)
        _close(o2, o, 1e-13, f"kv O = square O causal={causal}")
        _close(lse2, lse, 1e-13, f"kv LSE = square LSE causal={causal}")
        g = orc.attention_backward(q, k, v, do, 0.3, causal)
        g2 = orc.attention_backward_kv(q, k, v, do, 0.3, causal)
        for a, b, n in zip(g2, g, "QKV"):
            _close(a, b, 1e-12, f"kv d{n} = square d{n} causal={causal}")


def pin_kv_worked_example(orc):
    with open(os.path.join(GOLDEN, "kv_worked_example.json")) as f:
        g = json.load(f)
    q, k, v, do = (_mat(g[n])[None, None] for n in ("q", "k", "v", "do"))
    pad = g["padded"]
    qp = np.concatenate([q, _mat([pad["q_pad_row"]])[None, None]], axis=2)
    kp = np.concatenate([k, _mat([pad["k_pad_row"]])[None, None]], axis=2)
    vp = np.concatenate([v, _mat([pad["v_pad_row"]])[None, None]], axis=2)
    dop = np.concatenate([do, _mat([pad["do_pad_row"]])[None, None]], axis=2)
    for mode, causal in (("noncausal", False), ("causal", True)):
        e = g[mode]
        want = {n: _mat(e[n]) for n in ("o", "dq", "dk", "dv")}
        want_lse = [_ev(x) for x in e["lse"]]
        o, lse = orc.attention_forward_kv(q, k, v, g["scale"], causal)
        _close(o[0, 0], want["o"], 1e-14, f"kv worked O {mode}")
        _close(lse[0, 0], want_lse, 1e-14, f"kv worked LSE {mode}")
        dq, dk, dv = orc.attention_backward_kv(q, k, v, do, g["scale"], causal)
        _close(dq[0, 0], want["dq"], 1e-14, f"kv worked dQ {mode}")
        _close(dk[0, 0], want["dk"], 1e-14, f"kv worked dK {mode}")
        _close(dv[0, 0], want["dv"], 1e-14, f"kv worked dV {mode}")
        # padded to 3 query rows / 4 key rows, lengths (2, 3): same values, zero padding rows
        o, lse = orc.attention_forward_kv(qp, kp, vp, g["scale"], causal, pad["seqlens_q"], pad["seqlens_k"])
        _close(o[0, 0], np.vstack([want["o"], np.zeros((1, 2))]), 1e-14, f"kv padded O {mode}")
        assert lse[0, 0, 2] == -math.inf, f"kv padded LSE row {mode}"
        _close(lse[0, 0, :2], want_lse, 1e-14, f"kv padded LSE {mode}")
        dq, dk, dv = orc.attention_backward_kv(qp, kp, vp, dop, g["scale"], causal, pad["seqlens_q"], pad["seqlens_k"])
        _close(dq[0, 0], np.vstack([want["dq"], np.zeros((1, 1))]), 1e-14, f"kv padded dQ {mode}")
        _close(dk[0, 0], np.vstack([want["dk"], np.zeros((1, 1))]), 1e-14, f"kv padded dK {mode}")
        _close(dv[0, 0], np.vstack([want["dv"], np.zeros((1, 2))]), 1e-14, f"kv padded dV {mode}")


def pin_kv_bruteforce(orc):
    """Ragged lengths, both alignments of counts, rows that see no key."""
    q, k, v = _qkv_kv(32, 3, 2, 6, 5, 3)
    lens = ([6, 4, 2], [5, 5, 3])  # lq > lk (empty causal rows), lq < lk, lq < lk
    for causal in (False, True):
        for scale in (0.7, -0.4):
            o, lse = orc.attention_forward_kv(q, k, v, scale, causal, *lens)
            for b in range(3):
                for h in range(2):
                    bo, bl = _brute_kv(q[b, h].tolist(), k[b, h].tolist(), v[b, h].tolist(), scale, causal,
                                       lens[0][b], lens[1][b])
                    _close(o[b, h], bo, 1e-12, f"kv brute O b={b} causal={causal}")
                    assert np.array_equal(np.isinf(lse[b, h]), np.isinf(bl)), f"kv brute empty rows b={b}"
                    fin = ~np.isinf(np.asarray(bl))
                    _close(lse[b, h][fin], np.asarray(bl)[fin], 1e-12, f"kv brute LSE b={b} causal={causal}")


def pin_kv_decode_and_empty(orc):
    q, k, v = _qkv_kv(33, 2, 2, 1, 9, 4)
    # one query at the end of the sequence sees every key: causal = non-causal
    oc, lc = orc.attention_forward_kv(q, k, v, 0.5, True)
    on, ln_ = orc.attention_forward_kv(q, k, v, 0.5, False)
    _close(oc, on, 1e-15, "decode causal = non-causal")
    _close(lc, ln_, 1e-15, "decode LSE")
    # three queries, one key, causal: rows 0 and 1 see nothing; row 2 sees key 0 only
    q, k, v = _qkv_kv(34, 1, 1, 3, 1, 4)
    o, lse = orc.attention_forward_kv(q, k, v, 0.5, True)
    _close(o[0, 0, :2], np.zeros((2, 4)), 0.0, "empty rows O = 0")
    assert np.all(lse[0, 0, :2] == -math.inf), "empty rows LSE = -inf"
    _close(o[0, 0, 2], v[0, 0, 0], 1e-15, "single visible key: O = v_0")
    _close(lse[0, 0, 2], 0.5 * float(q[0, 0, 2] @ k[0, 0, 0]), 1e-15, "single visible key: LSE = s")
    do = _rng(35).standard_normal(q.shape)
    dq, dk, dv = orc.attention_backward_kv(q, k, v, do, 0.5, True)
    _close(dq[0, 0], np.zeros((3, 4)), 0.0, "one key: dS = 0 so dQ = 0")
    _close(dk[0, 0], np.zeros((1, 4)), 0.0, "one key: dK = 0")
    _close(dv[0, 0, 0], do[0, 0, 2], 1e-15, "one key: dV_0 = dO of the row that sees it")
    # no keys at all
    o, lse = orc.attention_forward_kv(q, k, v, 0.5, False, None, [0])
    _close(o, np.zeros_like(o), 0.0, "lk = 0: O = 0")
    assert np.all(lse == -math.inf), "lk = 0: LSE = -inf"


def pin_kv_padding_invariance(orc):
    """Values past the lengths change nothing; lengths outside [0, N] are clamped."""
    q, k, v = _qkv_kv(36, 2, 2, 7, 8, 4)
    do = _rng(37).standard_normal(q.shape)
    lq, lk = [5, 7], [8, 3]
    q2, k2, v2, do2 = q.copy(), k.copy(), v.copy(), do.copy()
    q2[0, :, 5:] = 9.0; do2[0, :, 5:] = -3.0
    k2[1, :, 3:] = 7.0; v2[1, :, 3:] = 5.0
    for causal in (False, True):
        a = orc.attention_forward_kv(q, k, v, 0.4, causal, lq, lk)
        b = orc.attention_forward_kv(q2, k2, v2, 0.4, causal, lq, lk)
        for x, y, n in zip(a, b, ("O", "LSE")):
            assert np.array_equal(x, y), f"padding values leak into {n} causal={causal}"
        assert np.all(a[0][0, :, 5:] == 0) and np.all(a[1][0, :, 5:] == -math.inf), "padding rows"
        ga = orc.attention_backward_kv(q, k, v, do, 0.4, causal, lq, lk)
        gb = orc.attention_backward_kv(q2, k2, v2, do2, 0.4, causal, lq, lk)
        for x, y, n in zip(ga, gb, "QKV"):
            assert np.array_equal(x, y), f"padding values leak into d{n} causal={causal}"
        assert np.all(ga[0][0, :, 5:] == 0) and np.all(ga[1][1, :, 3:] == 0) and np.all(ga[2][1, :, 3:] == 0)
        c = orc.attention_forward_kv(q, k, v, 0.4, causal, [99, 5], [8, -4])
        d = orc.attention_forward_kv(q, k, v, 0.4, causal, [7, 5], [8, 0])
        assert np.array_equal(c[0], d[0]) and np.array_equal(c[1], d[1]), "lengths are clamped into [0, N]"


def pin_kv_torch_autograd(orc):
    """Per sequence: torch float64 autograd of the naive expression with an explicit mask."""
    import torch
    q, k, v = _qkv_kv(38, 2, 2, 6, 9, 5)
    do = _rng(39).standard_normal(q.shape)
    lq, lk = [6, 4], [9, 7]
    for causal in (False, True):
        o, lse = orc.attention_forward_kv(q, k, v, 0.35, causal, lq, lk)
        dq, dk, dv = orc.attention_backward_kv(q, k, v, do, 0.35, causal, lq, lk)
        for b in range(2):
            a, c = lq[b], lk[b]
            tq, tk, tv = (torch.tensor(x[b, :, :n], dtype=torch.float64, requires_grad=True)
                          for x, n in ((q, a), (k, c), (v, c)))
            s = 0.35 * torch.matmul(tq, tk.transpose(-1, -2).contiguous())
            if causal:
                i = torch.arange(a)[:, None] + (c - a)
                j = torch.arange(c)[None, :]
                s = s.masked_fill(j > i, float("-inf"))
            out = torch.matmul(torch.softmax(s, dim=-1), tv)
            (out * torch.tensor(do[b, :, :a])).sum().backward()
            _close(o[b, :, :a], out.detach().numpy(), 1e-12, f"kv autograd O b={b} causal={causal}")
            _close(lse[b, :, :a], torch.logsumexp(s, dim=-1).detach().numpy(), 1e-12, f"kv autograd LSE b={b}")
            _close(dq[b, :, :a], tq.grad.numpy(), 1e-10, f"kv autograd dQ b={b} causal={causal}")
            _close(dk[b, :, :c], tk.grad.numpy(), 1e-10, f"kv autograd dK b={b} causal={causal}")
            _close(dv[b, :, :c], tv.grad.numpy(), 1e-10, f"kv autograd dV b={b} causal={causal}")


def pin_kv_finite_differences(orc):
    q, k, v = _qkv_kv(40, 1, 1, 4, 5, 3)
    do = _rng(41).standard_normal(q.shape)
    lq, lk = [3], [4]
    for causal in (False, True):
        grads = orc.attention_backward_kv(q, k, v, do, 0.45, causal, lq, lk)
        base = [q, k, v]
        h = 1e-6
        for which in range(3):
            num = np.zeros_like(base[which])
            for idx in np.ndindex(base[which].shape):
                loss = []
                for sgn in (1.0, -1.0):
                    xs = [x.copy() for x in base]
                    xs[which][idx] += sgn * h
                    o, _ = orc.attention_forward_kv(*xs, 0.45, causal, lq, lk)
                    loss.append(np.sum(o * do))
                num[idx] = (loss[0] - loss[1]) / (2 * h)
            err = np.max(np.abs(num - grads[which])) / max(1.0, np.max(np.abs(num)))
            assert err < 1e-7, f"kv finite differences grad {which} causal={causal}: {err:.2e}"


# ------------------------------------------------------------- block sparse
# Reading (the pages name the extension, not a format): a 0/1 mask over
# (query block, key block) pairs removes those scores, on top of the causal
# mask; rows that see no key output O = 0 and LSE = -inf.
def _mask_rand(seed, B, H, nb, p_keep=0.6):
    m = (_rng(seed).random((B, H, nb, nb)) < p_keep).astype(np.uint8)
    return m


def pin_sparse_all_ones_is_dense(orc):
    q, k, v = _qkv(50, 2, 2, 21, 8)
    do = _rng(51).standard_normal(q.shape)
    ones = np.ones((2, 2, 6, 6), dtype=np.uint8)
    for causal in (False, True):
        o, lse = orc.attention_forward(q, k, v, 0.3, causal)
        o2, lse2 = orc.attention_forward_sparse(q, k, v, 0.3, causal, ones, block=4)
        _close(o2, o, 1e-13, f"sparse all-ones O causal={causal}")
        _close(lse2, lse, 1e-13, f"sparse all-ones LSE causal={causal}")
        for a, b, n in zip(orc.attention_backward_sparse(q, k, v, do, 0.3, causal, ones, block=4),
                           orc.attention_backward(q, k, v, do, 0.3, causal), "QKV"):
            _close(a, b, 1e-12, f"sparse all-ones d{n} causal={causal}")


def pin_sparse_bruteforce(orc):
    q, k, v = _qkv(52, 2, 2, 11, 3)
    m = _mask_rand(53, 2, 2, 3)
    m[0, 0, 1, :] = 0  # a query block that sees nothing
    for causal in (False, True):
        o, lse = orc.attention_forward_sparse(q, k, v, 0.6, causal, m, block=4)
        for b in range(2):
            for h in range(2):
                n = 11
                qq, kk, vv = q[b, h].tolist(), k[b, h].tolist(), v[b, h].tolist()
                for i in range(n):
                    js = [j for j in range(n) if m[b, h, i // 4, j // 4] and (not causal or j <= i)]
                    if not js:
                        assert np.all(o[b, h, i] == 0) and lse[b, h, i] == -math.inf, "sparse empty row"
                        continue
                    s = {j: 0.6 * math.fsum(x * y for x, y in zip(qq[i], kk[j])) for j in js}
                    mx = max(s.values())
                    w = {j: math.exp(s[j] - mx) for j in js}
                    z = math.fsum(w.values())
                    _close(lse[b, h, i], mx + math.log(z), 1e-12, f"sparse brute LSE b={b} h={h} i={i}")
                    for c in range(3):
                        _close(o[b, h, i, c], math.fsum(w[j] * vv[j][c] for j in js) / z, 1e-12,
                               f"sparse brute O b={b} h={h} i={i}")


def pin_sparse_block_diagonal(orc):
    """A block-diagonal mask is attention inside each block, computed independently."""
    q, k, v = _qkv(54, 1, 2, 14, 4)
    do = _rng(55).standard_normal(q.shape)
    eye = np.broadcast_to(np.eye(4, dtype=np.uint8), (1, 2, 4, 4)).copy()
    for causal in (False, True):
        o, lse = orc.attention_forward_sparse(q, k, v, 0.5, causal, eye, block=4)
        g = orc.attention_backward_sparse(q, k, v, do, 0.5, causal, eye, block=4)
        for c0 in range(0, 14, 4):
            c1 = min(14, c0 + 4)
            sl = (slice(None), slice(None), slice(c0, c1))
            oc, lc = orc.attention_forward(q[sl], k[sl], v[sl], 0.5, causal)
            _close(o[sl], oc, 1e-13, f"block-diagonal O chunk {c0} causal={causal}")
            _close(lse[sl], lc, 1e-13, f"block-diagonal LSE chunk {c0}")
            gc = orc.attention_backward(q[sl], k[sl], v[sl], do[sl], 0.5, causal)
            for a, b, n in zip(g, gc, "QKV"):
                _close(a[sl], b, 1e-12, f"block-diagonal d{n} chunk {c0} causal={causal}")


def pin_sparse_torch_autograd(orc):
    import torch
    q, k, v = _qkv(56, 2, 2, 13, 5)
    do = _rng(57).standard_normal(q.shape)
    m = _mask_rand(58, 2, 2, 4)
    m[1, 1, 2, :] = 0
    vis = np.zeros((2, 2, 13, 13), dtype=bool)
    idx = np.arange(13) // 4
    for b in range(2):
        for h in range(2):
            vis[b, h] = m[b, h][idx[:, None], idx[None, :]].astype(bool)
    for causal in (False, True):
        allowed = vis & (np.tril(np.ones((13, 13), dtype=bool)) if causal else True)
        tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
        s = 0.4 * torch.matmul(tq, tk.transpose(-1, -2).contiguous())
        s = s.masked_fill(~torch.tensor(allowed), float("-inf"))
        rows = torch.tensor(allowed.any(axis=-1))
        p = torch.where(rows[..., None], torch.softmax(torch.where(rows[..., None], s, torch.zeros_like(s)), dim=-1)
                        * torch.tensor(allowed), torch.zeros_like(s))
        p = p / torch.where(rows[..., None], p.sum(-1, keepdim=True), torch.ones_like(p[..., :1]))
        out = torch.matmul(p, tv)
        (out * torch.tensor(do)).sum().backward()
        o, lse = orc.attention_forward_sparse(q, k, v, 0.4, causal, m, block=4)
        _close(o, out.detach().numpy(), 1e-12, f"sparse autograd O causal={causal}")
        dq, dk, dv = orc.attention_backward_sparse(q, k, v, do, 0.4, causal, m, block=4)
        _close(dq, tq.grad.numpy(), 1e-10, f"sparse autograd dQ causal={causal}")
        _close(dk, tk.grad.numpy(), 1e-10, f"sparse autograd dK causal={causal}")
        _close(dv, tv.grad.numpy(), 1e-10, f"sparse autograd dV causal={causal}")


def pin_sparse_finite_differences(orc):
    q, k, v = _qkv(59, 1, 1, 7, 3)
    do = _rng(60).standard_normal(q.shape)
    m = np.array([[[[1, 0], [1, 1]]]], dtype=np.uint8)
    for causal in (False, True):
        grads = orc.attention_backward_sparse(q, k, v, do, 0.45, causal, m, block=4)
        base = [q, k, v]
        h = 1e-6
        for which in range(3):
            num = np.zeros_like(base[which])
            for idx in np.ndindex(base[which].shape):
                loss = []
                for sgn in (1.0, -1.0):
                    xs = [x.copy() for x in base]
                    xs[which][idx] += sgn * h
                    o, _ = orc.attention_forward_sparse(*xs, 0.45, causal, m, block=4)
                    loss.append(np.sum(o * do))
                num[idx] = (loss[0] - loss[1]) / (2 * h)
            err = np.max(np.abs(num - grads[which])) / max(1.0, np.max(np.abs(num)))
            assert err < 1e-7, f"sparse finite differences grad {which} causal={causal}: {err:.2e}"


# ------------------------------------------------------------------ dropout
# Reading (the pages name dropout as fused, with no generator): O = (P * Z) V,
# Z = keep / (1 - p), keep_ij = [r_ij >= floor(p 2^32)], r_ij = word j & 3 of
# Philox4x32-10 with key = seed and counter (j >> 2, i, b H + h, offset).
def pin_philox_known_answers(orc):
    with open(os.path.join(GOLDEN, "philox_kat.json")) as f:
        g = json.load(f)
    for vec in g["vectors"]:
        ctr = [int(x, 16) for x in vec["counter"]]
        key = [int(x, 16) for x in vec["key"]]
        got = orc.philox4x32(*ctr, *key)
        assert [int(x) for x in got] == [int(x, 16) for x in vec["output"]], f"Philox KAT {vec['counter']}"


def _philox_scalar(c, k):
    """Philox4x32-10 on Python ints, written out separately from the oracle's array version."""
    c, k = list(c), list(k)
    for r in range(10):
        if r:
            k = [(k[0] + 0x9E3779B9) & 0xFFFFFFFF, (k[1] + 0xBB67AE85) & 0xFFFFFFFF]
        a, b = 0xD2511F53 * c[0], 0xCD9E8D57 * c[2]
        c = [(b >> 32) ^ c[1] ^ k[0], b & 0xFFFFFFFF, (a >> 32) ^ c[3] ^ k[1], a & 0xFFFFFFFF]
    return c


def pin_dropout_p0_is_dense(orc):
    q, k, v = _qkv(70, 2, 2, 17, 8)
    do = _rng(71).standard_normal(q.shape)
    for causal in (False, True):
        o, lse = orc.attention_forward(q, k, v, 0.3, causal)
        o2, lse2 = orc.attention_forward_dropout(q, k, v, 0.3, causal, 0.0, 1234, 5)
        _close(o2, o, 1e-13, f"dropout p=0 O causal={causal}")
        _close(lse2, lse, 1e-13, f"dropout p=0 LSE causal={causal}")
        for a, b, n in zip(orc.attention_backward_dropout(q, k, v, do, 0.3, causal, 0.0, 1234, 5),
                           orc.attention_backward(q, k, v, do, 0.3, causal), "QKV"):
            _close(a, b, 1e-12, f"dropout p=0 d{n} causal={causal}")


def pin_dropout_bruteforce(orc):
    """Scalar loops: Philox on ints, the keep test, softmax, (P * Z) V."""
    B, H, N, d = 1, 2, 9, 3
    q, k, v = _qkv(72, B, H, N, d)
    p, seed, offset = 0.35, 0xDEADBEEF12345, 7
    t = math.floor(p * 2 ** 32)
    for causal in (False, True):
        o, lse = orc.attention_forward_dropout(q, k, v, 0.5, causal, p, seed, offset)
        for h in range(H):
            for i in range(N):
                js = [j for j in range(N) if not causal or j <= i]
                s = {j: 0.5 * math.fsum(x * y for x, y in zip(q[0, h, i], k[0, h, j])) for j in js}
                mx = max(s.values())
                w = {j: math.exp(s[j] - mx) for j in js}
                z = math.fsum(w.values())
                _close(lse[0, h, i], mx + math.log(z), 1e-12, "dropout LSE is the undropped one")
                keep = {j: _philox_scalar((j >> 2, i, h, offset), (seed & 0xFFFFFFFF, seed >> 32))[j & 3] >= t
                        for j in js}
                for c in range(d):
                    want = math.fsum(w[j] * v[0, h, j, c] for j in js if keep[j]) / z / (1 - p)
                    _close(o[0, h, i, c], want, 1e-12, f"dropout brute O h={h} i={i} causal={causal}")


def pin_dropout_keep_rate(orc):
    """keep is Bernoulli(1 - p) per entry; streams differ across heads and offsets, repeat for the same ones."""
    for p in (0.1, 0.5, 0.9):
        m = orc.dropout_keep(256, 256, 3, p, 99, 0)
        n = m.size
        want = 1.0 - orc.dropout_threshold(p) / 2 ** 32
        sd = math.sqrt(n * want * (1 - want))
        assert abs(m.sum() - n * want) < 5 * sd, f"keep rate for p={p}: {m.mean():.4f} vs {want:.4f}"
    a = orc.dropout_keep(64, 64, 3, 0.5, 99, 0)
    assert np.array_equal(a, orc.dropout_keep(64, 64, 3, 0.5, 99, 0)), "same stream, same mask"
    for other in (orc.dropout_keep(64, 64, 4, 0.5, 99, 0), orc.dropout_keep(64, 64, 3, 0.5, 99, 1),
                  orc.dropout_keep(64, 64, 3, 0.5, 100, 0)):
        assert 0.3 < np.mean(a != other) < 0.7, "independent streams for another head / offset / seed"


def pin_dropout_unbiased(orc):
    """E over seeds of O with dropout is the dense O (mean of 400 draws within 6 standard errors)."""
    q, k, v = _qkv(73, 1, 1, 6, 4)
    o_dense, _ = orc.attention_forward(q, k, v, 0.5, False)
    draws = np.stack([orc.attention_forward_dropout(q, k, v, 0.5, False, 0.3, s, 0)[0] for s in range(400)])
    mean, se = draws.mean(axis=0), draws.std(axis=0) / math.sqrt(len(draws))
    assert np.all(np.abs(mean - o_dense) <= 6 * se + 1e-12), "dropout output is unbiased"


def pin_dropout_torch_autograd(orc):
    import torch
    q, k, v = _qkv(74, 2, 2, 11, 5)
    do = _rng(75).standard_normal(q.shape)
    p, seed, offset = 0.25, 42, 3
    z = np.stack([np.stack([orc.dropout_keep(11, 11, b * 2 + h, p, seed, offset) for h in range(2)])
                  for b in range(2)]) / (1 - p)
    for causal in (False, True):
        tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
        s = 0.4 * torch.matmul(tq, tk.transpose(-1, -2).contiguous())
        if causal:
            s = s.masked_fill(torch.ones(11, 11, dtype=torch.bool).triu(1), float("-inf"))
        out = torch.matmul(torch.softmax(s, dim=-1) * torch.tensor(z), tv)
        (out * torch.tensor(do)).sum().backward()
        o, _ = orc.attention_forward_dropout(q, k, v, 0.4, causal, p, seed, offset)
        _close(o, out.detach().numpy(), 1e-12, f"dropout autograd O causal={causal}")
        dq, dk, dv = orc.attention_backward_dropout(q, k, v, do, 0.4, causal, p, seed, offset)
        _close(dq, tq.grad.numpy(), 1e-10, f"dropout autograd dQ causal={causal}")
        _close(dk, tk.grad.numpy(), 1e-10, f"dropout autograd dK causal={causal}")
        _close(dv, tv.grad.numpy(), 1e-10, f"dropout autograd dV causal={causal}")


def pin_dropout_finite_differences(orc):
    q, k, v = _qkv(76, 1, 1, 6, 3)
    do = _rng(77).standard_normal(q.shape)
    for causal in (False, True):
        grads = orc.attention_backward_dropout(q, k, v, do, 0.45, causal, 0.3, 11, 2)
        base = [q, k, v]
        h = 1e-6
        for which in range(3):
            num = np.zeros_like(base[which])
            for idx in np.ndindex(base[which].shape):
                loss = []
                for sgn in (1.0, -1.0):
                    xs = [x.copy() for x in base]
                    xs[which][idx] += sgn * h
                    o, _ = orc.attention_forward_dropout(*xs, 0.45, causal, 0.3, 11, 2)
                    loss.append(np.sum(o * do))
                num[idx] = (loss[0] - loss[1]) / (2 * h)
            err = np.max(np.abs(num - grads[which])) / max(1.0, np.max(np.abs(num)))
            assert err < 1e-7, f"dropout finite differences grad {which} causal={causal}: {err:.2e}"


def pin_sparse_rows_match_full(orc):
    """The per-row sparse sampler equals rows of the full sparse oracle (random masks, an empty block row)."""
    r = _rng(61)
    q, k, v = _qkv(61, 1, 2, 23, 3)
    for causal in (False, True):
        m = (r.random((1, 2, 6, 6)) < 0.5).astype(np.uint8)
        m[0, 1, 2, :] = 0
        o, lse = orc.attention_forward_sparse(q, k, v, 0.7, causal, m, block=4)
        for h in range(2):
            rows = [0, 5, 8, 9, 17, 22]
            so, sl = orc.attention_forward_sparse_rows(q, k, v, 0.7, causal, m, 0, h, rows, block=4)
            _close(so, o[0, h, rows], 1e-13, f"sparse rows O causal={causal}")
            assert np.array_equal(np.isinf(sl), np.isinf(lse[0, h, rows])), "sparse rows: empty rows differ"
            fin = ~np.isinf(sl)
            _close(sl[fin], lse[0, h, rows][fin], 1e-13, f"sparse rows LSE causal={causal}")


# ------------------------------------------------------------------ fp8 inputs
# Reading (the pages name lower-precision paths, no format): q, k, v are OCP
# E4M3 codes, each tensor with one dequantisation factor; the result is exact
# attention on the dequantised values.
def _e4m3_fixture():
    with open(os.path.join(GOLDEN, "e4m3_values.json")) as f:
        return {int(c, 16): (math.nan if v is None else v) for c, v in json.load(f)["values"].items()}


def pin_e4m3_table(orc):
    for code, want in _e4m3_fixture().items():
        got = float(orc.e4m3_decode(np.array([code], dtype=np.uint8))[0])
        if math.isnan(want):
            assert math.isnan(got), f"e4m3 code {code:#04x} should be NaN, got {got}"
        else:
            assert got == want and math.copysign(1.0, got) == math.copysign(1.0, want), \
                f"e4m3 code {code:#04x}: {got} != {want}"


def pin_e4m3_library(orc):
    """All 256 codes against torch's float8_e4m3fn (the same OCP format)."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = orc.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref)), "e4m3 NaN codes differ from torch"
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok]), "e4m3 values differ from torch"


def pin_e4m3_order(orc):
    pos = orc.e4m3_decode(np.arange(127, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0), "codes 0x00..0x7e must increase strictly"
    neg = orc.e4m3_decode(np.arange(128, 255, dtype=np.uint8))
    assert np.array_equal(neg, -pos), "the sign bit must negate"


def pin_fp8_bruteforce(orc):
    """Scalar loops over fixture codes with three different dequantisation factors."""
    table = {c: v for c, v in _e4m3_fixture().items() if not math.isnan(v) and abs(v) <= 3.0}
    codes = np.array(sorted(table), dtype=np.uint8)
    r = _rng(71)
    for causal, (N, d) in ((False, (5, 3)), (True, (6, 4))):
        q8, k8, v8 = (codes[r.integers(0, len(codes), (1, 2, N, d))] for _ in range(3))
        dq, dk, dv, scale = 0.75, 1.25, 0.5, 0.4
        o, lse = orc.attention_forward_fp8(q8, k8, v8, dq, dk, dv, scale, causal)
        for h in range(2):
            q = [[dq * table[int(x)] for x in row] for row in q8[0, h]]
            k = [[dk * table[int(x)] for x in row] for row in k8[0, h]]
            v = [[dv * table[int(x)] for x in row] for row in v8[0, h]]
            bo, bl = _brute_head(q, k, v, scale, causal)
            _close(o[0, h], bo, 1e-12, f"fp8 brute O causal={causal}")
            _close(lse[0, h], bl, 1e-12, f"fp8 brute LSE causal={causal}")


def pin_fp8_descale_invariances(orc):
    r = _rng(72)
    q8, k8, v8 = (r.integers(0, 127, (1, 2, 9, 8)).astype(np.uint8) | (r.integers(0, 2, (1, 2, 9, 8)) * 128).astype(np.uint8)
                  for _ in range(3))
    q8[q8 & 127 == 127] = 0x38  # no NaN codes
    k8[k8 & 127 == 127] = 0x38
    v8[v8 & 127 == 127] = 0x38
    base_o, base_l = orc.attention_forward_fp8(q8, k8, v8, 0.01, 0.02, 0.5, 0.3, True)
    o, l = orc.attention_forward_fp8(q8, k8, v8, 0.01, 0.02, 1.0, 0.3, True)
    _close(o, 2.0 * base_o, 1e-12, "O is linear in descale_v")
    _close(l, base_l, 1e-12, "LSE does not see descale_v")
    o, l = orc.attention_forward_fp8(q8, k8, v8, 0.04, 0.02, 0.5, 0.075, True)
    _close(o, base_o, 1e-12, "descale_q * 4 with scale / 4")
    _close(l, base_l, 1e-12, "descale_q * 4 with scale / 4 (LSE)")
    ones = np.full_like(v8, 0x38)
    o, _ = orc.attention_forward_fp8(q8, k8, ones, 0.01, 0.02, 0.5, 0.3, False)
    _close(o, np.full(o.shape, 0.5), 1e-14, "constant V = descale_v * 1")


# E5M2 codes (same specification) as a second input format: IEEE-like, with
# infinities at exponent field 31.
def _e5m2_fixture():
    def val(v):
        return math.nan if v is None else float(v)  # "inf" / "-inf" strings parse as floats
    with open(os.path.join(GOLDEN, "e5m2_values.json")) as f:
        return {int(c, 16): val(v) for c, v in json.load(f)["values"].items()}


def pin_e5m2_table(orc):
    for code, want in _e5m2_fixture().items():
        got = float(orc.e5m2_decode(np.array([code], dtype=np.uint8))[0])
        if math.isnan(want):
            assert math.isnan(got), f"e5m2 code {code:#04x} should be NaN, got {got}"
        else:
            assert got == want and math.copysign(1.0, got) == math.copysign(1.0, want), \
                f"e5m2 code {code:#04x}: {got} != {want}"


def pin_e5m2_library(orc):
    """All 256 codes against torch's float8_e5m2 (the same OCP format)."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e5m2).to(torch.float64).numpy()
    got = orc.e5m2_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref)), "e5m2 NaN codes differ from torch"
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok]), "e5m2 values differ from torch"


def pin_e5m2_order(orc):
    """Codes 0x00..0x7c increase strictly up to +inf; 0x7d..0x7f are NaN; the
    sign bit negates; each binade holds four codes that double across it."""
    pos = orc.e5m2_decode(np.arange(125, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0) and pos[-1] == np.inf, "codes 0x00..0x7c must increase to +inf"
    assert np.all(np.isnan(orc.e5m2_decode(np.arange(125, 128, dtype=np.uint8)))), "0x7d..0x7f are NaN"
    neg = orc.e5m2_decode(np.arange(128, 253, dtype=np.uint8))
    assert np.array_equal(neg, -pos), "the sign bit must negate"
    normal = pos[4:124]
    assert np.array_equal(normal[4:], 2.0 * normal[:-4]), "a step of four codes doubles a normal value"
    sub = pos[:4]
    assert np.array_equal(sub, np.arange(4) * sub[1]) and sub[1] == pos[4] / 4, "subnormals are even steps of 2^-16"


def pin_fp8_e5m2_bruteforce(orc):
    """Scalar loops over E5M2 fixture codes with three dequantisation factors."""
    table = {c: v for c, v in _e5m2_fixture().items() if math.isfinite(v) and abs(v) <= 3.0}
    codes = np.array(sorted(table), dtype=np.uint8)
    r = _rng(73)
    for causal, (N, d) in ((False, (5, 3)), (True, (6, 4))):
        q8, k8, v8 = (codes[r.integers(0, len(codes), (1, 2, N, d))] for _ in range(3))
        dq, dk, dv, scale = 0.5, 1.5, 0.25, 0.7
        o, lse = orc.attention_forward_fp8(q8, k8, v8, dq, dk, dv, scale, causal, fmt="e5m2")
        for h in range(2):
            q = [[dq * table[int(x)] for x in row] for row in q8[0, h]]
            k = [[dk * table[int(x)] for x in row] for row in k8[0, h]]
            v = [[dv * table[int(x)] for x in row] for row in v8[0, h]]
            bo, bl = _brute_head(q, k, v, scale, causal)
            _close(o[0, h], bo, 1e-12, f"fp8 e5m2 brute O causal={causal}")
            _close(lse[0, h], bl, 1e-12, f"fp8 e5m2 brute LSE causal={causal}")


def pin_fp8_formats_agree(orc):
    """Values that both formats hold exactly (powers of two in 2^-6..2^8 and
    their 1.5 multiples) give the same attention through either decoder."""
    r = _rng(74)
    vals = np.array([s * m * 2.0 ** e for s in (1, -1) for m in (1.0, 1.5) for e in range(-6, 6)])
    x = vals[r.integers(0, len(vals), (3, 1, 2, 11, 8))]
    enc4 = {float(v): c for c, v in enumerate(orc.e4m3_decode(np.arange(256, dtype=np.uint8))) if np.isfinite(v)}
    enc5 = {float(v): c for c, v in enumerate(orc.e5m2_decode(np.arange(256, dtype=np.uint8))) if np.isfinite(v)}
    c4 = np.vectorize(lambda t: enc4[float(t)])(x).astype(np.uint8)
    c5 = np.vectorize(lambda t: enc5[float(t)])(x).astype(np.uint8)
    for causal in (False, True):
        o4, l4 = orc.attention_forward_fp8(c4[0], c4[1], c4[2], 0.3, 0.2, 2.0, 0.5, causal, fmt="e4m3")
        o5, l5 = orc.attention_forward_fp8(c5[0], c5[1], c5[2], 0.3, 0.2, 2.0, 0.5, causal, fmt="e5m2")
        _close(o5, o4, 1e-14, f"formats agree O causal={causal}")
        _close(l5, l4, 1e-14, f"formats agree LSE causal={causal}")


ALL_PINS = [pin_bruteforce_forward, pin_worked_example, pin_probability_rows, pin_constant_v,
            pin_q_zero, pin_causal_row0_and_n1, pin_shift_invariance, pin_permutation,
            pin_online_recurrence, pin_scipy_logsumexp, pin_torch_autograd,
            pin_finite_differences, pin_backward_invariants,
            pin_kv_reduces_to_square, pin_kv_worked_example, pin_kv_bruteforce, pin_kv_decode_and_empty,
            pin_kv_padding_invariance, pin_kv_torch_autograd, pin_kv_finite_differences,
            pin_sparse_all_ones_is_dense, pin_sparse_bruteforce, pin_sparse_block_diagonal,
            pin_sparse_torch_autograd, pin_sparse_finite_differences, pin_sparse_rows_match_full,
            pin_philox_known_answers, pin_dropout_p0_is_dense, pin_dropout_bruteforce, pin_dropout_keep_rate,
            pin_dropout_unbiased, pin_dropout_torch_autograd, pin_dropout_finite_differences,
            pin_e4m3_table, pin_e4m3_library, pin_e4m3_order, pin_fp8_bruteforce, pin_fp8_descale_invariances,
            pin_e5m2_table, pin_e5m2_library, pin_e5m2_order, pin_fp8_e5m2_bruteforce, pin_fp8_formats_agree]
