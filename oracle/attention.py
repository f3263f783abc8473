"""Plain fp64 CPU oracle for exact attention and its gradients.

TEST INFRASTRUCTURE ONLY.  This module is imported by the tests, by the smoke
check and by the benchmark's CPU-baseline leg, never by the library.  It shares
no code with the HIP path; both read their inputs from the seeded generators in
exact_io_aware_51_amd.workloads, which hold no attention arithmetic.

What is computed (all in float64, one (batch, head) slice at a time):

* Forward -- the definition softmax(Q K^T / sqrt(d)) V with the optional causal
  mask ("How Flash Attention Works: Tiling, Softmax, GPU I/O", section "How
  Flash Attention Works: The Exact-Attention Idea"; "attn-flash-equivalence",
  section "Standard attention I/O is the bottleneck", which lists the three
  materialising steps S = QK^T/sqrt(d_k), P = softmax(S), O = P V).  The score
  matrix S and the probability matrix P are materialised, exactly as the naive
  pipeline does; this is the plain definition, not the tiled algorithm.
  The scale is an argument (the kernels receive it as an fp32 number).
  Causal mask: key j is visible to query i iff j <= i.
  Side output: the per-row log-sum-exp LSE_i = ln sum_j exp(S_ij), i.e. the
  "compact per-row statistics" the backward pass needs ("How Flash Attention
  Works", section "The Backward Pass: Recomputation Instead of Stored
  Activations"), folded into one number per row (running max m plus ln of the
  normaliser l).

* Backward -- the pages give no formulas; this is the chain rule applied to the
  same definition, with P recomputed from S:
      dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij,
      dS = P * (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q.

For long sequences the forward materialises S and P in panels of whole rows;
every row is still formed and normalised in one piece, and rows never interact,
so the panel size changes no arithmetic.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    """Accept numpy arrays or torch tensors (any float dtype) and return float64 numpy."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch  # local: only when torch tensors are passed
        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _scores(q, k, scale, causal, row0=0):
    """Rows row0 .. row0+len(q)-1 of S = scale * q k^T, masked entries = -inf."""
    s = scale * (q @ k.T)
    if causal:
        rows = np.arange(row0, row0 + q.shape[0])[:, None]
        cols = np.arange(k.shape[0])[None, :]
        s = np.where(cols > rows, -np.inf, s)
    return s


def _softmax_rows(s):
    """Row softmax of s and each row's log-sum-exp.

    The row max is subtracted before exponentiating; it cancels in the ratio
    and only keeps exp() in range.
    """
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    l = np.sum(e, axis=1, keepdims=True)
    return e / l, (m + np.log(l))[:, 0]


def attention_probs(q, k, scale, causal):
    """P = softmax(scale * q k^T [+ mask]) for one head: q, k are [N, d]."""
    q, k = _f64(q), _f64(k)
    p, _ = _softmax_rows(_scores(q, k, scale, causal))
    return p


def _forward_head(q, k, v, scale, causal, panel_rows):
    n = q.shape[0]
    o = np.empty((n, v.shape[1]))
    lse = np.empty(n)
    for r0 in range(0, n, panel_rows):
        r1 = min(n, r0 + panel_rows)
        p, lse[r0:r1] = _softmax_rows(_scores(q[r0:r1], k, scale, causal, row0=r0))
        o[r0:r1] = p @ v
    return o, lse


def attention_forward(q, k, v, scale, causal, panel_rows=2048):
    """O = softmax(scale * Q K^T [+ causal mask]) V and LSE, for [B, H, N, d] inputs.

    Returns (O [B,H,N,d] float64, LSE [B,H,N] float64, natural log).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, _ = q.shape
    o = np.empty(q.shape[:3] + (v.shape[3],))
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = _forward_head(q[b, h], k[b, h], v[b, h], scale, causal, panel_rows)
    return o, lse


def attention_forward_rows(q, k, v, scale, causal, b, h, rows):
    """O and LSE for selected query rows of one (b, h) slice (for spot checks at full size).

    Row i needs only q_i and all keys/values: O_i = sum_j P_ij v_j with P_i = softmax(S_i).
    """
    qh, kh, vh = _f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h])
    rows = [int(i) for i in rows]
    o = np.empty((len(rows), vh.shape[1]))
    lse = np.empty(len(rows))
    for t, i in enumerate(rows):
        p, lse[t:t + 1] = _softmax_rows(_scores(qh[i:i + 1], kh, scale, causal, row0=i))
        o[t] = (p @ vh)[0]
    return o, lse


def attention_forward_panel(q, k, v, scale, causal, b, h, r0, r1):
    """O and LSE for the contiguous query rows r0 .. r1-1 of one (b, h) slice.

    The same definition as attention_forward on whole rows (rows never
    interact), for checking long sequences a panel at a time.
    """
    qh, kh, vh = _f64(q[b, h, r0:r1]), _f64(k[b, h]), _f64(v[b, h])
    p, lse = _softmax_rows(_scores(qh, kh, scale, causal, row0=r0))
    return p @ vh, lse


def _backward_terms(q, k, v, do, scale, causal):
    """P, dP = dO V^T, D_i = sum_j P_ij dP_ij and dS = P * (dP - D) for one head."""
    p, _ = _softmax_rows(_scores(q, k, scale, causal))
    dp = do @ v.T
    dsum = np.sum(p * dp, axis=1, keepdims=True)
    ds = p * (dp - dsum)
    return p, dp, dsum[:, 0], ds


def _backward_head(q, k, v, do, scale, causal):
    p, _, _, ds = _backward_terms(q, k, v, do, scale, causal)
    dv = p.T @ do
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def attention_backward_terms(q, k, v, do, scale, causal, b, h):
    """The intermediate matrices of one (b, h) slice's backward pass:
    (P, dP, D, dS), each N x N except D (length N).  For error models of
    implementations that round P or dS before multiplying."""
    return _backward_terms(_f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h]), _f64(do[b, h]), scale, causal)


def attention_backward(q, k, v, do, scale, causal, heads=None):
    """dQ, dK, dV of L = sum(dO * O) for [B, H, N, d] inputs (float64).

    heads: optional list of (b, h) pairs; only those slices are computed and the
    result is a dict {(b, h): (dq, dk, dv)}.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    if heads is not None:
        return {(b, h): _backward_head(q[b, h], k[b, h], v[b, h], do[b, h], scale, causal)
                for (b, h) in heads}
    dq, dk, dv = np.empty(q.shape), np.empty(k.shape), np.empty(v.shape)
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            dq[b, h], dk[b, h], dv[b, h] = _backward_head(q[b, h], k[b, h], v[b, h], do[b, h], scale, causal)
    return dq, dk, dv


def attention_backward_rows(q, k, v, do, scale, causal, b, h, rows):
    """dQ for selected query rows of one (b, h) slice.

    Row i of dQ needs only row i of P and dP: dQ_i = scale * sum_j P_ij (dP_ij - D_i) k_j.
    """
    qh, kh, vh, doh = (_f64(x[b, h]) for x in (q, k, v, do))
    out = np.empty((len(rows), kh.shape[1]))
    for t, i in enumerate(list(rows)):
        p, _ = _softmax_rows(_scores(qh[i:i + 1], kh, scale, causal, row0=i))
        dp = doh[i:i + 1] @ vh.T
        ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
        out[t] = scale * (ds @ kh)[0]
    return out


# ---------------------------------------------------------------------------
# Queries and keys of different counts, and padded batches.
#
# The pages tie the causal mask to autoregressive decoding, and apply causal
# masking and padding tile by tile, with boundary tiles cut by the mask
# ("How Flash Attention Works: Tiling, Softmax, GPU I/O", sections "How Flash
# Attention Works: The Exact-Attention Idea" and "Tiling Q, K, and V for Fast
# On-Chip Memory").  They fix neither the alignment of a causal mask when the
# query count differs from the key count nor what a padded row outputs; the
# readings taken here:
#   * sequence b has lq_b real queries and lk_b real keys (lengths outside
#     [0, Nq] / [0, Nk] are clamped into them); rows at or past a length are
#     padding;
#   * the lq_b queries are the last lq_b positions of the lk_b-key sequence
#     (decoding with a cache of earlier keys), so under the causal mask query i
#     sees key j iff j <= i + (lk_b - lq_b);
#   * a query that sees no key, and every padding row, outputs O = 0 and
#     LSE = -inf, and contributes nothing to any gradient; padding rows of
#     dQ, dK and dV are 0.
# ---------------------------------------------------------------------------


def _lengths(lens, B, n):
    """Per-sequence lengths clamped into [0, n] (all n when lens is None)."""
    if lens is None:
        return [n] * B
    return [min(max(int(x), 0), n) for x in np.asarray(lens).reshape(-1)[:B]]


def _scores_kv(q, k, scale, causal, off):
    """S = scale * q k^T for one sequence; query i may see key j iff j <= i + off (causal)."""
    s = scale * (q @ k.T)
    if causal:
        rows = np.arange(q.shape[0])[:, None] + off
        cols = np.arange(k.shape[0])[None, :]
        s = np.where(cols > rows, -np.inf, s)
    return s


def _softmax_rows_kv(s):
    """Row softmax and LSE where a row may have no visible key (P = 0, LSE = -inf)."""
    n = s.shape[0]
    if s.shape[1] == 0:
        return np.zeros_like(s), np.full(n, -np.inf)
    m = np.max(s, axis=1)
    seen = np.isfinite(m)
    m0 = np.where(seen, m, 0.0)[:, None]
    e = np.exp(s - m0)  # exp(-inf) = 0 for the masked entries
    l = np.sum(e, axis=1)
    p = np.zeros_like(e)
    p[seen] = e[seen] / l[seen, None]
    lse = np.full(n, -np.inf)
    lse[seen] = m[seen] + np.log(l[seen])
    return p, lse


def attention_forward_kv(q, k, v, scale, causal, seqlens_q=None, seqlens_k=None):
    """O and LSE for q [B,H,Nq,d], k and v [B,H,Nk,d] under the readings above.

    Returns (O [B,H,Nq,d] float64, LSE [B,H,Nq] float64, natural log).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Nq, _ = q.shape
    Nk = k.shape[2]
    lq, lk = _lengths(seqlens_q, B, Nq), _lengths(seqlens_k, B, Nk)
    o = np.zeros(q.shape[:3] + (v.shape[3],))
    lse = np.full((B, H, Nq), -np.inf)
    for b in range(B):
        off = lk[b] - lq[b]
        for h in range(H):
            p, lse[b, h, :lq[b]] = _softmax_rows_kv(_scores_kv(q[b, h, :lq[b]], k[b, h, :lk[b]], scale, causal, off))
            o[b, h, :lq[b]] = p @ v[b, h, :lk[b]]
    return o, lse


def attention_backward_kv(q, k, v, do, scale, causal, seqlens_q=None, seqlens_k=None):
    """dQ, dK, dV of L = sum(dO * O) for the forward above (float64).

    Per sequence, on its real rows only: dV = P^T dO, dP = dO V^T,
    D_i = sum_j P_ij dP_ij, dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, Nq, _ = q.shape
    Nk = k.shape[2]
    lq, lk = _lengths(seqlens_q, B, Nq), _lengths(seqlens_k, B, Nk)
    dq, dk, dv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    for b in range(B):
        a, c, off = lq[b], lk[b], lk[b] - lq[b]
        for h in range(H):
            qh, kh, vh, doh = q[b, h, :a], k[b, h, :c], v[b, h, :c], do[b, h, :a]
            p, _ = _softmax_rows_kv(_scores_kv(qh, kh, scale, causal, off))
            dv[b, h, :c] = p.T @ doh
            dp = doh @ vh.T
            ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
            dq[b, h, :a] = scale * (ds @ kh)
            dk[b, h, :c] = scale * (ds.T @ qh)
    return dq, dk, dv


# ---------------------------------------------------------------------------
# Block-sparse attention.  The pages name a block-sparse extension studied
# alongside the dense algorithm as a separate configuration ("FlashAttention"
# glossary entry, its definition) without fixing a mask format; the reading
# taken here: a 0/1 mask
# of shape [B, H, ceil(N / block), ceil(N / block)] removes every score of a
# (query block, key block) pair whose entry is 0, on top of the causal mask.
# Rows that see no key output O = 0 and LSE = -inf, as above.
# ---------------------------------------------------------------------------


def _block_visible(mask_bh, n, block):
    """Elementwise n x n visibility from one head's block mask."""
    idx = np.arange(n) // block
    return np.asarray(mask_bh, dtype=bool)[idx[:, None], idx[None, :]]


def attention_forward_sparse(q, k, v, scale, causal, block_mask, block=128):
    """O and LSE for [B,H,N,d] inputs with a block mask [B, H, nb, nb] (nonzero = keep)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, _ = q.shape
    bm = np.asarray(block_mask)
    o = np.zeros(q.shape[:3] + (v.shape[3],))
    lse = np.full((B, H, N), -np.inf)
    for b in range(B):
        for h in range(H):
            s = _scores_kv(q[b, h], k[b, h], scale, causal, 0)
            s = np.where(_block_visible(bm[b, h], N, block), s, -np.inf)
            p, lse[b, h] = _softmax_rows_kv(s)
            o[b, h] = p @ v[b, h]
    return o, lse


def attention_forward_sparse_rows(q, k, v, scale, causal, block_mask, b, h, rows, block=128):
    """O and LSE for selected query rows of one (b, h) slice under a block mask (spot checks at any size).

    Row i sees key j iff its mask block (i // block, j // block) is kept and,
    causal, j <= i; the row is the softmax over those keys alone.
    """
    qh, kh, vh = _f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h])
    n = kh.shape[0]
    bm = np.asarray(block_mask)[b, h].astype(bool)
    keys = np.arange(n)
    o = np.zeros((len(rows), vh.shape[1]))
    lse = np.full(len(rows), -np.inf)
    for t, i in enumerate(int(r) for r in rows):
        seen = bm[i // block, keys // block]
        if causal:
            seen &= keys <= i
        if not seen.any():
            continue
        s = scale * (kh[seen] @ qh[i])
        m = np.max(s)
        e = np.exp(s - m)
        lse[t] = m + np.log(np.sum(e))
        o[t] = (e / np.sum(e)) @ vh[seen]
    return o, lse


def attention_backward_sparse(q, k, v, do, scale, causal, block_mask, block=128):
    """dQ, dK, dV of L = sum(dO * O) for the block-sparse forward above."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, N, _ = q.shape
    bm = np.asarray(block_mask)
    dq, dk, dv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    for b in range(B):
        for h in range(H):
            s = _scores_kv(q[b, h], k[b, h], scale, causal, 0)
            s = np.where(_block_visible(bm[b, h], N, block), s, -np.inf)
            p, _ = _softmax_rows_kv(s)
            dv[b, h] = p.T @ do[b, h]
            dpm = do[b, h] @ v[b, h].T
            dsm = p * (dpm - np.sum(p * dpm, axis=1, keepdims=True))
            dq[b, h] = scale * (dsm @ k[b, h])
            dk[b, h] = scale * (dsm.T @ q[b, h])
    return dq, dk, dv


# ---------------------------------------------------------------------------
# Dropout on the attention weights.  The pages list dropout among the work the
# fused kernel does ("How Flash Attention Works", section "Kernel Fusion and
# Incremental Output Accumulation") without a random-number scheme; the
# reading taken here:
#   * O = (P * Z) V with Z_ij = keep_ij / (1 - p); P is the softmax of the
#     scores (its normaliser and the LSE do not see the dropout);
#   * keep_ij = [r_ij >= floor(p * 2^32)] for a 32-bit word r_ij of the
#     counter-based generator Philox4x32-10 (Salmon, Moraes, Dror and Shaw,
#     "Parallel random numbers: as easy as 1, 2, 3", SC 2011): key = the 64-bit
#     seed (low word first), counter = (j >> 2, i, b * H + h, offset), and
#     r_ij is output word j & 3;
#   * the backward is the chain rule through Z: dV = (P * Z)^T dO,
#     dP = (dO V^T) * Z, D_i = sum_j P_ij dP_ij (= sum_c dO_ic O_ic),
#     dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q.
# ---------------------------------------------------------------------------

_PHILOX_M = (0xD2511F53, 0xCD9E8D57)  # round multipliers
_PHILOX_W = (0x9E3779B9, 0xBB67AE85)  # key increments (golden ratio, sqrt(3) - 1)


def philox4x32(c0, c1, c2, c3, k0, k1, rounds=10):
    """Philox4x32-R on arrays of uint32 counters with a uint32 key pair; returns four uint32 arrays.

    One round: (hi0, lo0) = M0 * c0, (hi1, lo1) = M1 * c2 (64-bit products);
    c <- (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); the key gains (W0, W1)
    between rounds.
    """
    m = np.uint64(0xFFFFFFFF)
    c = [np.asarray(x, dtype=np.uint64) & m for x in (c0, c1, c2, c3)]
    k0, k1 = np.uint64(k0) & m, np.uint64(k1) & m
    for r in range(rounds):
        if r:
            k0 = (k0 + np.uint64(_PHILOX_W[0])) & m
            k1 = (k1 + np.uint64(_PHILOX_W[1])) & m
        p0 = np.uint64(_PHILOX_M[0]) * c[0]
        p1 = np.uint64(_PHILOX_M[1]) * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & m
        hi1, lo1 = p1 >> np.uint64(32), p1 & m
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
    return tuple(x.astype(np.uint32) for x in c)


def dropout_threshold(p):
    """keep iff the 32-bit word is >= this (p in [0, 1))."""
    return int(np.floor(float(p) * 4294967296.0))


def dropout_keep(n_q, n_k, bh, p, seed, offset):
    """Boolean [n_q, n_k] keep mask of one (b, h) slice."""
    i = np.arange(n_q, dtype=np.uint64)[:, None] * np.ones((1, n_k), dtype=np.uint64)
    j = np.ones((n_q, 1), dtype=np.uint64) * np.arange(n_k, dtype=np.uint64)[None, :]
    seed = int(seed)
    words = philox4x32(j >> np.uint64(2), i, np.full(i.shape, bh, dtype=np.uint64),
                       np.full(i.shape, int(offset) & 0xFFFFFFFF, dtype=np.uint64),
                       seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    sel = (j & np.uint64(3)).astype(np.int64)
    r = np.choose(sel, words)
    return r >= np.uint32(dropout_threshold(p))


def attention_forward_dropout(q, k, v, scale, causal, p, seed, offset):
    """O = (P * Z) V and the (undropped) LSE for [B, H, N, d] inputs."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, _ = q.shape
    o = np.empty(q.shape[:3] + (v.shape[3],))
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            pr, lse[b, h] = _softmax_rows_kv(_scores_kv(q[b, h], k[b, h], scale, causal, 0))
            z = dropout_keep(N, N, b * H + h, p, seed, offset) / (1.0 - p)
            o[b, h] = (pr * z) @ v[b, h]
    return o, lse


def attention_backward_dropout(q, k, v, do, scale, causal, p, seed, offset):
    """dQ, dK, dV of L = sum(dO * O) for the dropout forward above."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, N, _ = q.shape
    dq, dk, dv = np.empty(q.shape), np.empty(k.shape), np.empty(v.shape)
    for b in range(B):
        for h in range(H):
            pr, _ = _softmax_rows_kv(_scores_kv(q[b, h], k[b, h], scale, causal, 0))
            z = dropout_keep(N, N, b * H + h, p, seed, offset) / (1.0 - p)
            dv[b, h] = (pr * z).T @ do[b, h]
            dpz = (do[b, h] @ v[b, h].T) * z
            dsz = pr * (dpz - np.sum(pr * dpz, axis=1, keepdims=True))
            dq[b, h] = scale * (dsz @ k[b, h])
            dk[b, h] = scale * (dsz.T @ q[b, h])
    return dq, dk, dv


# ---------------------------------------------------------------------------
# 8-bit floating-point inputs.  The pages say FlashAttention 3 adds
# lower-precision paths where the GPU supports them ("How Flash Attention
# Works", section "FlashAttention 1 vs 2 vs 3") and fix no format or scaling.
# The reading taken here:
#   * q, k and v hold OCP E4M3 codes ("OCP 8-bit Floating Point Specification
#     (OFP8)", revision 1.0, 2023): one sign bit, four exponent bits with bias
#     7, three mantissa bits; exponent field 0 encodes the subnormals
#     m / 8 * 2^-6; the codes with all exponent and mantissa bits set are NaN;
#     there are no infinities.  Or all three hold E5M2 codes of the same
#     specification (decoded by e5m2_decode below);
#   * each tensor carries one real dequantisation factor, so the attention
#     inputs are descale_q * E(q), descale_k * E(k), descale_v * E(v);
#   * the result is the plain definition on those values: exact attention
#     and its LSE, computed here in float64.
# ---------------------------------------------------------------------------

def e4m3_decode(codes):
    """float64 values of uint8 OCP E4M3 codes (any array shape)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >= 128, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    return np.where((c & 127) == 127, np.nan, sign * mag)


def e5m2_decode(codes):
    """float64 values of uint8 OCP E5M2 codes (any array shape).

    E5M2 (same specification): one sign bit, five exponent bits with bias 15,
    two mantissa bits; exponent field 0 encodes the subnormals m / 4 * 2^-14;
    exponent field 31 encodes infinity (mantissa 0) and NaN (mantissa != 0),
    as in IEEE 754 binary formats."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >= 128, -1.0, 1.0)
    e = (c >> 2) & 31
    m = (c & 3).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 4.0, -14), np.ldexp(1.0 + m / 4.0, e - 15))
    mag = np.where(e == 31, np.where(m == 0, np.inf, np.nan), mag)
    return sign * mag


FP8_DECODERS = {"e4m3": e4m3_decode, "e5m2": e5m2_decode}


def attention_forward_fp8(q8, k8, v8, descale_q, descale_k, descale_v, scale, causal, fmt="e4m3"):
    """O, LSE of exact attention on dequantised 8-bit inputs ([B, H, N, d] code
    arrays, all three in format `fmt`: "e4m3" or "e5m2")."""
    dec = FP8_DECODERS[fmt]
    q = dec(_codes(q8)) * float(descale_q)
    k = dec(_codes(k8)) * float(descale_k)
    v = dec(_codes(v8)) * float(descale_v)
    return attention_forward(q, k, v, scale, causal)


def _codes(x):
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").numpy()
    return np.asarray(x, dtype=np.uint8)
