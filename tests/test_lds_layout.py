"""CPU model of the LDS tile of the 16-key dK/dV kernel (dkdv16n_kernel, d = 128).

The kernel stores 64-row Q and dO tiles with the 16-byte chunks of row r
XOR-permuted by sw(r) = 2 (r mod 8) + (r / 8 mod 2), and reads them in two
patterns: row fragments (16-byte reads, lane l: row 16 qb + l % 16, chunk
4 ks + l / 16) and transposing reads (ds_read_b64_tr_b16, lane l = 16 g + i:
row 4 g + i / 4 (+ 16 for the second read, + 32 per query half), chunk
2 nb + (i % 4) / 2, byte 8 (i % 2)).  This model restates those formulas and
checks, with a 64-bank model of the LDS (16 lanes per cycle for 16-byte
reads, 32 for 8-byte reads), that both patterns are conflict-free; that the
transposing reads, under the instruction's semantics (per 16-lane group, lane
i receives element e of M[4 e + i / 4][i % 4], M[j] being the four 16-bit
values at lane j's address), hand the 16x16x32 product the A operand that
matches P taken from the accumulators (query of contraction slot (g, e):
16 (e / 4) + 4 g + e % 4), so that the product is dO^T P exactly; and that
the direct loads place every chunk where the reads expect it.
"""
import numpy as np

ROWB, CPR, ROWS = 256, 16, 64


def sw(r):
    return ((r & 7) << 1) | ((r >> 3) & 1)


def phys(r, c):
    return r * ROWB + ((c ^ sw(r)) << 4)


def row_addr(l, qb, ks):
    return phys(16 * qb + (l & 15), 4 * ks + (l >> 4))


def tr_addr(l, nb, hq, rd):
    g, i = l >> 4, l & 15
    return phys(32 * hq + 16 * rd + 4 * g + (i >> 2), 2 * nb + ((i & 3) >> 1)) + 8 * (i & 1)


def _banks(addr, nbytes):
    return [((addr >> 2) + w) % 64 for w in range(nbytes // 4)]


def test_row_fragments_are_conflict_free_and_in_bounds():
    for qb in range(4):
        for ks in range(4):
            a = [row_addr(l, qb, ks) for l in range(64)]
            assert all(0 <= x and x + 16 <= ROWS * ROWB for x in a)
            for grp in range(4):
                banks = [b for l in range(16 * grp, 16 * grp + 16) for b in _banks(a[l], 16)]
                assert len(set(banks)) == 64, (qb, ks, grp)


def test_transposing_reads_are_conflict_free_and_in_bounds():
    for nb in range(8):
        for hq in range(2):
            for rd in range(2):
                a = [tr_addr(l, nb, hq, rd) for l in range(64)]
                assert all(0 <= x and x + 8 <= ROWS * ROWB for x in a)
                for half in range(2):
                    banks = [b for l in range(32 * half, 32 * half + 32) for b in _banks(a[l], 8)]
                    assert len(set(banks)) == 64, (nb, hq, rd, half)


def test_the_old_permutation_would_conflict():
    """The 32-key kernel's permutation for 256-byte rows, 4 (r mod 4) + (r / 4 mod 4),
    suits its own read patterns but not these transposing reads."""
    def phys_old(r, c):
        return r * ROWB + ((c ^ (4 * (r & 3) + ((r >> 2) & 3))) << 4)
    a = [phys_old(4 * (l >> 4) + ((l & 15) >> 2), (l & 3) >> 1) + 8 * (l & 1) for l in range(32)]
    banks = [b for x in a for b in _banks(x, 8)]
    assert len(set(banks)) < 64


def _tr_read(mem, addrs):
    out = np.zeros((64, 4))
    for grp in range(4):
        m = [mem[addrs[16 * grp + j] // 2: addrs[16 * grp + j] // 2 + 4] for j in range(16)]
        for i in range(16):
            for e in range(4):
                out[16 * grp + i][e] = m[4 * e + i // 4][i % 4]
    return out


def test_transposing_operands_give_dO_transpose_P():
    rng = np.random.default_rng(1)
    dO = rng.integers(-3, 4, (64, 128)).astype(np.float64)
    P = rng.integers(-3, 4, (64, 16)).astype(np.float64)   # [query][key] of one wave's 16 keys
    mem = np.zeros(ROWS * ROWB // 2)
    for q in range(64):
        for c in range(128):
            byte = phys(q, (2 * c) // 16) + (2 * c) % 16
            mem[byte // 2] = dO[q][c]

    def slot_query(g, e):
        return 16 * (e // 4) + 4 * g + e % 4

    for hq in range(2):
        for nb in range(8):
            A = np.concatenate([_tr_read(mem, [tr_addr(l, nb, hq, 0) for l in range(64)]),
                                _tr_read(mem, [tr_addr(l, nb, hq, 1) for l in range(64)])], axis=1)
            B = np.array([[P[32 * hq + slot_query(l >> 4, e)][l & 15] for e in range(8)] for l in range(64)])
            Am = np.array([[A[m + 16 * (k // 8)][k % 8] for k in range(32)] for m in range(16)])
            Bm = np.array([[B[n + 16 * (k // 8)][k % 8] for n in range(16)] for k in range(32)])
            want = dO[32 * hq: 32 * hq + 32, 16 * nb: 16 * nb + 16].T @ P[32 * hq: 32 * hq + 32]
            assert np.array_equal(Am @ Bm, want), (hq, nb)


def test_row_fragments_give_Q_K_transpose():
    """S = Q K^T from row fragments (A) and the lane's key row (B), per 16-query block and 32-channel step."""
    rng = np.random.default_rng(2)
    Q = rng.integers(-3, 4, (64, 128)).astype(np.float64)
    K = rng.integers(-3, 4, (16, 128)).astype(np.float64)
    mem = np.zeros(ROWS * ROWB // 2)
    for q in range(64):
        for c in range(128):
            byte = phys(q, (2 * c) // 16) + (2 * c) % 16
            mem[byte // 2] = Q[q][c]
    for qb in range(4):
        S = np.zeros((16, 16))
        for ks in range(4):
            A = np.array([mem[row_addr(l, qb, ks) // 2: row_addr(l, qb, ks) // 2 + 8] for l in range(64)])
            B = np.array([K[l & 15][32 * ks + 8 * (l >> 4): 32 * ks + 8 * (l >> 4) + 8] for l in range(64)])
            Am = np.array([[A[m + 16 * (k // 8)][k % 8] for k in range(32)] for m in range(16)])
            Bm = np.array([[B[n + 16 * (k // 8)][k % 8] for n in range(16)] for k in range(32)])
            S += Am @ Bm
        assert np.array_equal(S, Q[16 * qb: 16 * qb + 16] @ K.T), qb


def test_direct_loads_place_every_chunk():
    """Eight waves x 64 lanes x 2 rounds: slot s = (8 r + wave) * 64 + lane lands at LDS byte 16 s
    and loads logical chunk (s % 16) ^ sw(row) of row s / 16."""
    placed = {}
    for r in range(2):
        for w in range(8):
            for l in range(64):
                s = (r * 8 + w) * 64 + l
                row, pc = s // CPR, s % CPR
                placed[16 * s] = row * ROWB + ((pc ^ sw(row)) << 4)
    assert len(placed) == ROWS * CPR
    for row in range(ROWS):
        for c in range(CPR):
            assert placed[phys(row, c)] == row * ROWB + 16 * c
