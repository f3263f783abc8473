"""Plant plausible mistakes in copies of the oracle and check a pin catches each.

The mistakes are planted in the oracle's own source text (on the CPU), never in
the HIP path.  Every mutant must fail at least one pin; a mutant that survives
would mean the pins cannot tell that mistake from the definition.
"""
import os
import types

import pytest

from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "attention.py")

MUTANTS = {
    "dropped scale": ("s = scale * (q @ k.T)", "s = (q @ k.T)"),
    "transposed operand": ("s = scale * (q @ k.T)", "s = scale * (k @ q.T)"),
    "mask direction": ("cols > rows", "cols < rows"),
    "mask off by one": ("cols > rows", "cols >= rows"),
    "mask ignores panel offset": ("np.arange(row0, row0 + q.shape[0])", "np.arange(0, q.shape[0])"),
    "lse without max": ("(m + np.log(l))[:, 0]", "(np.log(l))[:, 0]"),
    "unnormalised P": ("return e / l, (m", "return e, (m"),
    "max along wrong axis": ("np.max(s, axis=1, keepdims=True)", "np.max(s, axis=0, keepdims=True)"),
    "sum along wrong axis": ("l = np.sum(e, axis=1, keepdims=True)", "l = np.sum(e, axis=0, keepdims=True)"),
    "dV not transposed": ("dv = p.T @ do", "dv = p @ do"),
    "dP uses K": ("dp = do @ v.T", "dp = do @ k.T"),
    "dropped D term": ("ds = p * (dp - dsum)", "ds = p * dp"),
    "D wrong axis": ("dsum = np.sum(p * dp, axis=1, keepdims=True)", "dsum = np.sum(p * dp, axis=0, keepdims=True)"),
    "dQ missing scale": ("dq = scale * (ds @ k)", "dq = (ds @ k)"),
    "dK not transposed": ("dk = scale * (ds.T @ q)", "dk = scale * (ds @ q)"),
    "dK sign": ("dk = scale * (ds.T @ q)", "dk = -scale * (ds.T @ q)"),
    "dQ uses V": ("dq = scale * (ds @ k)", "dq = scale * (ds @ v)"),
    "output uses K": ("o[r0:r1] = p @ v", "o[r0:r1] = p @ k"),
    # unequal counts and padded batches
    "kv top-left alignment": ("rows = np.arange(q.shape[0])[:, None] + off", "rows = np.arange(q.shape[0])[:, None]"),
    "kv offset sign (forward)": ("off = lk[b] - lq[b]", "off = lq[b] - lk[b]"),
    "kv offset sign (backward)": ("a, c, off = lq[b], lk[b], lk[b] - lq[b]", "a, c, off = lq[b], lk[b], lq[b] - lk[b]"),
    "kv key lengths ignored": ("lq, lk = _lengths(seqlens_q, B, Nq), _lengths(seqlens_k, B, Nk)",
                               "lq, lk = _lengths(seqlens_q, B, Nq), _lengths(None, B, Nk)"),
    "kv lengths not clamped": ("return [min(max(int(x), 0), n) for x", "return [int(x) for x"),
    "kv padding rows not zero": ("o = np.zeros(q.shape[:3] + (v.shape[3],))", "o = np.ones(q.shape[:3] + (v.shape[3],))"),
    "kv empty rows weighted": ("p[seen] = e[seen] / l[seen, None]", "p = e / np.maximum(l, 1e-300)[:, None] + (~seen)[:, None]"),
    "kv dQ missing scale": ("dq[b, h, :a] = scale * (ds @ kh)", "dq[b, h, :a] = (ds @ kh)"),
    "sparse mask transposed": ("return np.asarray(mask_bh, dtype=bool)[idx[:, None], idx[None, :]]",
                               "return np.asarray(mask_bh, dtype=bool).T[idx[:, None], idx[None, :]]"),
    "sparse block size off by one": ("idx = np.arange(n) // block", "idx = np.arange(n) // (block + 1)"),
    "sparse mask ignored in backward": ("            s = np.where(_block_visible(bm[b, h], N, block), s, -np.inf)\n            p, _ = ",
                                        "            p, _ = "),
    "sparse dV not transposed": ("dv[b, h] = p.T @ do[b, h]", "dv[b, h] = p @ do[b, h]"),
    "philox multiplier": ("_PHILOX_M = (0xD2511F53, 0xCD9E8D57)", "_PHILOX_M = (0xD2511F53, 0xCD9E8D55)"),
    "philox key bump on every round": ("        if r:\n            k0 = (k0", "        if True:\n            k0 = (k0"),
    "dropout keep below threshold": ("return r >= np.uint32(dropout_threshold(p))", "return r < np.uint32(dropout_threshold(p))"),
    "dropout scaled by (1 - p)": ("z = dropout_keep(N, N, b * H + h, p, seed, offset) / (1.0 - p)\n            o[b, h]",
                                  "z = dropout_keep(N, N, b * H + h, p, seed, offset) * (1.0 - p)\n            o[b, h]"),
    "dropout counter transposed": ("words = philox4x32(j >> np.uint64(2), i,", "words = philox4x32(i >> np.uint64(2), j,"),
    "dropout dP without Z": ("dpz = (do[b, h] @ v[b, h].T) * z", "dpz = (do[b, h] @ v[b, h].T)"),
    "dropout dV without Z": ("dv[b, h] = (pr * z).T @ do[b, h]", "dv[b, h] = pr.T @ do[b, h]"),
    "sparse rows mask transposed": ("seen = bm[i // block, keys // block]", "seen = bm[keys // block, i // block]"),
    "e4m3 exponent bias 8": ("np.ldexp(1.0 + m / 8.0, e - 7)", "np.ldexp(1.0 + m / 8.0, e - 8)"),
    "e4m3 subnormals as normals": ("np.where(e == 0, np.ldexp(m / 8.0, -6)", "np.where(e == -1, np.ldexp(m / 8.0, -6)"),
    "e4m3 subnormal exponent": ("np.ldexp(m / 8.0, -6)", "np.ldexp(m / 8.0, -7)"),
    "e4m3 NaN code": ("(c & 127) == 127", "(c & 127) == 126"),
    "fp8 descale_v dropped": ("v = dec(_codes(v8)) * float(descale_v)", "v = dec(_codes(v8))"),
    "fp8 k takes descale_q": ("k = dec(_codes(k8)) * float(descale_k)", "k = dec(_codes(k8)) * float(descale_q)"),
    "e5m2 exponent bias 16": ("np.ldexp(1.0 + m / 4.0, e - 15)", "np.ldexp(1.0 + m / 4.0, e - 16)"),
    "e5m2 three mantissa bits": ("e = (c >> 2) & 31\n    m = (c & 3)", "e = (c >> 3) & 15\n    m = (c & 7)"),
    "e5m2 subnormal exponent": ("np.ldexp(m / 4.0, -14)", "np.ldexp(m / 4.0, -15)"),
    "e5m2 no infinities": ("np.where(m == 0, np.inf, np.nan)", "np.where(m == 0, np.nan, np.nan)"),
    "e5m2 sign ignored": ("sign = np.where(c >= 128, -1.0, 1.0)\n    e = (c >> 2)", "sign = 1.0\n    e = (c >> 2)"),
    "fp8 format ignored": ("dec = FP8_DECODERS[fmt]", "dec = e4m3_decode"),
    "kv dropped D term": ("ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))\n            dq[b, h, :a]",
                          "ds = p * dp\n            dq[b, h, :a]"),
}


def _mutant(old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"pattern not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)  # noqa: S102
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(*MUTANTS[name])
    failures = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # AssertionError, or a crash caused by the mistake
            failures.append(f"{pin.__name__}: {type(e).__name__}")
    assert failures, f"no pin catches the planted mistake '{name}'"
