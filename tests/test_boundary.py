"""The C-ABI boundary on the CPU: libfa.so loads, exports what include/fa.h
declares, and rejects every invalid call before any HIP call.

Calls here use made-up (but aligned, non-overlapping) addresses, so they must
never reach a kernel on a machine that has a GPU: every call that could pass
validation is skipped unless the machine has no GPU at all.
"""
import ctypes
import math
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def _no_gpu_here():
    if os.path.exists("/dev/kfd"):
        return False
    import torch
    return torch.cuda.device_count() == 0


@pytest.fixture(scope="module")
def fa():
    import exact_io_aware_51_amd as m
    m.load()
    return m


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_abi():
    assert _declared() == sorted(["fa_fwd", "fa_bwd", "fa_bwd_workspace_bytes", "fa_bwd_rowsum", "fa_bwd_dkdv",
                                  "fa_bwd_dq", "fa_fwd_kv", "fa_bwd_kv", "fa_fwd_sparse", "fa_bwd_sparse",
                                  "fa_fwd_dropout", "fa_bwd_dropout", "fa_fwd_fp8", "fa_fwd_kv_split",
                                  "fa_fwd_kv_split_workspace_bytes", "fa_fwd_kv_split_hint", "fa_status_string",
                                  "fa_version", "fa_bwd_static", "fa_fwd_fp8_fmt",
                                  "fa_bwd_dq_rowsum"])


def test_library_exports_every_declared_symbol(fa):
    lib = ctypes.CDLL(fa.library_path())
    for name in _declared():
        assert hasattr(lib, name), f"libfa.so does not export {name}"


def test_status_strings(fa):
    for st in (0, -1, -2, -3, -4, -5):
        s = fa.fa_status_string(st)
        assert s and s != "unknown status"
    assert fa.fa_status_string(12345) == "unknown status"
    assert fa.fa_version() == 10100


def test_workspace_bytes(fa):
    assert fa.fa_bwd_workspace_bytes(2, 16, 4096, 128, fa.FA_BF16) == 2 * 16 * 4096 * 4
    assert fa.fa_bwd_workspace_bytes(1, 1, 1, 64, fa.FA_F32) == 256          # rounded up to 256 B
    assert fa.fa_bwd_workspace_bytes(1, 1, 1, 96, fa.FA_F16) == 0            # unsupported d
    assert fa.fa_bwd_workspace_bytes(0, 1, 1, 64, fa.FA_F16) == 0            # bad size
    assert fa.fa_bwd_workspace_bytes(1, 1, 1, 64, 7) == 0                    # bad dtype


# Fake, 16-byte aligned, widely spaced addresses (never dereferenced).
BASE = 1 << 40
SPAN = 1 << 34


def _ptr(i, off=0):
    return BASE + i * SPAN + off


def _fwd(fa, **kw):
    a = dict(q=_ptr(0), k=_ptr(1), v=_ptr(2), o=_ptr(3), lse=_ptr(4), B=1, H=2, N=256, d=64,
             scale=0.125, causal=0, dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return fa.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"],
                     a["scale"], a["causal"], a["dtype"], a["stream"])


def _bwd(fa, **kw):
    a = dict(q=_ptr(0), k=_ptr(1), v=_ptr(2), o=_ptr(3), dout=_ptr(4), lse=_ptr(5), dq=_ptr(6),
             dk=_ptr(7), dv=_ptr(8), ws=_ptr(9), wsb=1 << 20, B=1, H=2, N=256, d=64, scale=0.125,
             causal=1, dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return fa.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"], a["dk"], a["dv"],
                     a["ws"], a["wsb"], a["B"], a["H"], a["N"], a["d"], a["scale"], a["causal"],
                     a["dtype"], a["stream"])


FWD_BAD = [
    ("null q", dict(q=None), -1), ("null o", dict(o=None), -1),
    ("misaligned k", dict(k=_ptr(1, 8)), -1), ("misaligned o", dict(o=_ptr(3, 2)), -1),
    ("misaligned lse", dict(lse=_ptr(4, 2)), -1),
    ("B=0", dict(B=0), -1), ("H<0", dict(H=-1), -1), ("N=0", dict(N=0), -1), ("d=0", dict(d=0), -1),
    ("huge B*H*N", dict(B=1 << 16, H=1 << 10, N=1 << 10), -1),
    ("d=96", dict(d=96), -2), ("d=256", dict(d=256), -2), ("dtype 5", dict(dtype=5), -2),
    ("nan scale", dict(scale=float("nan")), -1), ("inf scale", dict(scale=float("inf")), -1),
    ("scale overflows log2e", dict(scale=3.0e38), -1),
    ("causal 2", dict(causal=2), -1),
    ("o aliases q", dict(o=_ptr(0)), -1), ("o overlaps v", dict(o=_ptr(2, 4096)), -1),
    ("lse aliases k", dict(lse=_ptr(1)), -1), ("lse inside o", dict(lse=_ptr(3, 64)), -1),
]

BWD_BAD = [
    ("null dout", dict(dout=None), -1), ("null lse", dict(lse=None), -1), ("null dv", dict(dv=None), -1),
    ("misaligned dq", dict(dq=_ptr(6, 4)), -1), ("misaligned lse", dict(lse=_ptr(5, 1)), -1),
    ("d=32", dict(d=32), -2), ("N=0", dict(N=0), -1), ("causal -1", dict(causal=-1), -1),
    ("no workspace", dict(ws=None), -3), ("small workspace", dict(wsb=100), -3),
    ("misaligned workspace", dict(ws=_ptr(9, 4)), -3),
    ("workspace overlaps dk", dict(ws=_ptr(7, 16)), -3), ("workspace overlaps q", dict(ws=_ptr(0)), -3),
    ("dq aliases dk", dict(dk=_ptr(6)), -1), ("dv aliases v", dict(dv=_ptr(2)), -1),
    ("dq aliases lse", dict(dq=_ptr(5)), -1),
]


@pytest.mark.parametrize("name,kw,want", FWD_BAD, ids=[x[0] for x in FWD_BAD])
def test_fwd_rejects(fa, name, kw, want):
    assert _fwd(fa, **kw) == want


@pytest.mark.parametrize("name,kw,want", BWD_BAD, ids=[x[0] for x in BWD_BAD])
def test_bwd_rejects(fa, name, kw, want):
    assert _bwd(fa, **kw) == want


def _bwd_static(fa, **kw):
    a = dict(q=_ptr(0), k=_ptr(1), v=_ptr(2), o=_ptr(3), dout=_ptr(4), lse=_ptr(5), dq=_ptr(6),
             dk=_ptr(7), dv=_ptr(8), B=1, H=2, N=256, d=64, scale=0.125, causal=1, dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return fa.fa_bwd_static(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"], a["dk"], a["dv"],
                            a["B"], a["H"], a["N"], a["d"], a["scale"], a["causal"], a["dtype"], a["stream"])


STATIC_BAD = [
    ("null dout", dict(dout=None), -1), ("null lse", dict(lse=None), -1), ("misaligned dk", dict(dk=_ptr(7, 2)), -1),
    ("d=32", dict(d=32), -2), ("N=0", dict(N=0), -1), ("causal 2", dict(causal=2), -1),
    ("dq aliases q", dict(dq=_ptr(0)), -1), ("inf scale", dict(scale=float("inf")), -1),
    # one row past the static scratch, and far past it; the addresses are never touched
    ("B*H*N = capacity + 1", dict(B=1, H=1, N=(1 << 22) + 1), -5),
    ("B*H*N = 6 x 700000", dict(B=2, H=3, N=700000), -5),
]


@pytest.mark.parametrize("name,kw,want", STATIC_BAD, ids=[x[0] for x in STATIC_BAD])
def test_bwd_static_rejects(fa, name, kw, want):
    assert _bwd_static(fa, **kw) == want


def test_bwd_static_capacity_is_declared(fa):
    text = open(HEADER).read()
    assert re.search(r"#define FA_STATIC_SCRATCH_ROWS \(1 << 22\)", text)
    assert fa.STATIC_SCRATCH_ROWS == 1 << 22
    assert "fa_bwd_static" in fa.fa_status_string(fa.FA_ERR_TOO_LARGE)


STAGE_BAD = [
    ("rowsum null o", lambda fa: fa.fa_bwd_rowsum(None, _ptr(4), _ptr(9), 1 << 20, 1, 2, 256, 64, fa.FA_BF16, None), -1),
    ("rowsum small ws", lambda fa: fa.fa_bwd_rowsum(_ptr(3), _ptr(4), _ptr(9), 64, 1, 2, 256, 64, fa.FA_BF16, None), -3),
    ("rowsum ws aliases o", lambda fa: fa.fa_bwd_rowsum(_ptr(3), _ptr(4), _ptr(3), 1 << 20, 1, 2, 256, 64, fa.FA_BF16, None), -3),
    ("rowsum d=80", lambda fa: fa.fa_bwd_rowsum(_ptr(3), _ptr(4), _ptr(9), 1 << 20, 1, 2, 256, 80, fa.FA_BF16, None), -2),
    ("dkdv null lse", lambda fa: fa.fa_bwd_dkdv(_ptr(0), _ptr(1), _ptr(2), _ptr(4), None, _ptr(9), 1 << 20, _ptr(7), _ptr(8), 1, 2, 256, 64, 0.125, 1, fa.FA_BF16, None), -1),
    ("dkdv dk aliases dv", lambda fa: fa.fa_bwd_dkdv(_ptr(0), _ptr(1), _ptr(2), _ptr(4), _ptr(5), _ptr(9), 1 << 20, _ptr(7), _ptr(7), 1, 2, 256, 64, 0.125, 1, fa.FA_BF16, None), -1),
    ("dkdv nan scale", lambda fa: fa.fa_bwd_dkdv(_ptr(0), _ptr(1), _ptr(2), _ptr(4), _ptr(5), _ptr(9), 1 << 20, _ptr(7), _ptr(8), 1, 2, 256, 64, float("nan"), 1, fa.FA_BF16, None), -1),
    ("dq misaligned dq", lambda fa: fa.fa_bwd_dq(_ptr(0), _ptr(1), _ptr(2), _ptr(4), _ptr(5), _ptr(9), 1 << 20, _ptr(6, 8), 1, 2, 256, 64, 0.125, 1, fa.FA_BF16, None), -1),
    ("dq no workspace", lambda fa: fa.fa_bwd_dq(_ptr(0), _ptr(1), _ptr(2), _ptr(4), _ptr(5), None, 1 << 20, _ptr(6), 1, 2, 256, 64, 0.125, 1, fa.FA_BF16, None), -3),
    ("dq aliases k", lambda fa: fa.fa_bwd_dq(_ptr(0), _ptr(1), _ptr(2), _ptr(4), _ptr(5), _ptr(9), 1 << 20, _ptr(1), 1, 2, 256, 64, 0.125, 1, fa.FA_BF16, None), -1),
    # the dQ stage that also writes the row sums: o is read, the workspace written
    ("dq_rowsum null o", lambda fa: _dq_rowsum(fa, o=None), -1),
    ("dq_rowsum misaligned o", lambda fa: _dq_rowsum(fa, o=_ptr(3, 8)), -1),
    ("dq_rowsum no workspace", lambda fa: _dq_rowsum(fa, ws=None), -3),
    ("dq_rowsum small workspace", lambda fa: _dq_rowsum(fa, wsb=64), -3),
    ("dq_rowsum workspace aliases o", lambda fa: _dq_rowsum(fa, ws=_ptr(3)), -3),
    ("dq_rowsum dq aliases o", lambda fa: _dq_rowsum(fa, dq=_ptr(3)), -1),
    ("dq_rowsum dq aliases workspace", lambda fa: _dq_rowsum(fa, dq=_ptr(9)), -3),
    ("dq_rowsum d=96", lambda fa: _dq_rowsum(fa, d=96), -2),
    ("dq_rowsum causal=3", lambda fa: _dq_rowsum(fa, causal=3), -1),
]


def _dq_rowsum(fa, **kw):
    a = dict(q=_ptr(0), k=_ptr(1), v=_ptr(2), o=_ptr(3), do=_ptr(4), lse=_ptr(5), ws=_ptr(9), wsb=1 << 20,
             dq=_ptr(6), B=1, H=2, N=256, d=64, scale=0.125, causal=1, dtype=fa.FA_BF16)
    a.update(kw)
    return fa.fa_bwd_dq_rowsum(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["ws"], a["wsb"], a["dq"],
                               a["B"], a["H"], a["N"], a["d"], a["scale"], a["causal"], a["dtype"], None)


@pytest.mark.parametrize("name,call,want", STAGE_BAD, ids=[x[0] for x in STAGE_BAD])
def test_bwd_stages_reject(fa, name, call, want):
    assert call(fa) == want


# Unequal counts: q/o hold Nq = 256 rows, k/v Nk = 1024 rows per (b, h); with
# B = 1, H = 2, d = 64, bf16 that is 65536 B for q and 262144 B for k.
KV_K_BYTES = 2 * 1024 * 64 * 2


def _fwd_kv(fa, **kw):
    a = dict(q=_ptr(0), k=_ptr(1), v=_ptr(2), o=_ptr(3), lse=_ptr(4), B=1, H=2, Nq=256, Nk=1024, d=64,
             sq=_ptr(10), sk=_ptr(11), scale=0.125, causal=1, dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return fa.fa_fwd_kv(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"], a["Nk"], a["d"],
                        a["sq"], a["sk"], a["scale"], a["causal"], a["dtype"], a["stream"])


def _bwd_kv(fa, **kw):
    a = dict(q=_ptr(0), k=_ptr(1), v=_ptr(2), o=_ptr(3), dout=_ptr(4), lse=_ptr(5), dq=_ptr(6),
             dk=_ptr(7), dv=_ptr(8), ws=_ptr(9), wsb=1 << 20, B=1, H=2, Nq=256, Nk=1024, d=64,
             sq=_ptr(10), sk=_ptr(11), scale=0.125, causal=1, dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return fa.fa_bwd_kv(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"], a["dk"], a["dv"],
                        a["ws"], a["wsb"], a["B"], a["H"], a["Nq"], a["Nk"], a["d"], a["sq"], a["sk"],
                        a["scale"], a["causal"], a["dtype"], a["stream"])


KV_FWD_BAD = [
    ("Nq=0", dict(Nq=0), -1), ("Nk=0", dict(Nk=0), -1), ("Nk<0", dict(Nk=-5), -1),
    ("huge B*H*Nk", dict(B=1 << 16, H=1 << 10, Nk=1 << 10), -1),
    ("misaligned seqlens_q", dict(sq=_ptr(10, 2)), -1), ("misaligned seqlens_k", dict(sk=_ptr(11, 1)), -1),
    ("d=48", dict(d=48), -2), ("causal 3", dict(causal=3), -1), ("null v", dict(v=None), -1),
    ("o inside k (sized by Nk)", dict(o=_ptr(1, KV_K_BYTES - 4096)), -1),
    ("o over seqlens_q", dict(o=_ptr(10)), -1), ("lse over seqlens_k", dict(lse=_ptr(11)), -1),
]

KV_BWD_BAD = [
    ("Nk=0", dict(Nk=0), -1), ("misaligned seqlens_k", dict(sk=_ptr(11, 2)), -1),
    ("workspace sized by Nq", dict(wsb=2 * 256 * 4 - 4), -3),
    ("dk inside v (sized by Nk)", dict(dk=_ptr(2, KV_K_BYTES - 4096)), -1),
    ("dq over seqlens_q", dict(dq=_ptr(10)), -1), ("dv over seqlens_k", dict(dv=_ptr(11)), -1),
    ("workspace over seqlens_k", dict(ws=_ptr(11)), -3),
    ("null dout", dict(dout=None), -1), ("dtype 9", dict(dtype=9), -2),
]


@pytest.mark.parametrize("name,kw,want", KV_FWD_BAD, ids=[x[0] for x in KV_FWD_BAD])
def test_fwd_kv_rejects(fa, name, kw, want):
    assert _fwd_kv(fa, **kw) == want


@pytest.mark.parametrize("name,kw,want", KV_BWD_BAD, ids=[x[0] for x in KV_BWD_BAD])
def test_bwd_kv_rejects(fa, name, kw, want):
    assert _bwd_kv(fa, **kw) == want


# Block sparse: N = 256 -> a [1, 2, 2, 2] mask of 8 bytes.
def _fwd_sp(fa, **kw):
    a = dict(q=_ptr(0), k=_ptr(1), v=_ptr(2), o=_ptr(3), lse=_ptr(4), B=1, H=2, N=256, d=64, m=_ptr(12),
             scale=0.125, causal=1, dtype=fa.FA_F16, stream=None)
    a.update(kw)
    return fa.fa_fwd_sparse(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"], a["m"],
                            a["scale"], a["causal"], a["dtype"], a["stream"])


def _bwd_sp(fa, **kw):
    a = dict(q=_ptr(0), k=_ptr(1), v=_ptr(2), o=_ptr(3), dout=_ptr(4), lse=_ptr(5), dq=_ptr(6),
             dk=_ptr(7), dv=_ptr(8), ws=_ptr(9), wsb=1 << 20, B=1, H=2, N=256, d=64, m=_ptr(12), scale=0.125,
             causal=0, dtype=fa.FA_F16, stream=None)
    a.update(kw)
    return fa.fa_bwd_sparse(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"], a["dk"], a["dv"],
                            a["ws"], a["wsb"], a["B"], a["H"], a["N"], a["d"], a["m"], a["scale"], a["causal"],
                            a["dtype"], a["stream"])


SP_FWD_BAD = [
    ("null mask", dict(m=None), -1), ("N=0", dict(N=0), -1), ("d=80", dict(d=80), -2),
    ("N past the mask table", dict(N=524288 + 1), -2),
    ("o over mask", dict(o=_ptr(12, -4096)), -1), ("lse over mask end", dict(lse=_ptr(12, 4)), -1),
    ("null k", dict(k=None), -1), ("inf scale", dict(scale=float("inf")), -1),
]
SP_BWD_BAD = [
    ("null mask", dict(m=None), -1), ("dk over mask", dict(dk=_ptr(12)), -1),
    ("workspace over mask", dict(ws=_ptr(12, -16)), -3), ("small workspace", dict(wsb=8), -3),
    ("misaligned dv", dict(dv=_ptr(8, 2)), -1),
]


@pytest.mark.parametrize("name,kw,want", SP_FWD_BAD, ids=[x[0] for x in SP_FWD_BAD])
def test_fwd_sparse_rejects(fa, name, kw, want):
    assert _fwd_sp(fa, **kw) == want


@pytest.mark.parametrize("name,kw,want", SP_BWD_BAD, ids=[x[0] for x in SP_BWD_BAD])
def test_bwd_sparse_rejects(fa, name, kw, want):
    assert _bwd_sp(fa, **kw) == want


# Dropout: the probability must lie in [0, 1); seed and offset take any value.
def _fwd_dp(fa, **kw):
    a = dict(q=_ptr(0), k=_ptr(1), v=_ptr(2), o=_ptr(3), lse=_ptr(4), B=1, H=2, N=256, d=64, scale=0.125,
             causal=1, p=0.1, seed=(1 << 64) - 1, offset=(1 << 32) - 1, dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return fa.fa_fwd_dropout(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"],
                             a["scale"], a["causal"], a["p"], a["seed"], a["offset"], a["dtype"], a["stream"])


def _bwd_dp(fa, **kw):
    a = dict(q=_ptr(0), k=_ptr(1), v=_ptr(2), o=_ptr(3), dout=_ptr(4), lse=_ptr(5), dq=_ptr(6),
             dk=_ptr(7), dv=_ptr(8), ws=_ptr(9), wsb=1 << 20, B=1, H=2, N=256, d=64, scale=0.125,
             causal=0, p=0.25, seed=7, offset=3, dtype=fa.FA_F16, stream=None)
    a.update(kw)
    return fa.fa_bwd_dropout(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"], a["dk"], a["dv"],
                             a["ws"], a["wsb"], a["B"], a["H"], a["N"], a["d"], a["scale"], a["causal"], a["p"],
                             a["seed"], a["offset"], a["dtype"], a["stream"])


DP_FWD_BAD = [
    ("p=1", dict(p=1.0), -1), ("p<0", dict(p=-1e-3), -1), ("p=nan", dict(p=float("nan")), -1),
    ("p=inf", dict(p=float("inf")), -1), ("N=0", dict(N=0), -1), ("d=96", dict(d=96), -2),
    ("null v", dict(v=None), -1), ("o over q", dict(o=_ptr(0, 16)), -1), ("dtype 7", dict(dtype=7), -2),
]
DP_BWD_BAD = [
    ("p=1", dict(p=1.0), -1), ("p=nan", dict(p=float("nan")), -1), ("null lse", dict(lse=None), -1),
    ("small workspace", dict(wsb=8), -3), ("dq over dk", dict(dq=_ptr(7)), -1),
]


@pytest.mark.parametrize("name,kw,want", DP_FWD_BAD, ids=[x[0] for x in DP_FWD_BAD])
def test_fwd_dropout_rejects(fa, name, kw, want):
    assert _fwd_dp(fa, **kw) == want


@pytest.mark.parametrize("name,kw,want", DP_BWD_BAD, ids=[x[0] for x in DP_BWD_BAD])
def test_bwd_dropout_rejects(fa, name, kw, want):
    assert _bwd_dp(fa, **kw) == want


# Split-key forward: B=1, H=2, Nq=4, Nk=4096, d=128, 8 splits -> 8 * 8 * 129 * 4 bytes of workspace.
def _fwd_split(fa, **kw):
    a = dict(q=_ptr(0), k=_ptr(1), v=_ptr(2), o=_ptr(3), lse=_ptr(4), B=1, H=2, Nq=4, Nk=4096, d=128,
             sq=None, sk=_ptr(11), scale=0.088, causal=1, ns=8, ws=_ptr(9), wsb=1 << 20, dtype=fa.FA_BF16,
             stream=None)
    a.update(kw)
    return fa.fa_fwd_kv_split(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"], a["Nk"], a["d"],
                              a["sq"], a["sk"], a["scale"], a["causal"], a["ns"], a["ws"], a["wsb"], a["dtype"],
                              a["stream"])


def test_split_workspace_and_hint(fa):
    assert fa.fa_fwd_kv_split_workspace_bytes(1, 2, 4, 4096, 128, 8) == 8 * 8 * 129 * 4
    assert fa.fa_fwd_kv_split_workspace_bytes(1, 2, 4, 4096, 128, 1) == 0
    assert fa.fa_fwd_kv_split_workspace_bytes(1, 2, 4, 4096, 128, 0) == 0
    assert fa.fa_fwd_kv_split_workspace_bytes(1, 2, 4, 4096, 96, 8) == 0
    assert fa.fa_fwd_kv_split_hint(1, 8, 1, 32768, 128) == 32      # at least 1024 keys per split
    assert fa.fa_fwd_kv_split_hint(4, 32, 1, 8192, 128) == 4       # about 512 workgroups
    assert fa.fa_fwd_kv_split_hint(1, 8, 1, 1024, 128) == 1
    assert fa.fa_fwd_kv_split_hint(4, 32, 8192, 8192, 64) == 1     # already thousands of workgroups
    assert fa.fa_fwd_kv_split_hint(1, 1, 1, 64, 64) == 1


SPLIT_BAD = [
    ("0 splits", dict(ns=0), -1), ("257 splits", dict(ns=257), -1), ("fp32 split", dict(dtype=0), -2),
    ("null workspace", dict(ws=None), -3), ("small workspace", dict(wsb=4096), -3),
    ("misaligned workspace", dict(ws=_ptr(9, 8)), -3), ("workspace over k", dict(ws=_ptr(1, 64)), -3),
    ("workspace over lengths", dict(ws=_ptr(11, -64)), -3), ("d=80", dict(d=80), -2), ("Nk=0", dict(Nk=0), -1),
    ("o over q", dict(o=_ptr(0, 32)), -1),
    ("grid past 2^31", dict(B=1 << 13, H=1 << 10, Nq=1, Nk=64, ns=256, wsb=1 << 62), -1),  # 2^23 heads x 256 splits
]


@pytest.mark.parametrize("name,kw,want", SPLIT_BAD, ids=[x[0] for x in SPLIT_BAD])
def test_fwd_kv_split_rejects(fa, name, kw, want):
    assert _fwd_split(fa, **kw) == want


# 8-bit inputs: q, k, v are N*d bytes per head, o twice that (bf16).
def _fwd8(fa, **kw):
    a = dict(q=_ptr(0), k=_ptr(1), v=_ptr(2), o=_ptr(3), lse=_ptr(4), B=1, H=2, N=256, d=128, scale=0.088,
             causal=1, dq=0.01, dk=0.02, dv=0.5, stream=None, fmt=None)
    a.update(kw)
    args = (a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"], a["scale"], a["causal"],
            a["dq"], a["dk"], a["dv"])
    if a["fmt"] is None:
        return fa.fa_fwd_fp8(*args, a["stream"])
    return fa.fa_fwd_fp8_fmt(*args, a["fmt"], a["stream"])


FP8_BAD = [
    ("N=0", dict(N=0), -1), ("d=96", dict(d=96), -2), ("causal=2", dict(causal=2), -1),
    ("null q", dict(q=None), -1), ("misaligned k", dict(k=_ptr(1, 8)), -1), ("misaligned lse", dict(lse=_ptr(4, 2)), -1),
    ("inf descale_q", dict(dq=float("inf")), -1), ("nan descale_v", dict(dv=float("nan")), -1),
    ("scale product overflows", dict(scale=1e30, dq=1e30, dk=1e10), -1),
    # o is bf16: 2 bytes per element, so it reaches into the next input at twice the input size
    ("o over v", dict(o=_ptr(2, -2 * 256 * 128)), -1), ("lse over o", dict(lse=_ptr(3, 4)), -1),
    ("B*H*N too large", dict(B=1 << 16, H=1 << 8, N=1 << 8), -1),
]


@pytest.mark.parametrize("fmt", [None, 0, 1], ids=["fp8", "fmt-e4m3", "fmt-e5m2"])
@pytest.mark.parametrize("name,kw,want", FP8_BAD, ids=[x[0] for x in FP8_BAD])
def test_fwd_fp8_rejects(fa, name, kw, want, fmt):
    assert _fwd8(fa, fmt=fmt, **kw) == want


@pytest.mark.parametrize("fmt", [-1, 2, 255])
def test_fwd_fp8_fmt_rejects_unknown_formats(fa, fmt):
    assert _fwd8(fa, fmt=fmt) == -1


@pytest.mark.skipif(not _no_gpu_here(), reason="would launch on fake addresses; only meaningful with no GPU")
def test_valid_call_without_device_reports_hip_error(fa):
    assert _fwd(fa) == fa.FA_ERR_HIP
    assert _fwd(fa, lse=None, causal=1, dtype=fa.FA_F32, scale=-1.0) == fa.FA_ERR_HIP
    assert _bwd(fa) == fa.FA_ERR_HIP
    assert _bwd_static(fa) == fa.FA_ERR_HIP
    assert _bwd_static(fa, B=1, H=1, N=1 << 22) == fa.FA_ERR_HIP  # exactly the capacity is accepted
    assert fa.fa_bwd_rowsum(_ptr(3), _ptr(4), _ptr(9), 1 << 20, 1, 2, 256, 64, fa.FA_BF16, None) == fa.FA_ERR_HIP
    assert _dq_rowsum(fa) == fa.FA_ERR_HIP
    assert _dq_rowsum(fa, dtype=fa.FA_F32, causal=0, d=128) == fa.FA_ERR_HIP
    assert _fwd_kv(fa) == fa.FA_ERR_HIP
    assert _fwd_kv(fa, sq=None, sk=None, Nq=1) == fa.FA_ERR_HIP
    assert _bwd_kv(fa) == fa.FA_ERR_HIP
    assert _fwd_sp(fa) == fa.FA_ERR_HIP
    assert _bwd_sp(fa) == fa.FA_ERR_HIP
    assert _fwd_dp(fa) == fa.FA_ERR_HIP
    assert _fwd_dp(fa, p=0.0) == fa.FA_ERR_HIP
    assert _fwd_dp(fa, p=float(np.nextafter(np.float32(1), np.float32(0)))) == fa.FA_ERR_HIP
    assert _bwd_dp(fa) == fa.FA_ERR_HIP
    assert _fwd8(fa) == fa.FA_ERR_HIP
    assert _fwd_split(fa) == fa.FA_ERR_HIP
    assert _fwd_split(fa, ns=1, ws=None) == fa.FA_ERR_HIP
    assert _fwd8(fa, lse=None, causal=0, d=64, scale=-0.1) == fa.FA_ERR_HIP
    assert _fwd8(fa, fmt=fa.FA_FP8_E5M2) == fa.FA_ERR_HIP
    assert _fwd8(fa, fmt=fa.FA_FP8_E4M3, causal=0, d=64) == fa.FA_ERR_HIP


def test_python_helpers_refuse_cpu_tensors(fa):
    import torch
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.forward(q, q, q)
    with pytest.raises(ValueError):
        fa.backward(q, q, q, q, torch.zeros(1, 1, 4), q)
    with pytest.raises(ValueError):
        fa.forward_kv(q, q, q, seqlens_q=[4])
    with pytest.raises(ValueError):
        fa.backward_kv(q, q, q, q, torch.zeros(1, 1, 4), q)
    assert math.isclose(1 / math.sqrt(64), 0.125)


def test_python_helpers_check_caller_buffers(fa):
    """Caller-supplied out / lse / workspace are checked before any launch: the
    C ABI sees only addresses, so a wrong shape, dtype, device or an undersized
    workspace would otherwise reach a kernel.  The checks are device-agnostic,
    so CPU tensors stand in for device tensors here."""
    import torch
    q = torch.zeros(2, 3, 5, 64, dtype=torch.bfloat16)
    assert fa._check_like(torch.empty_like(q), q, "out") is not None
    for bad in (torch.empty(2, 3, 5, 64, dtype=torch.float16), torch.empty(2, 3, 6, 64, dtype=torch.bfloat16),
                torch.empty(2, 3, 64, 5, dtype=torch.bfloat16).transpose(2, 3), "not a tensor"):
        with pytest.raises(ValueError):
            fa._check_like(bad, q, "out")
    dev = q.device
    assert fa._check_rows(torch.empty(2, 3, 5), (2, 3, 5), dev, "lse") is not None
    for bad in (torch.empty(2, 3, 5, dtype=torch.bfloat16), torch.empty(2, 3, 4), torch.empty(2, 5, 3).transpose(1, 2),
                torch.empty(30)):
        with pytest.raises(ValueError):
            fa._check_rows(bad, (2, 3, 5), dev, "lse")
    ws, nb = fa._workspace(torch.empty(64, dtype=torch.float32), 256, dev)
    assert nb == 256
    with pytest.raises(ValueError):
        fa._workspace(torch.empty(63, dtype=torch.float32), 256, dev)
    with pytest.raises(ValueError):
        fa._workspace(torch.empty(128, dtype=torch.float32)[::2], 256, dev)
    ws, nb = fa._workspace(None, 1000, dev)
    assert nb >= 1000 and ws.device == dev
