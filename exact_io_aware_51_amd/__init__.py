"""Python binding of libfa, the gfx950 fused exact-attention library.

The functions named like the C entry points (fa_fwd, fa_bwd, fa_fwd_kv,
fa_bwd_kv, fa_fwd_sparse, fa_bwd_sparse, fa_fwd_dropout, fa_bwd_dropout,
fa_fwd_fp8, fa_fwd_fp8_fmt, fa_fwd_kv_split, fa_bwd_workspace_bytes, ...) take raw device
addresses and sizes exactly as include/fa.h declares them.  forward(), backward(), forward_kv(),
backward_kv(), forward_sparse(), backward_sparse(), forward_dropout(),
backward_dropout() and forward_fp8() are conveniences for torch tensors:
they check shapes, allocate the outputs with torch, pass data_ptr()s and
torch's current HIP stream, and raise FaError on a non-zero status.  All
arithmetic happens in the HIP kernels; there is no CPU or PyTorch fallback,
and a missing library is an error.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = ["FA_F32", "FA_F16", "FA_BF16", "FaError", "fa_fwd", "fa_bwd", "fa_bwd_workspace_bytes",
           "fa_bwd_rowsum", "fa_bwd_dkdv", "fa_bwd_dq", "fa_bwd_dq_rowsum", "fa_fwd_kv", "fa_bwd_kv", "fa_fwd_sparse",
           "fa_bwd_sparse", "fa_status_string", "fa_version", "forward", "backward", "forward_kv",
           "backward_kv", "forward_sparse", "backward_sparse", "fa_fwd_dropout", "fa_bwd_dropout",
           "forward_dropout", "backward_dropout", "fa_fwd_fp8", "fa_fwd_fp8_fmt", "forward_fp8", "fa_fwd_kv_split",
           "fa_fwd_kv_split_workspace_bytes", "fa_fwd_kv_split_hint", "fa_bwd_static", "STATIC_SCRATCH_ROWS",
           "FA_FP8_E4M3", "FA_FP8_E5M2",
           "SPARSE_BLOCK", "library_path", "load"]

FA_F32, FA_F16, FA_BF16 = 0, 1, 2
SPARSE_BLOCK = 128  # rows and keys per block of a block-sparse mask (FA_SPARSE_BLOCK)
FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_HIP, FA_ERR_TOO_LARGE = 0, -1, -2, -3, -4, -5
STATIC_SCRATCH_ROWS = 1 << 22  # capacity of fa_bwd_static's device array (FA_STATIC_SCRATCH_ROWS)
FA_FP8_E4M3, FA_FP8_E5M2 = 0, 1  # fa_fp8_format

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

EXPORTS = ("fa_fwd", "fa_bwd", "fa_bwd_workspace_bytes", "fa_bwd_rowsum", "fa_bwd_dkdv", "fa_bwd_dq",
           "fa_fwd_kv", "fa_bwd_kv", "fa_fwd_sparse", "fa_bwd_sparse", "fa_fwd_dropout", "fa_bwd_dropout",
           "fa_fwd_fp8", "fa_fwd_fp8_fmt", "fa_fwd_kv_split", "fa_fwd_kv_split_workspace_bytes",
           "fa_fwd_kv_split_hint", "fa_bwd_static", "fa_bwd_dq_rowsum", "fa_status_string", "fa_version")


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: status {status}: {fa_status_string(status)}")
        self.status = status


def library_path() -> str:
    return os.path.join(_HERE, "libfa.so")


def load() -> ctypes.CDLL:
    """Load libfa.so (built in-tree by exact_io_aware_51_amd.build); raise if it is missing."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m exact_io_aware_51_amd.build` "
                           "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    u64, u32 = ctypes.c_ulonglong, ctypes.c_uint
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
    lib.fa_fwd.restype = i
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, i, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd_static.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
    lib.fa_bwd_static.restype = i
    lib.fa_bwd_rowsum.argtypes = [vp, vp, vp, sz, i, i, i, i, i, vp]
    lib.fa_bwd_rowsum.restype = i
    lib.fa_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, sz, vp, vp, i, i, i, i, f, i, i, vp]
    lib.fa_bwd_dkdv.restype = i
    lib.fa_bwd_dq.argtypes = [vp, vp, vp, vp, vp, vp, sz, vp, i, i, i, i, f, i, i, vp]
    lib.fa_bwd_dq.restype = i
    lib.fa_bwd_dq_rowsum.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, vp, i, i, i, i, f, i, i, vp]
    lib.fa_bwd_dq_rowsum.restype = i
    lib.fa_fwd_kv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp, vp, f, i, i, vp]
    lib.fa_fwd_kv.restype = i
    lib.fa_bwd_kv.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, vp, vp, f, i, i, vp]
    lib.fa_bwd_kv.restype = i
    lib.fa_fwd_sparse.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, vp, f, i, i, vp]
    lib.fa_fwd_sparse.restype = i
    lib.fa_bwd_sparse.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, vp, f, i, i, vp]
    lib.fa_bwd_sparse.restype = i
    lib.fa_fwd_dropout.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, f, u64, u32, i, vp]
    lib.fa_fwd_dropout.restype = i
    lib.fa_bwd_dropout.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, f, u64, u32, i, vp]
    lib.fa_bwd_dropout.restype = i
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, f, f, f, vp]
    lib.fa_fwd_fp8.restype = i
    lib.fa_fwd_fp8_fmt.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, f, f, f, i, vp]
    lib.fa_fwd_fp8_fmt.restype = i
    lib.fa_fwd_kv_split.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp, vp, f, i, i, vp, sz, i, vp]
    lib.fa_fwd_kv_split.restype = i
    lib.fa_fwd_kv_split_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.fa_fwd_kv_split_workspace_bytes.restype = sz
    lib.fa_fwd_kv_split_hint.argtypes = [i, i, i, i, i]
    lib.fa_fwd_kv_split_hint.restype = i
    lib.fa_bwd_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.fa_bwd_workspace_bytes.restype = sz
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = i
    _LIB = lib
    return lib


# ------------------------------------------------------------------ raw C ABI
def fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, stream) -> int:
    return load().fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, stream)


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, N, d, scale, causal,
           dtype, stream) -> int:
    return load().fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, N, d,
                         scale, causal, dtype, stream)


def fa_bwd_static(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype, stream) -> int:
    return load().fa_bwd_static(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype, stream)


def fa_bwd_rowsum(o, dout, workspace, workspace_bytes, B, H, N, d, dtype, stream) -> int:
    return load().fa_bwd_rowsum(o, dout, workspace, workspace_bytes, B, H, N, d, dtype, stream)


def fa_bwd_dkdv(q, k, v, dout, lse, workspace, workspace_bytes, dk, dv, B, H, N, d, scale, causal,
                dtype, stream) -> int:
    return load().fa_bwd_dkdv(q, k, v, dout, lse, workspace, workspace_bytes, dk, dv, B, H, N, d, scale,
                              causal, dtype, stream)


def fa_bwd_dq(q, k, v, dout, lse, workspace, workspace_bytes, dq, B, H, N, d, scale, causal, dtype,
              stream) -> int:
    return load().fa_bwd_dq(q, k, v, dout, lse, workspace, workspace_bytes, dq, B, H, N, d, scale, causal,
                            dtype, stream)


def fa_bwd_dq_rowsum(q, k, v, o, dout, lse, workspace, workspace_bytes, dq, B, H, N, d, scale, causal, dtype,
                     stream) -> int:
    return load().fa_bwd_dq_rowsum(q, k, v, o, dout, lse, workspace, workspace_bytes, dq, B, H, N, d, scale,
                                   causal, dtype, stream)


def fa_fwd_kv(q, k, v, o, lse, B, H, Nq, Nk, d, seqlens_q, seqlens_k, scale, causal, dtype, stream) -> int:
    return load().fa_fwd_kv(q, k, v, o, lse, B, H, Nq, Nk, d, seqlens_q, seqlens_k, scale, causal, dtype, stream)


def fa_bwd_kv(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, Nq, Nk, d, seqlens_q,
              seqlens_k, scale, causal, dtype, stream) -> int:
    return load().fa_bwd_kv(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, Nq, Nk, d,
                            seqlens_q, seqlens_k, scale, causal, dtype, stream)


def fa_fwd_sparse(q, k, v, o, lse, B, H, N, d, block_mask, scale, causal, dtype, stream) -> int:
    return load().fa_fwd_sparse(q, k, v, o, lse, B, H, N, d, block_mask, scale, causal, dtype, stream)


def fa_bwd_sparse(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, N, d, block_mask,
                  scale, causal, dtype, stream) -> int:
    return load().fa_bwd_sparse(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, N, d,
                                block_mask, scale, causal, dtype, stream)


def fa_fwd_dropout(q, k, v, o, lse, B, H, N, d, scale, causal, dropout_p, seed, offset, dtype, stream) -> int:
    return load().fa_fwd_dropout(q, k, v, o, lse, B, H, N, d, scale, causal, dropout_p, seed, offset, dtype,
                                 stream)


def fa_bwd_dropout(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, N, d, scale, causal,
                   dropout_p, seed, offset, dtype, stream) -> int:
    return load().fa_bwd_dropout(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, N, d,
                                 scale, causal, dropout_p, seed, offset, dtype, stream)


def fa_fwd_fp8(q, k, v, o, lse, B, H, N, d, scale, causal, descale_q, descale_k, descale_v, stream) -> int:
    return load().fa_fwd_fp8(q, k, v, o, lse, B, H, N, d, scale, causal, descale_q, descale_k, descale_v, stream)


def fa_fwd_fp8_fmt(q, k, v, o, lse, B, H, N, d, scale, causal, descale_q, descale_k, descale_v, fmt, stream) -> int:
    return load().fa_fwd_fp8_fmt(q, k, v, o, lse, B, H, N, d, scale, causal, descale_q, descale_k, descale_v, fmt,
                                 stream)


def fa_fwd_kv_split(q, k, v, o, lse, B, H, Nq, Nk, d, seqlens_q, seqlens_k, scale, causal, num_splits, workspace,
                    workspace_bytes, dtype, stream) -> int:
    return load().fa_fwd_kv_split(q, k, v, o, lse, B, H, Nq, Nk, d, seqlens_q, seqlens_k, scale, causal, num_splits,
                                  workspace, workspace_bytes, dtype, stream)


def fa_fwd_kv_split_workspace_bytes(B, H, Nq, Nk, d, num_splits) -> int:
    return load().fa_fwd_kv_split_workspace_bytes(B, H, Nq, Nk, d, num_splits)


def fa_fwd_kv_split_hint(B, H, Nq, Nk, d) -> int:
    return load().fa_fwd_kv_split_hint(B, H, Nq, Nk, d)


def fa_bwd_workspace_bytes(B, H, N, d, dtype) -> int:
    return load().fa_bwd_workspace_bytes(B, H, N, d, dtype)


def fa_status_string(status: int) -> str:
    return load().fa_status_string(status).decode()


def fa_version() -> int:
    return load().fa_version()


# ------------------------------------------------------------ torch helpers
def _dtype_code(t):
    import torch
    codes = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _check(*ts):
    import torch
    ref = ts[0]
    if ref.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    for t in ts:
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise ValueError("tensors must live on a HIP device (no CPU path exists)")
        if t.shape != ref.shape or t.dtype != ref.dtype or t.device != ref.device:
            raise ValueError("q, k, v (, o, dout) must share shape, dtype and device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous [B, H, N, d]")


def _check_like(t, ref, what):
    """t must be a contiguous tensor with ref's shape, dtype and device."""
    import torch
    if not isinstance(t, torch.Tensor) or t.device != ref.device or t.dtype != ref.dtype:
        raise ValueError(f"{what} must be a {ref.dtype} tensor on {ref.device}")
    if tuple(t.shape) != tuple(ref.shape) or not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous with shape {tuple(ref.shape)}")
    return t


def _check_rows(t, shape, device, what):
    """t must be a contiguous float32 tensor of `shape` on `device` (LSE and row vectors)."""
    import torch
    if not isinstance(t, torch.Tensor) or t.device != device or t.dtype != torch.float32:
        raise ValueError(f"{what} must be a float32 tensor on {device}")
    if tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous with shape {tuple(shape)}")
    return t


def _workspace(workspace, need, device):
    """A caller's workspace (checked: device, contiguous, large enough) or a new one; returns (tensor, bytes)."""
    import torch
    if workspace is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
        return ws, ws.numel()
    if not isinstance(workspace, torch.Tensor) or workspace.device != device or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}")
    nbytes = workspace.numel() * workspace.element_size()
    if nbytes < need:
        raise ValueError(f"workspace holds {nbytes} bytes, {need} needed")
    return workspace, nbytes


def _stream(t, stream):
    import torch
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def forward(q, k, v, scale=None, causal=False, out=None, lse=None, need_lse=True, stream=None):
    """O, LSE = softmax(scale q k^T [+ causal mask]) v on the GPU.  scale defaults to 1/sqrt(d)."""
    import torch
    _check(q, k, v)
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else _check_like(out, q, "out")
    if lse is not None:
        _check_rows(lse, (B, H, N), q.device, "lse")
    elif need_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    st = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                lse.data_ptr() if lse is not None else None, B, H, N, d, scale, int(bool(causal)),
                _dtype_code(q), _stream(q, stream))
    if st != FA_OK:
        raise FaError(st, "fa_fwd")
    return o, lse


def backward(q, k, v, o, lse, dout, scale=None, causal=False, workspace=None, stream=None):
    """dQ, dK, dV of sum(dout * o) on the GPU, recomputing the score tiles from lse."""
    import torch
    _check(q, k, v, o, dout)
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    code = _dtype_code(q)
    _check_rows(lse, (B, H, N), q.device, "lse")
    workspace, wsb = _workspace(workspace, fa_bwd_workspace_bytes(B, H, N, d, code), q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    st = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), wsb,
                B, H, N, d, scale, int(bool(causal)), code, _stream(q, stream))
    if st != FA_OK:
        raise FaError(st, "fa_bwd")
    return dq, dk, dv


def _check_kv(q, k, v, extra_q=(), extra_k=()):
    import torch
    for t in (q, k, v, *extra_q, *extra_k):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise ValueError("tensors must live on a HIP device (no CPU path exists)")
        if t.dim() != 4 or not t.is_contiguous() or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("expected contiguous [B, H, N, d] tensors of one dtype and device")
    B, H, Nq, d = q.shape
    for t in (k, v, *extra_k):
        if t.shape[:2] != (B, H) or t.shape[3] != d or t.shape[2] != k.shape[2]:
            raise ValueError("k and v must be [B, H, Nk, d] with q's B, H and d")
    for t in extra_q:
        if t.shape != q.shape:
            raise ValueError("o and dout must have q's shape")
    return B, H, Nq, k.shape[2], d


def _lengths(t, B, device):
    import torch
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        t = torch.tensor(list(t), dtype=torch.int32, device=device)
    if t.device != device or t.dtype != torch.int32 or t.numel() != B or not t.is_contiguous():
        raise ValueError("sequence lengths must be a contiguous int32 device tensor of B entries")
    return t


def forward_kv(q, k, v, seqlens_q=None, seqlens_k=None, scale=None, causal=False, need_lse=True, stream=None):
    """fa_fwd_kv on torch tensors: q [B,H,Nq,d], k/v [B,H,Nk,d], optional per-sequence lengths.

    Under the causal mask the queries are the last positions of their key sequence
    (query i sees key j iff j <= i + lk - lq); padding rows get O = 0, LSE = -inf.
    """
    import torch
    B, H, Nq, Nk, d = _check_kv(q, k, v)
    sq, sk = _lengths(seqlens_q, B, q.device), _lengths(seqlens_k, B, q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if need_lse else None
    st = fa_fwd_kv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                   lse.data_ptr() if lse is not None else None, B, H, Nq, Nk, d,
                   sq.data_ptr() if sq is not None else None, sk.data_ptr() if sk is not None else None,
                   scale, int(bool(causal)), _dtype_code(q), _stream(q, stream))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_kv")
    return o, lse


def backward_kv(q, k, v, o, lse, dout, seqlens_q=None, seqlens_k=None, scale=None, causal=False, stream=None):
    """fa_bwd_kv on torch tensors (o and lse from forward_kv with the same arguments)."""
    import torch
    B, H, Nq, Nk, d = _check_kv(q, k, v, extra_q=(o, dout))
    sq, sk = _lengths(seqlens_q, B, q.device), _lengths(seqlens_k, B, q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    code = _dtype_code(q)
    _check_rows(lse, (B, H, Nq), q.device, "lse")
    workspace, _ = _workspace(None, fa_bwd_workspace_bytes(B, H, Nq, d, code), q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    st = fa_bwd_kv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                   dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), workspace.numel(),
                   B, H, Nq, Nk, d, sq.data_ptr() if sq is not None else None,
                   sk.data_ptr() if sk is not None else None, scale, int(bool(causal)), code, _stream(q, stream))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_kv")
    return dq, dk, dv


def _block_mask(m, B, H, N, device):
    import torch
    nb = (N + SPARSE_BLOCK - 1) // SPARSE_BLOCK
    if not isinstance(m, torch.Tensor) or m.device != device or m.dtype != torch.uint8:
        raise ValueError("block_mask must be a uint8 tensor on the tensors' device")
    if tuple(m.shape) != (B, H, nb, nb) or not m.is_contiguous():
        raise ValueError(f"block_mask must be contiguous [B, H, {nb}, {nb}] (blocks of {SPARSE_BLOCK})")
    return m


def forward_sparse(q, k, v, block_mask, scale=None, causal=False, need_lse=True, stream=None):
    """fa_fwd_sparse on torch tensors: block_mask uint8 [B, H, nb, nb], 0 removes a 128 x 128 block."""
    import torch
    _check(q, k, v)
    B, H, N, d = q.shape
    m = _block_mask(block_mask, B, H, N, q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if need_lse else None
    st = fa_fwd_sparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                       lse.data_ptr() if lse is not None else None, B, H, N, d, m.data_ptr(), scale,
                       int(bool(causal)), _dtype_code(q), _stream(q, stream))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_sparse")
    return o, lse


def backward_sparse(q, k, v, o, lse, dout, block_mask, scale=None, causal=False, stream=None):
    """fa_bwd_sparse on torch tensors (o and lse from forward_sparse with the same mask)."""
    import torch
    _check(q, k, v, o, dout)
    B, H, N, d = q.shape
    m = _block_mask(block_mask, B, H, N, q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    code = _dtype_code(q)
    _check_rows(lse, (B, H, N), q.device, "lse")
    workspace, _ = _workspace(None, fa_bwd_workspace_bytes(B, H, N, d, code), q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    st = fa_bwd_sparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                       dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), workspace.numel(),
                       B, H, N, d, m.data_ptr(), scale, int(bool(causal)), code, _stream(q, stream))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_sparse")
    return dq, dk, dv


def forward_dropout(q, k, v, dropout_p, seed, offset=0, scale=None, causal=False, need_lse=True, stream=None):
    """fa_fwd_dropout on torch tensors: O = (P o Z) v with a Philox keep mask drawn from (seed, offset)."""
    import torch
    _check(q, k, v)
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if need_lse else None
    st = fa_fwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                        lse.data_ptr() if lse is not None else None, B, H, N, d, scale, int(bool(causal)),
                        float(dropout_p), int(seed), int(offset), _dtype_code(q), _stream(q, stream))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_dropout")
    return o, lse


def backward_dropout(q, k, v, o, lse, dout, dropout_p, seed, offset=0, scale=None, causal=False, stream=None):
    """fa_bwd_dropout on torch tensors (o and lse from forward_dropout with the same mask arguments)."""
    import torch
    _check(q, k, v, o, dout)
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    code = _dtype_code(q)
    _check_rows(lse, (B, H, N), q.device, "lse")
    workspace, _ = _workspace(None, fa_bwd_workspace_bytes(B, H, N, d, code), q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    st = fa_bwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), workspace.numel(),
                        B, H, N, d, scale, int(bool(causal)), float(dropout_p), int(seed), int(offset), code,
                        _stream(q, stream))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_dropout")
    return dq, dk, dv


def forward_fp8(q8, k8, v8, descale_q=1.0, descale_k=1.0, descale_v=1.0, scale=None, causal=False, need_lse=True,
                stream=None, fmt="e4m3"):
    """fa_fwd_fp8_fmt on torch tensors: 8-bit codes [B, H, N, d] in, bf16 O and fp32 LSE out.

    fmt is "e4m3" (codes as uint8 or float8_e4m3fn) or "e5m2" (uint8 or float8_e5m2)."""
    import torch
    formats = {"e4m3": (FA_FP8_E4M3, torch.float8_e4m3fn), "e5m2": (FA_FP8_E5M2, torch.float8_e5m2)}
    if fmt not in formats:
        raise ValueError(f"fmt must be one of {sorted(formats)}")
    code, fp8_dtype = formats[fmt]
    codes = []
    for t in (q8, k8, v8):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise ValueError("tensors must live on a HIP device (no CPU path exists)")
        if t.dtype == fp8_dtype:
            t = t.view(torch.uint8)
        if t.dtype != torch.uint8 or t.dim() != 4 or not t.is_contiguous() or t.shape != q8.shape:
            raise ValueError(f"q8, k8, v8 must be contiguous [B, H, N, d] {fmt.upper()} codes of one shape")
        codes.append(t)
    B, H, N, d = q8.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device) if need_lse else None
    st = fa_fwd_fp8_fmt(codes[0].data_ptr(), codes[1].data_ptr(), codes[2].data_ptr(), o.data_ptr(),
                        lse.data_ptr() if lse is not None else None, B, H, N, d, scale, int(bool(causal)),
                        float(descale_q), float(descale_k), float(descale_v), code, _stream(q8, stream))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_fp8_fmt")
    return o, lse


def forward_kv_split(q, k, v, seqlens_q=None, seqlens_k=None, scale=None, causal=False, num_splits=None,
                     need_lse=True, stream=None):
    """fa_fwd_kv_split on torch tensors; num_splits=None takes fa_fwd_kv_split_hint's value."""
    import torch
    B, H, Nq, Nk, d = _check_kv(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if num_splits is None:
        num_splits = fa_fwd_kv_split_hint(B, H, Nq, Nk, d)
    need = fa_fwd_kv_split_workspace_bytes(B, H, Nq, Nk, d, num_splits)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if need_lse else None
    sq, sk = _lengths(seqlens_q, B, q.device), _lengths(seqlens_k, B, q.device)
    st = fa_fwd_kv_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                         lse.data_ptr() if lse is not None else None, B, H, Nq, Nk, d,
                         sq.data_ptr() if sq is not None else None, sk.data_ptr() if sk is not None else None,
                         scale, int(bool(causal)), int(num_splits), ws.data_ptr(), ws.numel(), _dtype_code(q),
                         _stream(q, stream))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_kv_split")
    return o, lse
