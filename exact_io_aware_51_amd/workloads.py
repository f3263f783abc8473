"""Seeded synthetic workloads for fused exact attention.

This module only draws random numbers and names shapes; it holds none of the
attention arithmetic, so the CPU oracle and the HIP path can both take their
inputs from it without sharing any computation.

The five workloads are the shapes the attention path is measured on (the page "How Flash
Attention Works: Tiling, Softmax, GPU I/O" motivates the long-context sizes in
its introduction and in "Why Standard Attention Becomes a GPU Memory I/O
Bottleneck"; the page "attn-flash-equivalence" quotes n = 8192, fp16 in
"Standard attention I/O is the bottleneck").  Layout is [B, H, N, d], d fastest.

Recipe (one CPU generator per workload, seeded 1000 + workload number):
  * draws are fp32, taken in the order Q, K, V, dO;
  * "normal" is N(0, 1); workload c3 multiplies every draw by 0.5 (exact);
  * workload c4 draws V as 2 * U[0, 1) - 1, i.e. U(-1, 1);
  * the fp32 draws are rounded to the I/O dtype (round to nearest even).
The rounded tensors are what the device receives and what the oracle reads.
"""
from __future__ import annotations

import dataclasses
import math

import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    mode: str          # "fwd" or "fwd+bwd"
    dtype: str         # "f32" | "f16" | "bf16"
    B: int
    H: int
    N: int
    d: int
    causal: bool
    q_scale: float = 1.0   # multiplier applied to every draw (Q, K, V, dO); a power of two, so exact
    v_uniform: bool = False
    seed: int = 0

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(d), as the fp32 value handed to the kernels."""
        return float(torch.tensor(1.0 / math.sqrt(self.d), dtype=torch.float32))

    def fwd_flops(self) -> float:
        """4*B*H*N^2*d (two N x N x d products), halved under the causal mask."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    def bwd_flops(self) -> float:
        """10*B*H*N^2*d (five N x N x d products), halved under the causal mask."""
        f = 10.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f


WORKLOADS = {
    "c1": Workload("c1", "fwd", "f32", 1, 2, 256, 64, False, seed=1001),
    "c2": Workload("c2", "fwd", "bf16", 4, 16, 2048, 128, True, seed=1002),
    "c3": Workload("c3", "fwd", "f16", 2, 32, 8192, 64, False, q_scale=0.5, seed=1003),
    "c4": Workload("c4", "fwd", "bf16", 1, 8, 32768, 128, True, v_uniform=True, seed=1004),
    "c5": Workload("c5", "fwd+bwd", "bf16", 2, 16, 4096, 128, True, seed=1005),
}


def make_inputs(w: Workload, with_grad: bool | None = None, seed: int | None = None):
    """Return CPU tensors q, k, v (and do) in the workload's I/O dtype."""
    if with_grad is None:
        with_grad = w.mode == "fwd+bwd"
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed if seed is None else seed)
    shape = (w.B, w.H, w.N, w.d)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    if w.v_uniform:
        v = torch.rand(shape, generator=g, dtype=torch.float32) * 2.0 - 1.0
    else:
        v = torch.randn(shape, generator=g, dtype=torch.float32)
    out = [q, k, v]
    if with_grad:
        out.append(torch.randn(shape, generator=g, dtype=torch.float32))
    if w.q_scale != 1.0:
        out = [x * w.q_scale for x in out]
    dt = DTYPES[w.dtype]
    return tuple(x.to(dt) for x in out)


def shape_case(B, H, N, d, dtype, causal, seed, mode="fwd+bwd", q_scale=1.0):
    """A non-standard shape for parity sweeps, drawn with the same recipe."""
    return Workload(f"B{B}H{H}N{N}d{d}{dtype}{'c' if causal else ''}", mode, dtype,
                    B, H, N, d, causal, q_scale=q_scale, seed=seed)


def kv_inputs(B, H, Nq, Nk, d, dtype, seed, with_grad=True):
    """q [B,H,Nq,d], k and v [B,H,Nk,d] (and do [B,H,Nq,d]): N(0,1) fp32 draws cast to `dtype`."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    q = torch.randn((B, H, Nq, d), generator=g, dtype=torch.float32)
    k = torch.randn((B, H, Nk, d), generator=g, dtype=torch.float32)
    v = torch.randn((B, H, Nk, d), generator=g, dtype=torch.float32)
    out = [q, k, v]
    if with_grad:
        out.append(torch.randn((B, H, Nq, d), generator=g, dtype=torch.float32))
    dt = DTYPES[dtype]
    return tuple(x.to(dt) for x in out)


def block_mask(B, H, N, keep, seed, block=128):
    """uint8 [B, H, nb, nb] block mask, nb = ceil(N / block): each entry 1 with probability `keep`."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    nb = (N + block - 1) // block
    return (torch.rand((B, H, nb, nb), generator=g) < keep).to(torch.uint8)


FP8_FORMATS = {"e4m3": (torch.float8_e4m3fn, 448.0), "e5m2": (torch.float8_e5m2, 57344.0)}


def fp8_inputs(B, H, N, d, seed, q_scale=1.0, v_uniform=False, fmt="e4m3"):
    """OCP 8-bit codes q8, k8, v8 (torch.uint8 [B,H,N,d]) and their dequantisation factors.

    fp32 draws as in make_inputs (N(0,1) times q_scale; V optionally U(-1, 1)),
    then per tensor: descale = the smallest power of two >= amax / fmax (fmax =
    448 for E4M3, 57344 for E5M2), and the code is the rounding (to nearest
    even) of x / descale in format `fmt`, so every code is finite and the
    division is exact.  Returns (q8, k8, v8, (dq, dk, dv)).
    """
    fp8_dtype, fmax = FP8_FORMATS[fmt]
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    shape = (B, H, N, d)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = (torch.rand(shape, generator=g, dtype=torch.float32) * 2.0 - 1.0) if v_uniform else \
        torch.randn(shape, generator=g, dtype=torch.float32)
    codes, descales = [], []
    for x in (q * q_scale, k * q_scale, v * q_scale):
        amax = float(x.abs().max()) if x.numel() else 0.0
        ds = 2.0 ** math.ceil(math.log2(amax / fmax)) if amax > 0 else 1.0
        codes.append((x / ds).to(fp8_dtype).view(torch.uint8).contiguous())
        descales.append(ds)
    return codes[0], codes[1], codes[2], tuple(descales)


def fp8_wide_inputs(B, H, N, d, seed):
    """E5M2 codes q8, k8, v8 (torch.uint8 [B,H,N,d]) whose magnitudes are
    log-uniform over 2^-16 .. 2^15 with random signs (subnormals included,
    no overflow), and dequantisation factors (2^-12, 2^-13, 2^-9) that keep
    the scores at scale 0.125 within tens; code 0x01 (the smallest
    subnormal) fills the first 7 x 3 corner of q's first head."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    codes = []
    for _ in range(3):
        mag = torch.exp2(torch.rand((B, H, N, d), generator=g) * 31.0 - 16.0)
        sign = torch.where(torch.rand((B, H, N, d), generator=g) < 0.5, -1.0, 1.0)
        codes.append((mag * sign).to(torch.float8_e5m2).view(torch.uint8).contiguous())
    codes[0][0, 0, :7, :3] = 0x01
    return codes[0], codes[1], codes[2], (2.0 ** -12, 2.0 ** -13, 2.0 ** -9)
