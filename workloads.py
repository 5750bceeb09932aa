"""Seeded synthetic workloads for quantized attention (shared by tests and bench).

This module only draws inputs; it holds none of the method's arithmetic.  It
stands in for the long-context video-model activations the pages measure on
(37,810 tokens, 56 heads, head dimension 128), which are not available.

Recipe (CPU, ``torch.Generator`` seeded per workload), in this draw order:
  1. Q  = randn [B, N, H, 128]              (float32)
  2. K  = randn [B, N, H, 128]
  3. K += 3 * randn [H, 128]                 per-channel offset, constant over
                                             tokens (standard deviation 3)
  4. V  = randn [B, N, H, 128]
  5. outliers (Mid only): randperm(H*128)[:round(0.01*H*128)] channels of K,
     offset included, are multiplied by 8
  6. round each tensor to BF16 (round to nearest even)
Optional RMSNorm + RoPE parameters (``norm_rope_params``): weights
1 + 0.2 * randn [128] for Q and for K (FP32), the rotary angle table of 1-D
positions n = 0..N-1 with frequencies 10000^(-i/64), i = 0..63, evaluated in
float64 and rounded to FP32, and eps = 1e-6.
Layouts: "separate" gives three contiguous [B, N, H, 128] tensors;
"projection" gives three strided views into one BF16 buffer [B, N, 3*H*128]
(Q, K, V as consecutive column slices), so stride_n = 3*H*128.
"""
from dataclasses import dataclass
from typing import Optional

import torch

HD = 128


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    N: int
    H: int
    seed: int
    layout: str = "separate"        # "separate" | "projection"
    outlier_frac: float = 0.0       # fraction of K channels scaled by 8


def tiny() -> Workload:
    return Workload("tiny", 1, 200, 2, seed=0)


def sweep(n: int) -> Workload:
    return Workload("sweep_n%d" % n, 1, n, 4, seed=100 + n)


SWEEP_NS = (64, 128, 192, 256, 65, 127, 129)


def mid() -> Workload:
    return Workload("mid", 1, 4096, 8, seed=1, outlier_frac=0.01)


def large() -> Workload:
    return Workload("large", 1, 8192, 56, seed=2, layout="projection")


def canonical() -> Workload:
    return Workload("canonical", 1, 37810, 56, seed=3, layout="projection")


def by_name(name: str) -> Workload:
    if name.startswith("sweep_n"):
        return sweep(int(name[len("sweep_n"):]))
    return {"tiny": tiny, "mid": mid, "large": large, "canonical": canonical}[name]()


@dataclass
class Inputs:
    q: torch.Tensor      # BF16 [B, N, H, 128] view (CPU unless moved)
    k: torch.Tensor
    v: torch.Tensor
    buffer: Optional[torch.Tensor] = None   # the projection buffer, if any


def generate(w: Workload, device: str = "cpu") -> Inputs:
    """Draw the workload on the CPU and return BF16 tensors on ``device``."""
    g = torch.Generator(device="cpu").manual_seed(w.seed)
    shape = (w.B, w.N, w.H, HD)
    if w.layout == "projection":
        buf = torch.empty((w.B, w.N, 3 * w.H * HD), dtype=torch.bfloat16)
        views = [buf[:, :, i * w.H * HD:(i + 1) * w.H * HD].view(w.B, w.N, w.H, HD)
                 for i in range(3)]
    else:
        buf = None
        views = [torch.empty(shape, dtype=torch.bfloat16) for _ in range(3)]
    q = torch.randn(shape, generator=g)
    views[0].copy_(q)
    del q
    k = torch.randn(shape, generator=g)
    k += 3.0 * torch.randn((w.H, HD), generator=g)
    kview = k  # outliers applied after V is drawn (fixed draw order)
    v = torch.randn(shape, generator=g)
    views[2].copy_(v)
    del v
    if w.outlier_frac > 0:
        n_out = int(round(w.outlier_frac * w.H * HD))
        idx = torch.randperm(w.H * HD, generator=g)[:n_out]
        flat = kview.view(w.B, w.N, w.H * HD)
        flat[:, :, idx] *= 8.0
    views[1].copy_(kview)
    del k, kview
    if device != "cpu":
        if buf is not None:
            buf = buf.to(device)
            views = [buf[:, :, i * w.H * HD:(i + 1) * w.H * HD].view(w.B, w.N, w.H, HD)
                     for i in range(3)]
        else:
            views = [t.to(device) for t in views]
    return Inputs(views[0], views[1], views[2], buf)


@dataclass
class NormRopeParams:
    q_weight: torch.Tensor   # FP32 [128]
    k_weight: torch.Tensor   # FP32 [128]
    cos: torch.Tensor        # FP32 [N, 64], row n = token n
    sin: torch.Tensor        # FP32 [N, 64]
    eps: float = 1e-6


def norm_rope_params(N: int, seed: int = 7, device: str = "cpu") -> NormRopeParams:
    """Seeded RMSNorm weights and a rotary angle table for N tokens."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    qw = 1.0 + 0.2 * torch.randn(HD, generator=g)
    kw = 1.0 + 0.2 * torch.randn(HD, generator=g)
    pos = torch.arange(N, dtype=torch.float64)[:, None]
    freq = 10000.0 ** (-torch.arange(HD // 2, dtype=torch.float64) / (HD // 2))
    ang = pos * freq[None, :]
    cos = torch.cos(ang).to(torch.float32)
    sin = torch.sin(ang).to(torch.float32)
    return NormRopeParams(qw.to(device), kw.to(device), cos.to(device), sin.to(device), 1e-6)


def with_padding_rows(x: torch.Tensor, extra: int, fill_seed: int = 12345) -> torch.Tensor:
    """Copy of x [B,N,H,D] stored inside a larger buffer whose rows N..N+extra-1
    hold random garbage; returns the [B,N,H,D] view (for padding-independence tests)."""
    B, N, H, D = x.shape
    g = torch.Generator(device="cpu").manual_seed(fill_seed)
    big = (torch.randn((B, N + extra, H, D), generator=g) * 100.0).to(torch.bfloat16)
    big = big.to(x.device)
    big[:, :N].copy_(x)
    return big[:, :N]
