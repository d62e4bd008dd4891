"""Seeded synthetic inputs for the BitDelta linear and its compression pass.

This module only draws random tensors.  It holds none of the method's
arithmetic (no sign packing, no scale factor, no reconstruction, no
product): both the CPU oracle and the GPU path receive the same tensors
from here, bit for bit, and compute independently.

Distributions follow the workloads of "BitDelta : servir 14 modèles Zen
depuis un seul cluster GPU" (hanzo-blog, 2026-02-28):

* base weights: bf16 of N(0, 0.02^2) samples;
* fine-tuning deltas: Laplace(0, b), the model stated in the post's
  "Mathematical foundation" section, drawn as b * sgn * E with
  E = -log1p(-U) ~ Exp(1) (U uniform in [0, 1), so U = 0 gives a signed
  zero, which exercises the sign(0) convention) and sgn = -1 or +1 with
  probability 1/2 each;
* activations: bf16 of N(0, 1) samples;
* variant ids: uniform over the G variants;
* per-variant Laplace scales: uniform in [5e-4, 2e-3].

Tensors are drawn in a fixed order from one ``torch.Generator`` seeded per
workload, on whatever device is asked for.  CPU and GPU generators produce
different streams; parity tests therefore always hand the oracle a host
copy of the very tensors the GPU path consumed.
"""

from __future__ import annotations

import torch

# Seeds per workload (tiny, decode, prefill, grouped, full).
SEEDS = {"tiny": 1, "decode": 2, "prefill": 3, "grouped": 4, "full": 5}

# The seven projections of one Llama-70B-shaped transformer layer,
# as (name, d_out, d_in): hidden 8192, 64 query / 8 key-value heads of 128,
# FFN width 28672.
LLAMA70B_LAYER = (
    ("q", 8192, 8192),
    ("k", 1024, 8192),
    ("v", 1024, 8192),
    ("o", 8192, 8192),
    ("gate", 28672, 8192),
    ("up", 28672, 8192),
    ("down", 8192, 28672),
)


def generator(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def base_weight(gen: torch.Generator, d_out: int, d_in: int, device="cpu", std: float = 0.02):
    """bf16 [d_out, d_in] ~ N(0, std^2), rounded to bf16 by torch."""
    w = torch.randn((d_out, d_in), generator=gen, device=device, dtype=torch.float32)
    w.mul_(std)
    return w.to(torch.bfloat16)


def laplace_delta(gen: torch.Generator, d_out: int, d_in: int, b: float = 1e-3, device="cpu"):
    """fp32 [d_out, d_in] ~ Laplace(0, b)."""
    u = torch.rand((d_out, d_in), generator=gen, device=device, dtype=torch.float32)
    e = torch.log1p(u.neg_()).neg_()          # Exp(1); exactly 0 when u == 0
    s = torch.rand((d_out, d_in), generator=gen, device=device, dtype=torch.float32)
    sgn = torch.where(s < 0.5, -1.0, 1.0)
    e.mul_(sgn).mul_(b)
    return e


def base_weight_into(gen: torch.Generator, out: torch.Tensor, tmp: torch.Tensor, std: float = 0.02):
    """``base_weight`` drawn into an existing bf16 tensor (same values for the
    same generator state); ``tmp`` is fp32 scratch of at least ``out.numel()``."""
    t = tmp.view(-1)[: out.numel()].view(out.shape)
    torch.randn(out.shape, generator=gen, out=t)
    t.mul_(std)
    out.copy_(t)
    return out


def laplace_delta_into(gen: torch.Generator, out: torch.Tensor, tmp: torch.Tensor, b: float = 1e-3):
    """``laplace_delta`` drawn into an existing fp32 tensor (same values for the
    same generator state); ``tmp`` is fp32 scratch of at least ``out.numel()``."""
    t = tmp.view(-1)[: out.numel()].view(out.shape)
    torch.rand(out.shape, generator=gen, out=out)
    out.neg_().log1p_().neg_()                 # Exp(1); exactly 0 when u == 0
    torch.rand(out.shape, generator=gen, out=t)
    t.lt_(0.5).mul_(-2.0).add_(1.0)            # -1 where u' < 0.5, else +1
    out.mul_(t).mul_(b)
    return out


def activations(gen: torch.Generator, m: int, d_in: int, device="cpu"):
    """bf16 [m, d_in] ~ N(0, 1)."""
    return torch.randn((m, d_in), generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)


def variant_scales(gen: torch.Generator, g: int, device="cpu", lo: float = 5e-4, hi: float = 2e-3):
    """Per-variant Laplace scales b_g ~ U[lo, hi) as Python floats."""
    r = torch.rand((g,), generator=gen, device=device, dtype=torch.float32)
    return [float(lo + (hi - lo) * v) for v in r.cpu().tolist()]


def variant_ids(gen: torch.Generator, m: int, g: int, device="cpu"):
    """int32 [m] uniform over [0, g)."""
    return torch.randint(0, g, (m,), generator=gen, device=device, dtype=torch.int32)


def request_mix(gen: torch.Generator, requests: int, g: int, device="cpu"):
    """Variant of each request, uniform over the g variants: int32 [requests]."""
    return variant_ids(gen, requests, g, device)


def tiny(device="cpu", seed: int = SEEDS["tiny"]):
    """The tiny single linear: d_out 256, d_in 512, 4 tokens, b = 1e-3."""
    gen = generator(seed, device)
    w = base_weight(gen, 256, 512, device)
    d = laplace_delta(gen, 256, 512, 1e-3, device)
    x = activations(gen, 4, 512, device)
    return w, d, x


def projection(d_out: int, d_in: int, m: int, seed: int, device="cpu", b: float = 1e-3):
    """One projection: (w_base, delta, x)."""
    gen = generator(seed, device)
    w = base_weight(gen, d_out, d_in, device)
    d = laplace_delta(gen, d_out, d_in, b, device)
    x = activations(gen, m, d_in, device)
    return w, d, x


def grouped(d_out: int, d_in: int, m: int, g: int, seed: int = SEEDS["grouped"], device="cpu"):
    """Shared base + g deltas with per-variant scales, m tokens with ids."""
    gen = generator(seed, device)
    w = base_weight(gen, d_out, d_in, device)
    scales = variant_scales(gen, g, device)
    deltas = [laplace_delta(gen, d_out, d_in, b, device) for b in scales]
    x = activations(gen, m, d_in, device)
    ids = variant_ids(gen, m, g, device)
    return w, deltas, scales, x, ids
