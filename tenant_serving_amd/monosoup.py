"""MonoSoup merge of several fine-tuned checkpoints of one base, on the GPU.

"BitDelta : servir 14 modèles Zen depuis un seul cluster GPU" (hanzo-blog,
2026-02-28), section "MonoSoup": each checkpoint's task vector
Δ_i = W_i - W_base is replaced by its rank-r truncated SVD τ_i, and the merge
is W_merged = W_base + (1/k)·Σ τ_i.

This is a tool beside the serving path (the post uses it to average training
checkpoints), so it runs on the platform libraries through torch: the rank-r
subspace of each Δ_i comes from a randomized range finder (Halko, Martinsson
and Tropp, "Finding structure with randomness", 2011: a Gaussian test matrix
with r + p columns, q power iterations with re-orthonormalisation), the
products on hipBLASLt and the QR factorisations and the small SVD on
rocSOLVER, all in fp32.  When σ_r of Δ_i clearly exceeds σ_{r+1}, τ_i matches
the exact truncated SVD to within the power iterations' (σ_{r+1}/σ_r)^(2q+1)
factor.
"""

from __future__ import annotations

import torch


def truncated_svd(delta: torch.Tensor, rank: int, oversample: int = 8, power_iters: int = 2,
                  generator: torch.Generator | None = None):
    """(U [m, r], S [r], Vh [r, n]) of the rank-`rank` approximation of the
    fp32 CUDA matrix `delta`."""
    if delta.device.type != "cuda":
        raise ValueError("delta must be on the GPU; there is no CPU path")
    d = delta.float()
    m, n = d.shape
    r = min(rank, m, n)
    width = min(r + oversample, m, n)
    omega = torch.randn((n, width), device=d.device, dtype=torch.float32, generator=generator)
    q, _ = torch.linalg.qr(d @ omega)
    for _ in range(power_iters):
        z, _ = torch.linalg.qr(d.t() @ q)
        q, _ = torch.linalg.qr(d @ z)
    b = q.t() @ d                                   # [width, n]
    ub, s, vh = torch.linalg.svd(b, full_matrices=False)
    u = q @ ub
    return u[:, :r], s[:r], vh[:r, :]


def task_vector_rank_r(delta: torch.Tensor, rank: int, **kw) -> torch.Tensor:
    """τ = U·diag(S)·Vh, the rank-`rank` approximation of Δ (fp32)."""
    u, s, vh = truncated_svd(delta, rank, **kw)
    return (u * s) @ vh


def merge(w_base: torch.Tensor, checkpoints=None, deltas=None, rank: int = 64, seed: int = 0, **kw):
    """W_merged = W_base + (1/k)·Σ τ_i (fp32), from the checkpoints W_i or
    directly from their task vectors Δ_i."""
    if (checkpoints is None) == (deltas is None):
        raise ValueError("give either checkpoints or deltas")
    gen = torch.Generator(device=w_base.device)
    gen.manual_seed(int(seed))
    base = w_base.float()
    items = deltas if deltas is not None else checkpoints
    k = len(items)
    acc = torch.zeros_like(base)
    for it in items:
        d = it.float() if deltas is not None else it.float() - base
        acc += task_vector_rank_r(d, rank, generator=gen, **kw)
    return base + acc / k
