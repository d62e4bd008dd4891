"""MonoSoup merge, CPU oracle -- TEST INFRASTRUCTURE ONLY.

Only the tests may import this module.  "BitDelta : servir 14 modèles Zen
depuis un seul cluster GPU" (hanzo-blog, 2026-02-28), section "MonoSoup":
for checkpoints W_1 .. W_k of one base, each task vector Δ_i = W_i - W_base is
replaced by its rank-r truncated SVD τ_i = U_i[:, :r] · diag(S_i[:r]) ·
Vh_i[:r, :], and the merge is W_merged = W_base + (1/k) · Σ_i τ_i.

Plain fp64 numpy; the SVD is LAPACK's (numpy.linalg.svd), used as a library
step exactly as the definition states it.
"""

from __future__ import annotations

import numpy as np


def task_vector(w_i, w_base):
    """Δ_i = W_i - W_base in fp64."""
    return np.asarray(w_i, dtype=np.float64) - np.asarray(w_base, dtype=np.float64)


def truncated(delta, rank: int):
    """τ = the rank-`rank` truncated SVD of Δ (all of Δ when rank >= min(shape))."""
    d = np.asarray(delta, dtype=np.float64)
    u, s, vh = np.linalg.svd(d, full_matrices=False)
    r = min(rank, s.shape[0])
    return (u[:, :r] * s[:r]) @ vh[:r, :]


def merge(w_base, deltas, rank: int):
    """W_merged = W_base + (1/k) Σ τ_i for the k task vectors `deltas`."""
    k = len(deltas)
    acc = np.zeros(np.shape(w_base), dtype=np.float64)
    for d in deltas:
        acc += truncated(d, rank)
    return np.asarray(w_base, dtype=np.float64) + acc / k
