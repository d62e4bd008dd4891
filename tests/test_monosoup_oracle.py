"""Pins of the MonoSoup oracle against what the definition and linear
algebra fix, independently of LAPACK's SVD where possible."""

import numpy as np
import pytest

from oracle import monosoup as ms


def _rank_r(rng, m, n, r, scale=1.0):
    return scale * (rng.standard_normal((m, r)) @ rng.standard_normal((r, n)))


def test_exact_low_rank_task_vectors_pass_through():
    rng = np.random.default_rng(1)
    base = rng.standard_normal((40, 30))
    deltas = [_rank_r(rng, 40, 30, 3) for _ in range(4)]
    got = ms.merge(base, deltas, rank=3)
    want = base + sum(deltas) / 4          # τ_i = Δ_i, and the mean, not the sum
    assert np.allclose(got, want, rtol=0, atol=1e-10)


def test_full_rank_keeps_everything():
    rng = np.random.default_rng(2)
    d = rng.standard_normal((7, 5))
    assert np.allclose(ms.truncated(d, 5), d, atol=1e-12)
    assert np.allclose(ms.truncated(d, 9), d, atol=1e-12)


def test_eckart_young_residual():
    # ||Δ - τ||_F^2 = Σ_{j>r} σ_j^2, with σ from the eigenvalues of ΔᵀΔ
    # (a different routine from the SVD the oracle uses)
    rng = np.random.default_rng(3)
    d = rng.standard_normal((50, 20))
    lam = np.sort(np.linalg.eigvalsh(d.T @ d))[::-1]
    for r in (1, 4, 11):
        res = np.linalg.norm(d - ms.truncated(d, r)) ** 2
        assert abs(res - lam[r:].sum()) <= 1e-9 * lam.sum()


def test_rank_one_by_power_iteration():
    # brute force: the dominant singular pair by plain power iteration
    rng = np.random.default_rng(4)
    d = rng.standard_normal((6, 4))
    v = np.ones(4)
    for _ in range(2000):
        v = d.T @ (d @ v)
        v /= np.linalg.norm(v)
    u = d @ v
    sigma = np.linalg.norm(u)
    tau = np.outer(u / sigma, v) * sigma
    assert np.allclose(ms.truncated(d, 1), tau, atol=1e-9)


def test_single_checkpoint_and_task_vector():
    rng = np.random.default_rng(5)
    base = rng.standard_normal((12, 9))
    w1 = base + _rank_r(rng, 12, 9, 2)
    d = ms.task_vector(w1, base)
    assert np.allclose(ms.merge(base, [d], rank=2), w1, atol=1e-10)
    # truncating below the true rank drops exactly the smallest direction
    tau1 = ms.truncated(d, 1)
    assert np.linalg.matrix_rank(tau1, tol=1e-8) == 1
    s = np.linalg.svd(d, compute_uv=False)
    assert abs(np.linalg.norm(d - tau1) - s[1]) <= 1e-9 * s[0]


@pytest.mark.parametrize("k", [2, 3])
def test_merge_of_task_vectors_with_known_svd(k):
    # Each task vector is built from its own SVD: Δ_i = U_i·diag(s_i)·V_iᵀ with
    # orthonormal U_i, V_i (QR of Gaussian matrices) and distinct singular
    # values s_i.  Its rank-r truncation is then U_i[:, :r]·diag(s_i[:r])·
    # V_i[:, :r]ᵀ by construction (Eckart-Young), so the expected merge comes
    # from the construction, not from the oracle's own truncation or an SVD.
    rng = np.random.default_rng(6 + k)
    m, n, r = 15, 12, 4
    base = rng.standard_normal((m, n))
    deltas, kept = [], []
    for i in range(k):
        u, _ = np.linalg.qr(rng.standard_normal((m, n)))
        v, _ = np.linalg.qr(rng.standard_normal((n, n)))
        s = np.sort(rng.uniform(0.5, 3.0, size=n))[::-1] + np.linspace(0.5, 0.0, n)  # distinct, descending
        deltas.append((u * s) @ v.T)
        kept.append((u[:, :r] * s[:r]) @ v[:, :r].T)
    got = ms.merge(base, deltas, rank=r)
    want = base + sum(kept) / k
    assert np.allclose(got, want, rtol=0, atol=1e-10)
    # and a sum instead of the mean, or the untruncated Δ, would be caught
    assert not np.allclose(got, base + sum(kept), atol=1e-3)
    assert not np.allclose(got, base + sum(deltas) / k, atol=1e-3)
