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
def test_merge_is_the_mean_of_truncations(k):
    rng = np.random.default_rng(6 + k)
    base = rng.standard_normal((15, 15))
    deltas = [rng.standard_normal((15, 15)) for _ in range(k)]
    got = ms.merge(base, deltas, rank=4)
    want = base + sum(ms.truncated(d, 4) for d in deltas) / k
    assert np.allclose(got, want, atol=1e-12)
