"""Pins of the SVD-entropy oracle ([MS] "Muon is Scalable for LLM Training", Sec. 3.4).

The oracle computes H = -(1 / log n) sum q_i log q_i over q_i = sigma_i^2 / sum sigma_j^2
with a library SVD. It is pinned to values that do not come from that code:
* a flat spectrum (orthonormal rows or columns, any scale) gives exactly 1, and a
  rank-one matrix gives 0;
* two-level spectra, with values derived by hand: (4, 1, 1) gives 1 - ln 2 / (3 ln 3),
  (2, 1, 1) gives 3 ln 2 / (2 ln 3), and k copies of a with n - k copies of b give
  (ln T - (k a ln a + (n - k) b ln b) / T) / ln n with T = k a + (n - k) b;
* a 2 x n matrix through the quadratic formula for the eigenvalues of W W^T;
* eigenvalues of W W^T from a symmetric eigensolver, a different library routine;
* invariance under scaling, transposition and orthogonal transforms;
* the readings for zero singular values, one singular value and the zero matrix.
Planted mistakes (sigma instead of sigma^2, log of the larger dimension, a dropped
sign, normalising by sum sigma) are rejected.
"""
import math

import numpy as np
import pytest

from oracle import spectrum_oracle as S


def orthonormal(rows, cols, seed):
    """rows x cols with orthonormal columns (rows >= cols)."""
    q, r = np.linalg.qr(np.random.default_rng(seed).normal(size=(rows, cols)))
    return q * np.sign(np.diag(r))


def with_spectrum(a, b, sigma, seed):
    """An [a, b] matrix whose singular values are `sigma` (length min(a, b))."""
    n = min(a, b)
    assert len(sigma) == n
    p = orthonormal(a, n, seed)
    q = orthonormal(b, n, seed + 1)
    return p @ np.diag(sigma) @ q.T


@pytest.mark.parametrize("shape", [(5, 5), (4, 11), (13, 6), (64, 256)])
def test_flat_spectrum_is_one(shape):
    a, b = shape
    n = min(a, b)
    w = 0.37 * (orthonormal(b, a, 3).T if a <= b else orthonormal(a, b, 3))
    assert abs(S.svd_entropy(w) - 1.0) < 1e-12
    assert np.allclose(S.singular_values_sq(w), 0.37 ** 2, rtol=1e-12, atol=0)
    assert S.singular_values_sq(w).shape == (n,)


@pytest.mark.parametrize("shape", [(6, 6), (3, 40), (50, 7)])
def test_rank_one_is_zero(shape):
    rng = np.random.default_rng(4)
    w = np.outer(rng.normal(size=shape[0]), rng.normal(size=shape[1]))
    assert abs(S.svd_entropy(w)) < 1e-12


def test_hand_derived_three_value_spectra():
    w = with_spectrum(3, 7, [2.0, 1.0, 1.0], 10)  # sigma^2 = (4, 1, 1)
    assert abs(S.svd_entropy(w) - (1.0 - math.log(2.0) / (3.0 * math.log(3.0)))) < 1e-12
    assert abs(S.svd_entropy(w) - 0.789690082142848) < 1e-12
    w = with_spectrum(9, 3, [math.sqrt(2.0), 1.0, 1.0], 12)  # sigma^2 = (2, 1, 1)
    assert abs(S.svd_entropy(w) - 3.0 * math.log(2.0) / (2.0 * math.log(3.0))) < 1e-12
    assert abs(S.svd_entropy(w) - 0.946394630357186) < 1e-12


@pytest.mark.parametrize("n,k,a,b", [(5, 2, 9.0, 1.0), (8, 1, 100.0, 0.25), (6, 3, 2.0, 3.0)])
def test_two_level_spectrum_closed_form(n, k, a, b):
    sig = [math.sqrt(a)] * k + [math.sqrt(b)] * (n - k)
    w = with_spectrum(n, n + 5, sig, 20 + n)
    t = k * a + (n - k) * b
    expect = (math.log(t) - (k * a * math.log(a) + (n - k) * b * math.log(b)) / t) / math.log(n)
    assert abs(S.svd_entropy(w) - expect) < 1e-12
    lam = S.singular_values_sq(w)
    assert np.allclose(lam, sorted([a] * k + [b] * (n - k), reverse=True), rtol=1e-12)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_two_by_n_quadratic_formula(seed):
    w = np.random.default_rng(30 + seed).normal(size=(2, 9))
    g = w @ w.T
    tr, det = g[0, 0] + g[1, 1], g[0, 0] * g[1, 1] - g[0, 1] * g[1, 0]
    disc = math.sqrt(tr * tr - 4.0 * det)
    lam = [(tr + disc) / 2.0, (tr - disc) / 2.0]
    expect = -sum((x / tr) * math.log(x / tr) for x in lam) / math.log(2.0)
    assert abs(S.svd_entropy(w) - expect) < 1e-12
    assert np.allclose(S.singular_values_sq(w), lam, rtol=1e-12)


@pytest.mark.parametrize("shape", [(20, 20), (16, 70), (90, 12)])
def test_agrees_with_eigenvalues_of_the_gram(shape):
    w = np.random.default_rng(40).normal(size=shape) * 0.02
    g = w @ w.T if shape[0] <= shape[1] else w.T @ w
    lam = np.sort(np.linalg.eigvalsh(g))[::-1]
    assert np.allclose(S.singular_values_sq(w), lam, rtol=1e-10, atol=1e-14 * lam[0])
    q = np.clip(lam, 0.0, None) / np.sum(np.clip(lam, 0.0, None))
    h = -np.sum(q[q > 0] * np.log(q[q > 0])) / math.log(min(shape))
    assert abs(S.svd_entropy(w) - h) < 1e-12


def test_invariances():
    rng = np.random.default_rng(50)
    w = rng.normal(size=(12, 30)) * np.linspace(0.1, 3.0, 30)
    h = S.svd_entropy(w)
    assert 0.0 < h < 1.0
    assert abs(S.svd_entropy(7.5 * w) - h) < 1e-13
    assert abs(S.svd_entropy(w.T) - h) < 1e-13
    p, q = orthonormal(12, 12, 51), orthonormal(30, 30, 52)
    assert abs(S.svd_entropy(p @ w @ q) - h) < 1e-12


def test_degenerate_readings():
    # zero singular values count as 0 and still count in n: diag(1, 1, 0) -> ln 2 / ln 3
    w = np.zeros((3, 5))
    w[0, 0] = w[1, 1] = 1.0
    assert abs(S.svd_entropy(w) - math.log(2.0) / math.log(3.0)) < 1e-14
    assert S.svd_entropy(np.array([[3.0, 4.0, 0.0]])) == 0.0  # one singular value
    assert S.svd_entropy(np.ones((6, 1))) == 0.0
    assert math.isnan(S.svd_entropy(np.zeros((4, 6))))  # no spectrum to normalise
    with pytest.raises(ValueError):
        S.svd_entropy(np.zeros(5))


def _sigma_not_squared(w):
    s = np.sqrt(S.singular_values_sq(w))
    return S.entropy_of_spectrum(s)


def _log_of_larger_dim(w):
    return S.svd_entropy(w) * math.log(min(w.shape)) / math.log(max(w.shape))


def _sign_dropped(w):
    return -S.svd_entropy(w)


def _normalised_by_sum_sigma(w):
    lam = S.singular_values_sq(w)
    q = lam / np.sum(np.sqrt(lam))
    return -float(np.sum(q * np.log(q))) / math.log(lam.size)


@pytest.mark.parametrize("mutant", [_sigma_not_squared, _log_of_larger_dim, _sign_dropped,
                                    _normalised_by_sum_sigma])
def test_pins_reject_planted_mistakes(mutant):
    cases = [(with_spectrum(3, 7, [2.0, 1.0, 1.0], 10), 1.0 - math.log(2.0) / (3.0 * math.log(3.0))),
             (0.37 * orthonormal(11, 4, 3).T, 1.0)]
    assert any(abs(mutant(w) - h) > 1e-6 for w, h in cases)
