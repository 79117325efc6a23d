"""Pins of the closed-form fit of the conditional models (oracle/fit.py).

Each check reaches the fitted values by another route than the oracle's:
exact recovery of planted parameters, the ridge minimiser by an augmented
least-squares problem (orthogonal factorisation instead of normal equations),
the Laplace maximum-likelihood scale against the planted scale, and the
missing right neighbour of the last row.
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle import bf16, fit


def _planted(n, C=6, emb=5, seed=0):
    rng = np.random.default_rng(seed)
    e = rng.normal(0, 1, (n, emb))
    H0 = rng.normal(0, 0.5, (C, emb))
    return rng, e, H0


def test_mean_head_recovered_exactly_without_noise():
    rng, e, H0 = _planted(64)
    y = e @ H0.T
    f = fit.fit_coefficients(y, e, 0.0)
    np.testing.assert_allclose(f.H, H0, rtol=0, atol=1e-12)


def test_ridge_minimiser_by_augmented_least_squares():
    rng, e, H0 = _planted(40, seed=1)
    y = e @ H0.T + rng.normal(0, 0.3, (40, 6))
    lam = 0.05
    f = fit.fit_coefficients(y, e, lam)
    n, emb = e.shape
    # min |y - e H^T|^2 + lam n |H|^2  ==  min |[e; sqrt(lam n) I] H^T - [y; 0]|^2
    Ea = np.vstack([e, np.sqrt(lam * n) * np.eye(emb)])
    Ya = np.vstack([y, np.zeros((emb, y.shape[1]))])
    Ht, *_ = np.linalg.lstsq(Ea, Ya, rcond=None)
    np.testing.assert_allclose(f.H, Ht.T, rtol=1e-10, atol=1e-12)
    # the ridge shrinks: the fitted head is smaller than the unregularised one
    assert np.linalg.norm(f.H) < np.linalg.norm(fit.fit_coefficients(y, e, 0.0).H)


def test_neighbour_weights_recovered_on_planted_odd_rows():
    rng, e, H0 = _planted(101, seed=2)
    Hb = bf16.to_f64(bf16.from_f64(H0))
    m = e @ Hb.T
    y = m + rng.normal(0, 1.0, m.shape)          # even rows: anything
    a0 = np.array([0.0, 0.1, 0.25, 0.4, -0.2, 0.33])
    for j in range(1, 101, 2):                     # odd rows from their (even) neighbours
        s = y[j - 1] + (y[j + 1] if j + 1 < 101 else 0.0)
        y[j] = m[j] + a0 * s
    f = fit.fit_coefficients(y, e, 0.0)
    # the refit head reproduces the data's means only approximately (odd rows
    # are not pure means), so compare a against a regression with the refit m
    s = fit.neighbour_sum(y)
    odd = np.arange(1, 101, 2)
    r = y[odd] - f.m[odd]
    for c in range(6):
        a_c = np.dot(r[:, c], s[odd, c]) / np.dot(s[odd, c], s[odd, c])
        assert f.a[c] == pytest.approx(a_c, rel=1e-12, abs=1e-15)
    # planted exactly: odd rows carry no embedding (e = 0, so their mean is 0
    # and they do not move H) and are a0 times their neighbour sum
    e2 = e.copy()
    e2[1::2] = 0.0
    y2 = e2 @ H0.T
    for j in range(1, 101, 2):
        y2[j] = a0 * (y2[j - 1] + (y2[j + 1] if j + 1 < 101 else 0.0))
    f2 = fit.fit_coefficients(y2, e2, 0.0)
    np.testing.assert_allclose(f2.H, H0, atol=1e-12)
    np.testing.assert_allclose(f2.a, a0, rtol=1e-12, atol=1e-15)


def test_last_odd_row_has_no_right_neighbour():
    y = np.arange(1.0, 9.0).reshape(4, 2)  # rows 0..3; row 3 is odd and last
    s = fit.neighbour_sum(y)
    np.testing.assert_array_equal(s[3], y[2])
    np.testing.assert_array_equal(s[1], y[0] + y[2])
    np.testing.assert_array_equal(s[0], y[1])


def test_laplace_scale_is_the_maximum_likelihood_scale():
    rng = np.random.default_rng(7)
    n, C, emb = 200000, 3, 2
    e = np.zeros((n, emb))
    b0 = np.array([0.05, 0.5, 2.0])
    y = rng.laplace(0, b0, (n, C))
    f = fit.fit_coefficients(y, e, 1.0)  # zero embeddings: H = 0, means 0
    assert np.all(f.H == 0)
    # odd rows subtract a * s with a ~ 0 (independent rows): b ~ b0 (1 % at n = 2e5)
    assert np.all(np.abs(f.a) < 0.01)
    np.testing.assert_allclose(f.b, b0, rtol=0.01)
    # and it is the exact mean absolute residual
    mu = np.zeros_like(y)
    odd = np.arange(1, n, 2)
    mu[odd] = f.a.astype(np.float32).astype(np.float64) * fit.neighbour_sum(y)[odd]
    np.testing.assert_allclose(f.b, np.mean(np.abs(y - mu), axis=0), rtol=1e-12)
