"""Pins of the differentiable-rate oracle (oracle/rate.py) to things other than itself.

  - the interval probability against scipy's Laplace CDF / survival function;
  - at integer residuals, renormalised over the 255 symbols, the codec plan's
    own symbol model (which builds s = b / step on its own);
  - the probabilities of the unit intervals of any offset grid sum to one;
  - d bits / dt and d bits / ds against central differences of bits_of;
  - every gradient of the total rate (y with the straight-through chain into
    the odd neighbours' means, m, a, b) against central differences of the
    total on a tiny request, with the reconstruction held as its
    straight-through value (yhat = y + a constant offset);
  - the reconstruction is the codec's (integer multiples of the step around
    the conditional mean, within half a step of y; dropped components equal
    the mean), and edge cases (no coded rows, one row, odd N).
"""
from __future__ import annotations

import numpy as np
import pytest
import scipy.stats as st

from oracle import codec as ocodec
from oracle import plan as oplan
from oracle import rate
from tests.tiny import tiny_params, tiny_rows


def _scipy_bits(t, s):
    t = np.asarray(t, dtype=np.float64)
    lo = st.laplace.cdf(t + 0.5, scale=s) - st.laplace.cdf(t - 0.5, scale=s)
    hi = st.laplace.sf(t - 0.5, scale=s) - st.laplace.sf(t + 0.5, scale=s)
    return -np.log2(np.where(t < 0, lo, hi))


@pytest.mark.parametrize("s", [0.05, 0.3, 1.0, 5.0, 40.0])
def test_bits_match_scipy_laplace(s):
    t = np.concatenate([np.linspace(-6, 6, 241), [-0.5, 0.5, 0.4999999, -0.5000001, 0.0]])
    ref = _scipy_bits(t, s)
    got = rate.bits_of(t, s)
    ok = np.isfinite(ref) & (ref < 900)
    assert ok.sum() > 100
    assert np.all(np.abs(got[ok] - ref[ok]) <= 1e-9 * np.maximum(1.0, np.abs(ref[ok])))


def test_bits_at_integers_are_the_codec_symbol_model():
    params = tiny_params(seed=3, n_coef=8)
    b = np.array([0.03, 0.08, 0.2, 0.5, 1.0, 3.0, 12.0, 0.06], dtype=np.float32)
    p = oplan.make_plan(0.7, params["base_step"], b)
    assert 0 < p.c_active < 8
    k = np.arange(-127, 128, dtype=np.float64)
    # rows whose residual is exactly k steps: y = m + k * step, no noise
    N = k.size * 2  # even rows only are read (odd rows add neighbour terms)
    y = np.zeros((N, 8))
    m = np.zeros((N, 8))
    y[0::2] = k[:, None] * p.step.astype(np.float64)[None, :]
    yhat = y.copy()
    r = rate.rate_terms(y, m, yhat, p, np.zeros(8, np.float32), b, np.zeros((N, 8), np.float32))
    bits = r.bits[0::2]
    for rk, c in enumerate(p.act_idx):
        pk = 2.0 ** -bits[:, c]
        np.testing.assert_allclose(pk / pk.sum(), p.pmf[rk], rtol=1e-12, atol=1e-300)
    assert np.all(r.bits[:, ~p.active] == 0)


@pytest.mark.parametrize("s", [0.05, 0.7, 5.0])
@pytest.mark.parametrize("phase", [0.0, 0.3, -0.49])
def test_interval_probabilities_sum_to_one(s, phase):
    k = np.arange(-2000, 2001, dtype=np.float64) + phase
    assert abs(np.sum(2.0 ** -rate.bits_of(k, s)) - 1.0) < 1e-12


@pytest.mark.parametrize("s", [0.05, 0.4, 3.0])
def test_local_derivatives_match_finite_differences(s):
    t = np.concatenate([np.linspace(-3.3, 3.3, 67), [0.0, 0.2, -0.45, 0.55, -0.7]])
    # d bits / dt is continuous at |t| = 1/2 but its own slope jumps there, so
    # central differences straddling that point are left out
    t = t[np.abs(np.abs(t) - 0.5) > 1e-4]
    h = 1e-6
    fd_t = (rate.bits_of(t + h, s) - rate.bits_of(t - h, s)) / (2 * h)
    np.testing.assert_allclose(rate.dbits_dt(t, s), fd_t, rtol=2e-6, atol=2e-6)
    hs = 1e-7 * s
    fd_s = (rate.bits_of(t, s + hs) - rate.bits_of(t, s - hs)) / (2 * hs)
    np.testing.assert_allclose(rate.dbits_ds(t, s), fd_s, rtol=2e-6, atol=2e-6 / s)


def _tiny_request(N, seed):
    params = tiny_params(seed=seed, n_coef=8)
    b = params["laplace_scale"].copy()
    b[[2, 5]] = np.float32(0.01)        # two dropped components
    params["laplace_scale"] = b
    p = oplan.make_plan(0.6, params["base_step"], b)
    assert p.c_active == 6
    T = N + params["keep_head"] + params["keep_tail"]
    rows, tok = tiny_rows(params, T, seed=seed + 1, scale=1.5)
    y, m = rate.coefficients(rows, tok, params)
    u = np.random.default_rng(seed + 2).uniform(-0.5, 0.5, y.shape).astype(np.float32)
    return params, p, rows, tok, y, m, u


@pytest.mark.parametrize("N", [6, 7])
def test_rate_gradients_match_finite_differences(N):
    params, p, _, _, y, m, u = _tiny_request(N, seed=11 + N)
    a = params["nbr_weight"]
    b = params["laplace_scale"]
    r = rate.rate_forward(y, m, p, a, b, u)
    shift = r.yhat - y

    def total(y2=y, m2=m, a2=a, b2=b):
        return rate.rate_terms(y2, m2, y2 + shift, p, a2, b2, u).total

    h = 1e-6
    g_y = np.zeros_like(y)
    g_m = np.zeros_like(m)
    for j in range(N):
        for c in range(y.shape[1]):
            e = np.zeros_like(y)
            e[j, c] = h
            g_y[j, c] = (total(y2=y + e) - total(y2=y - e)) / (2 * h)
            g_m[j, c] = (total(m2=m + e) - total(m2=m - e)) / (2 * h)
    scale = np.max(np.abs(r.g_y))
    np.testing.assert_allclose(r.g_y, g_y, rtol=0, atol=2e-6 * scale)
    np.testing.assert_allclose(r.g_m, g_m, rtol=0, atol=2e-6 * scale)
    # the even rows' reconstruction feeds the odd means: the chain is not zero
    even_chain = r.g_y[0::2] + r.g_m[0::2]
    assert np.max(np.abs(even_chain[:, p.active])) > 1e-3 * scale
    # per-component parameters: the FD of a float64 copy (a, b are rounded to
    # fp32 inside, so perturb through float64 inputs of the same values)
    a64 = a.astype(np.float64)
    b64 = b.astype(np.float64)
    g_a = np.zeros(8)
    g_b = np.zeros(8)
    for c in range(8):
        e = np.zeros(8)
        e[c] = h
        g_a[c] = (_total64(y, m, shift, p, a64 + e, b64, u) - _total64(y, m, shift, p, a64 - e, b64, u)) / (2 * h)
        e[c] = h * b64[c]
        g_b[c] = (_total64(y, m, shift, p, a64, b64 + e, u) - _total64(y, m, shift, p, a64, b64 - e, u)) / (2 * h * b64[c])
    np.testing.assert_allclose(r.g_a, g_a, rtol=1e-6, atol=1e-6 * np.max(np.abs(g_a)))
    np.testing.assert_allclose(r.g_b, g_b, rtol=1e-6, atol=1e-6 * np.max(np.abs(g_b)))
    assert np.all(r.g_a[~p.active] == 0) and np.all(r.g_b[~p.active] == 0)


def _total64(y, m, shift, p, a64, b64, u):
    """The total rate with float64 a and b (the oracle itself rounds them to
    float32 as the codec holds them; the finite difference needs them exact)."""
    N = y.shape[0]
    step = p.step.astype(np.float64)[None, :]
    odd = (np.arange(N) % 2 == 1)[:, None]
    yhat = y + shift
    mu = m + np.where(odd, a64[None, :] * rate.neighbours(yhat), 0.0)
    t = (y - mu) / step + u.astype(np.float64)
    s = (b64 / p.step.astype(np.float64))[None, :]
    return float(np.sum(np.where(p.active[None, :], rate.bits_of(t, s), 0.0)))


def test_reconstruction_is_the_codec_reconstruction():
    params, p, rows, tok, y, m, u = _tiny_request(9, seed=4)
    r = rate.rate_forward(y, m, p, params["nbr_weight"], params["laplace_scale"], u)
    enc = ocodec.encode(rows, tok, params, p)
    np.testing.assert_array_equal(r.q, enc.q)
    np.testing.assert_allclose(r.yhat, enc.yhat, rtol=0, atol=1e-12)
    step = p.step.astype(np.float64)
    k = (r.yhat - r.mu) / step[None, :]
    assert np.allclose(k, np.rint(k), atol=1e-9)
    act = p.active
    assert np.all(np.abs(y - r.yhat)[:, act] <= 0.5 * step[act] * (1 + 1e-6))
    assert np.array_equal(r.yhat[:, ~act], r.mu[:, ~act])
    assert np.all(r.g_y[:, ~act] == 0) and np.all(r.g_m[:, ~act] == 0)


def test_edge_cases():
    params, p, _, _, y, m, u = _tiny_request(1, seed=8)
    a, b = params["nbr_weight"], params["laplace_scale"]
    r = rate.rate_forward(y, m, p, a, b, u)
    # one even row: no neighbour terms anywhere
    np.testing.assert_array_equal(r.g_m, -r.g_y)
    assert np.all(r.g_a == 0)
    r0 = rate.rate_forward(np.zeros((0, 8)), np.zeros((0, 8)), p, a, b, np.zeros((0, 8), np.float32))
    assert r0.total == 0.0 and r0.bits_tok.shape == (0,) and np.all(r0.g_b == 0)
    rows, tok = tiny_rows(params, 3, seed=2)
    y0, m0 = rate.coefficients(rows, tok, params)
    assert y0.shape == (0, 8)


@pytest.mark.parametrize("N", [5, 6])
def test_weight_gradients_match_finite_differences(N):
    """dR/dA and dR/dH against central differences of the total rate through the
    whole forward (y = A x, m = H e recomputed from the perturbed matrix), with
    the reconstruction held at its straight-through value."""
    from oracle import bf16
    params, p, rows, tok, y, m, u = _tiny_request(N, seed=21 + N)
    a, b = params["nbr_weight"], params["laplace_scale"]
    r = rate.rate_forward(y, m, p, a, b, u)
    shift = r.yhat - y
    gA, gH = rate.weight_grads(rows, tok, params, r)
    A = bf16.to_f64(params["analysis"])
    H = bf16.to_f64(params["mean_head"])
    sh = ocodec.shape_of(params)
    _, _, coded_t = ocodec.split_positions(rows.shape[0], sh.keep_head, sh.keep_tail)
    X = bf16.to_f64(rows[coded_t])
    Eg = bf16.to_f64(params["embedding"][tok[coded_t].astype(np.int64)])

    def total(A2, H2):
        y2 = X @ A2.T
        m2 = Eg @ H2.T
        return rate.rate_terms(y2, m2, y2 + shift, p, a, b, u).total

    h = 1e-6
    fA = np.zeros_like(A)
    for c in range(A.shape[0]):
        for d in range(A.shape[1]):
            e = np.zeros_like(A)
            e[c, d] = h
            fA[c, d] = (total(A + e, H) - total(A - e, H)) / (2 * h)
    fH = np.zeros_like(H)
    for c in range(H.shape[0]):
        for k in range(H.shape[1]):
            e = np.zeros_like(H)
            e[c, k] = h
            fH[c, k] = (total(A, H + e) - total(A, H - e)) / (2 * h)
    np.testing.assert_allclose(gA, fA, rtol=0, atol=3e-6 * np.max(np.abs(gA)))
    np.testing.assert_allclose(gH, fH, rtol=0, atol=3e-6 * np.max(np.abs(gH)))
    assert np.all(gA[~p.active] == 0) and np.all(gH[~p.active] == 0)
