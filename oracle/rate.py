"""Differentiable rate of the training objective (CPU, float64).

Test infrastructure: only tests, the package's smoke check and the
benchmark's CPU-baseline leg use this module.

Source: DCKV digest page (trove.briskstack.com, "DCKV: Learned Transform
Coding of the Prompt KV Cache in Hybrid Language Models"), section "How it
works", Training bullet: the loss adds the code length to a distortion term;
the rate is computed on coefficients with additive noise, and the
reconstruction uses rounded values whose gradient passes straight through.
The kongchang.com article "DCKV：端到端学习的KV缓存编解码器，压缩超百倍"
(its note on differentiable quantisation) names the same two devices:
additive uniform noise and the straight-through estimator.  The distortion term needs the language model and
is not computed here.

Readings taken where the pages are silent:
  * The rate of coefficient c of coded row j is the code length of the noisy
    residual under the codec's own Laplace model, in quantisation steps:
        t = (y - mu) / step + u,   u ~ U(-1/2, 1/2) (an input),
        bits = -log2( F_s(t + 1/2) - F_s(t - 1/2) ),  s = b / step,
    F_s the zero-mean Laplace CDF of scale s.  At integer t this is the code
    length of the codec's (unrenormalised) symbol probability.
  * mu is the codec's conditional mean: the embedding mean m_j for even j;
    m_j + a * (yhat_{j-1} + yhat_{j+1}) for odd j (yhat_N = 0).  The
    neighbours are the reconstruction: the codec's two-pass quantisation
    (rounded values), whose straight-through gradient is d yhat / d y = 1 and
    d yhat / d mu = 0.
  * Only active components carry a rate; dropped ones have bits 0, yhat = mu
    and no gradient.  Escapes are not charged separately (the likelihood
    alone is the training rate).
  * Outputs are the total R = sum of bits and its gradients with respect to
    the coefficients y, the embedding means m, the neighbour weights a and the
    Laplace scales b, and through y = A x and m = H e those with respect to
    the analysis matrix A and the mean head H.  Steps are held fixed.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import bf16
from . import codec as ocodec
from .plan import Plan

LN2 = float(np.log(2.0))


def bits_of(t: np.ndarray, s: np.ndarray) -> np.ndarray:
    """-log2(F_s(t + 1/2) - F_s(t - 1/2)) for the zero-mean Laplace of scale s.

    For |t| >= 1/2 the interval lies on one side of 0 and the probability is
    (1/2) exp(-(|t| - 1/2)/s) (1 - exp(-1/s)); inside, it is one minus the two
    tails (1/2) exp(-(1/2 -+ |t|)/s).  Both forms avoid cancellation."""
    t = np.asarray(t, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    at = np.abs(t)
    with np.errstate(over="ignore", divide="ignore", invalid="ignore"):
        out_side = 1.0 + (at - 0.5) / (s * LN2) - np.log2(-np.expm1(-1.0 / s))
        p_in = -0.5 * (np.expm1(-(0.5 - at) / s) + np.expm1(-(0.5 + at) / s))
        in_side = -np.log2(p_in)
    return np.where(at >= 0.5, out_side, in_side)


def dbits_dt(t: np.ndarray, s: np.ndarray) -> np.ndarray:
    """d bits / d t: sign(t) / (s ln 2) outside the central interval; inside,
    (e1 - e2) / (2 s P ln 2) with e1 = exp(-(1/2 - t)/s), e2 = exp(-(1/2 + t)/s)
    (the two densities at the interval's ends) and P the probability."""
    t = np.asarray(t, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    at = np.abs(t)
    with np.errstate(over="ignore", divide="ignore", invalid="ignore"):
        e1 = np.exp(-(0.5 - t) / s)
        e2 = np.exp(-(0.5 + t) / s)
        p_in = -0.5 * (np.expm1(-(0.5 - at) / s) + np.expm1(-(0.5 + at) / s))
        inside = (e1 - e2) / (2.0 * s * p_in * LN2)
    return np.where(at >= 0.5, np.sign(t) / (s * LN2), inside)


def dbits_ds(t: np.ndarray, s: np.ndarray) -> np.ndarray:
    """d bits / d s: (1/expm1(1/s) - (|t| - 1/2)) / (s^2 ln 2) outside;
    (e1 a1 + e2 a2) / (2 s P ln 2) inside, a1 = (1/2 - |t|)/s, a2 = (1/2 + |t|)/s,
    e_i = exp(-a_i)."""
    t = np.asarray(t, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    at = np.abs(t)
    with np.errstate(over="ignore", divide="ignore", invalid="ignore"):
        outside = (1.0 / np.expm1(1.0 / s) - (at - 0.5)) / (s * s * LN2)
        a1 = (0.5 - at) / s
        a2 = (0.5 + at) / s
        p_in = -0.5 * (np.expm1(-a1) + np.expm1(-a2))
        inside = (np.exp(-a1) * a1 + np.exp(-a2) * a2) / (2.0 * s * p_in * LN2)
    return np.where(at >= 0.5, outside, inside)


@dataclass
class Rate:
    bits: np.ndarray      # float64 [N][C] per-coefficient code length (0 for dropped)
    bits_tok: np.ndarray  # float64 [N] per coded token
    total: float
    q: np.ndarray         # int64 [N][C] codes of the reconstruction
    yhat: np.ndarray      # float64 [N][C] reconstruction (straight-through forward value)
    mu: np.ndarray        # float64 [N][C] conditional means
    g_y: np.ndarray       # float64 [N][C] dR/dy (straight-through through yhat)
    g_m: np.ndarray       # float64 [N][C] dR/dm
    g_a: np.ndarray       # float64 [C]    dR/da
    g_b: np.ndarray       # float64 [C]    dR/db


def neighbours(yhat: np.ndarray) -> np.ndarray:
    """yhat_{j-1} + yhat_{j+1} for every row (yhat_{-1} = yhat_N = 0)."""
    s = np.zeros_like(yhat)
    s[1:] += yhat[:-1]
    s[:-1] += yhat[1:]
    return s


def rate_terms(y: np.ndarray, m: np.ndarray, yhat: np.ndarray, p: Plan, a, b, u: np.ndarray) -> Rate:
    """The rate and its gradients given the reconstruction yhat (held as the
    straight-through value: its gradient is that of y)."""
    N, C = y.shape
    step = p.step.astype(np.float64)[None, :]
    act = p.active[None, :]
    a64 = np.asarray(a, dtype=np.float32).astype(np.float64)[None, :]
    s = (np.asarray(b, dtype=np.float32).astype(np.float64) / p.step.astype(np.float64))[None, :]
    odd = (np.arange(N) % 2 == 1)[:, None]
    nb = neighbours(yhat)
    mu = m + np.where(odd, a64 * nb, 0.0)
    t = (y - mu) / step + np.asarray(u, dtype=np.float32).astype(np.float64)
    bits = np.where(act, bits_of(t, s), 0.0)
    beta = np.where(act, dbits_dt(t, s), 0.0)
    gamma = np.where(act, dbits_ds(t, s), 0.0)
    g_mu = -beta / step                      # dR/dmu of each row
    g_y = beta / step
    # an even row's reconstruction feeds the means of its odd neighbours
    g_mu_odd = np.where(odd, g_mu, 0.0)
    chain = np.zeros_like(g_mu_odd)
    chain[1:] += g_mu_odd[:-1]
    chain[:-1] += g_mu_odd[1:]
    g_y = g_y + np.where(odd, 0.0, a64 * chain)
    g_a = np.sum(g_mu_odd * nb, axis=0)
    g_b = np.sum(gamma, axis=0) / p.step.astype(np.float64)
    return Rate(bits=bits, bits_tok=bits.sum(axis=1), total=float(bits.sum()), q=None, yhat=yhat, mu=mu,
                g_y=g_y, g_m=g_mu, g_a=g_a, g_b=g_b)


def rate_forward(y: np.ndarray, m: np.ndarray, p: Plan, a, b, u: np.ndarray, q: np.ndarray = None) -> Rate:
    """Rate of coefficients y with embedding means m.  The reconstruction is the
    codec's two-pass quantisation; q, if given, replaces its codes (a caller
    that certified a near-tie decision of another implementation)."""
    if q is None:
        q, yhat = ocodec.quantize(y, m, p, a)
    else:
        yhat = ocodec.dequantize(q, m, p, a)
    r = rate_terms(y, m, yhat, p, a, b, u)
    r.q = q
    return r


def coefficients(rows: np.ndarray, tok: np.ndarray, params: dict):
    """y = A x and the embedding means m of the coded rows of one request."""
    sh = ocodec.shape_of(params)
    T = rows.shape[0]
    N, _, coded_t = ocodec.split_positions(T, sh.keep_head, sh.keep_tail)
    C = params["analysis"].shape[0]
    if N == 0:
        return np.zeros((0, C)), np.zeros((0, C))
    X = bf16.to_f64(rows[coded_t])
    y = X @ bf16.to_f64(params["analysis"]).T
    return y, ocodec.embedding_mean(params, tok[coded_t])


def weight_grads(rows: np.ndarray, tok: np.ndarray, params: dict, r: Rate):
    """Gradients of the total rate with respect to the analysis matrix and the
    mean head: y_j = A x_j and m_j = H e_j (e_j the token's input embedding)
    give dR/dA = sum_j (dR/dy_j) x_j^T and dR/dH = sum_j (dR/dm_j) e_j^T over
    the coded rows (float64 [C][D] and [C][emb])."""
    return weight_grads_of(rows, tok, params, r.g_y, r.g_m)


def weight_grads_of(rows: np.ndarray, tok: np.ndarray, params: dict, g_y: np.ndarray, g_m: np.ndarray):
    """The same products for any upstream gradients g_y, g_m [N][C]."""
    sh = ocodec.shape_of(params)
    T = rows.shape[0]
    N, _, coded_t = ocodec.split_positions(T, sh.keep_head, sh.keep_tail)
    C, D = params["analysis"].shape
    emb = params["embedding"].shape[1]
    if N == 0:
        return np.zeros((C, D)), np.zeros((C, emb))
    X = bf16.to_f64(rows[coded_t])
    E = bf16.to_f64(params["embedding"][np.asarray(tok[coded_t], dtype=np.int64)])
    return np.asarray(g_y, np.float64).T @ X, np.asarray(g_m, np.float64).T @ E
