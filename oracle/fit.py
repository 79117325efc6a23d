"""Closed-form fit of the conditional models to a trained codec (CPU, float64).

Test infrastructure: only tests, the package's smoke check and the
benchmark's CPU-baseline leg use this module.

Source: DCKV digest page (trove.briskstack.com, "DCKV: Learned Transform
Coding of the Prompt KV Cache in Hybrid Language Models"), section Evidence:
fitting the conditional models in closed form to an already-trained codec
recovers a saving close to the jointly trained one, without retraining.  The
page names no estimator; the readings below are the plainest closed forms for
the models of "How it works" (Conditional entropy models bullet):

  * Calibration: n consecutive coded rows x_j of one prompt (row j's
    neighbours are rows j - 1 and j + 1) with token ids tok_j; coefficients
    y_j = A x_j.
  * Mean head: ridge least squares over all rows,
        H = argmin_H  sum_j |y_j - H e_j|^2 + lam * n * |H|_F^2,
    e_j = E[tok_j]; in closed form H^T = (E^T E + lam n I)^-1 E^T Y.
  * The codec holds H in bf16: the remaining fits use m_j = bf16(H) e_j.
  * Neighbour weights, per component c over the odd rows j, with
    s_j = y_{j-1} + y_{j+1} (y_n = 0, the codec's missing right neighbour) and
    r_j = y_j - m_j:  a_c = sum_j r_jc s_jc / sum_j s_jc^2 (0 if the sum of
    squares is 0).  The fit is open loop: it uses the calibration
    coefficients, not quantised ones.
  * Laplace scales: the maximum-likelihood scale of a zero-mean Laplace of the
    residual, b_c = mean_j |y_jc - mu_jc| over all rows, with mu_j = m_j for
    even j and m_j + a * s_j for odd j (a rounded to float32, as the codec
    holds it).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import bf16


@dataclass
class Fit:
    H: np.ndarray      # float64 [C][emb]
    H_b: np.ndarray    # bf16 bits of H
    a: np.ndarray      # float64 [C]
    b: np.ndarray      # float64 [C]
    y: np.ndarray      # float64 [n][C] calibration coefficients
    m: np.ndarray      # float64 [n][C] means from bf16(H)


def neighbour_sum(y: np.ndarray) -> np.ndarray:
    """s_j = y_{j-1} + y_{j+1} for every row (y_{-1} = y_n = 0)."""
    s = np.zeros_like(y)
    s[1:] += y[:-1]
    s[:-1] += y[1:]
    return s


def fit(rows: np.ndarray, tok: np.ndarray, params: dict, lam: float) -> Fit:
    """The fit from calibration rows (bf16 bits [n][D]) and their token ids."""
    A = bf16.to_f64(params["analysis"])
    E = bf16.to_f64(params["embedding"])
    y = bf16.to_f64(rows) @ A.T
    e = E[np.asarray(tok, dtype=np.int64)]
    return fit_coefficients(y, e, lam)


def fit_coefficients(y: np.ndarray, e: np.ndarray, lam: float) -> Fit:
    """The fit from coefficients y [n][C] and embeddings e [n][emb] (float64)."""
    n, emb = e.shape
    G = e.T @ e + lam * n * np.eye(emb)
    Ht = np.linalg.solve(G, e.T @ y)          # [emb][C]
    H = Ht.T.copy()
    H_b = bf16.from_f64(H)
    m = e @ bf16.to_f64(H_b).T
    s = neighbour_sum(y)
    odd = np.arange(1, n, 2)
    r = y[odd] - m[odd]
    den = np.sum(s[odd] ** 2, axis=0)
    num = np.sum(r * s[odd], axis=0)
    a = np.where(den > 0, num / np.where(den > 0, den, 1.0), 0.0)
    a32 = a.astype(np.float32).astype(np.float64)
    mu = m.copy()
    mu[odd] += a32[None, :] * s[odd]
    b = np.mean(np.abs(y - mu), axis=0)
    return Fit(H=H, H_b=H_b, a=a, b=b, y=y, m=m)
