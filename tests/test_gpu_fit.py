"""The closed-form fit of the conditional models on the GPU against the oracle.

Calibration rows are planted with a known structure: coefficients
y_j = H0 e_j + z_j (z Laplace with the codec's scales) and, on odd rows, plus
a0 times the sum of both neighbours; rows x_j = S y_j in bf16.  Bars: the mean
head within relative L2 2e-3 of the oracle's float64 fit (fp32 solve on bf16
products, E^T Y with 16 mantissa bits of Y); neighbour weights and Laplace
scales within relative L2 2e-3 and per component within 2e-3 of the largest;
EINVAL for an out-of-range token id and for a Gram matrix that is not
positive definite (no ridge, fewer rows than embedding dimensions).
"""
from __future__ import annotations

import functools

import numpy as np
import pytest

import dckv_synth as synth
from oracle import bf16, fit as ofit
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=None)
def _planted(n: int, seed: int = 11):
    w = synth.world()
    p = w.params()
    rng = np.random.default_rng(seed)
    tok = rng.integers(0, p["embedding"].shape[0], n).astype(np.int32)
    E = bf16.to_f64(p["embedding"])
    H0 = 10.0 * bf16.to_f64(p["mean_head"])
    a0 = np.asarray(p["nbr_weight"], np.float64)
    b0 = np.asarray(p["laplace_scale"], np.float64)
    y = E[tok] @ H0.T + rng.laplace(0.0, b0, (n, b0.size))
    for j in range(1, n, 2):
        y[j] += a0 * (y[j - 1] + (y[j + 1] if j + 1 < n else 0.0))
    rows = bf16.from_f64(y @ bf16.to_f64(p["synthesis"]).T)
    return rows, tok


def _run(n: int, ridge: float, tok_override=None):
    rows, tok = _planted(n)
    if tok_override is not None:
        tok = tok_override
    dk = gu.dk()
    H, Hb, a, b, st = dk.fit(gu.device_codec(), gu.rows_dev(rows), gu.to_dev(tok.astype(np.int32)), ridge)
    return rows, tok, H.cpu().numpy().astype(np.float64), Hb.cpu().numpy().view(np.uint16), \
        a.cpu().numpy().astype(np.float64), b.cpu().numpy().astype(np.float64), st


@pytest.mark.parametrize("n,ridge", [(4096, 1e-3), (1000, 1e-2), (1001, 1e-2)])
def test_fit_matches_oracle(n, ridge):
    rows, tok, H, Hb, a, b, st = _run(n, ridge)
    assert st == 0
    f = ofit.fit(rows, tok, synth.world().params(), ridge)
    eH, ea, eb = gu.rel_l2(H, f.H), gu.rel_l2(a, f.a), gu.rel_l2(b, f.b)
    gu.say("n=%d ridge=%g: H rel %.3g, a rel %.3g, b rel %.3g, bf16(H) equal %.4f" % (
        n, ridge, eH, ea, eb, np.mean(Hb == f.H_b)))
    assert eH <= gu.REL_L2_TOL and ea <= gu.REL_L2_TOL and eb <= gu.REL_L2_TOL
    assert np.max(np.abs(a - f.a)) <= 2e-3 * np.max(np.abs(f.a))
    assert np.max(np.abs(b - f.b)) <= 2e-3 * np.max(np.abs(f.b))
    # the planted structure is recovered (statistically, at this n)
    if n == 4096:
        w = synth.world().params()
        a0 = np.asarray(w["nbr_weight"], np.float64)
        assert np.corrcoef(f.a, a0)[0, 1] > 0.9


def test_fit_rejects_bad_token_id():
    rows, tok = _planted(1000)
    bad = tok.copy()
    bad[17] = 1 << 20
    *_, st = _run(1000, 1e-2, tok_override=bad)
    assert st == gu.dk().EINVAL


def test_fit_rejects_singular_gram():
    *_, st = _run(1000, 0.0)  # 1000 rows, 2048 embedding dimensions, no ridge
    assert st == gu.dk().EINVAL
