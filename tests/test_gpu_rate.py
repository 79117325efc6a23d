"""The training rate (additive-noise likelihood, straight-through
reconstruction) and its gradients on the GPU against the oracle, and the
weight gradients through the transforms (dR/dA, dR/dH) for seeded upstream
gradients, within their derived elementwise bound.

Workloads: the 512-token and 4,096-token prompts (a training sample is a
4,096-token prompt) with seeded uniform noise, plus edge cases: no coded rows,
one and seven coded rows (odd N: the last row is even with no right
neighbour), dropped components, and the status of bad inputs.

The GPU's reconstruction gives its codes (even rows against the oracle's
embedding means, odd rows against the means those give); they must equal the
oracle's float32 decisions up to certified ties, at the codec's symbol
agreement bar.  The oracle then runs on the GPU's codes and every output is
compared with it.  Bars, derived from the fp32 transform (relative error
about 1e-6 of |y|, i.e. about 3e-5 steps in t):
  - per-token bits within relative 1e-4;
  - reconstruction within relative L2 1e-5 per row (fp32 of the same codes);
  - dR/dy and dR/dm within relative L2 1e-3 per row (d beta / dt is at most
    1/s^2 per step inside the central interval);
  - dR/da and dR/db per component within 1e-3 of the sum of the magnitudes of
    their terms, plus how far those terms move when t moves by the residual's
    float32 accuracy (the bound the code ties are certified with).
"""
from __future__ import annotations

import numpy as np
import pytest

import dckv_synth as synth
from oracle import codec as ocodec
from oracle import rate as orate
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

BITS_TOL = 1e-4
YHAT_TOL = 1e-5
GRAD_TOL = 1e-3


def _gpu_rate(plan, rows, tok, u):
    import torch
    out = gu.dk().rate_forward(plan, gu.rows_dev(rows), gu.to_dev(tok.astype(np.int32)), gu.to_dev(u))
    res = {k: (v.cpu().numpy() if isinstance(v, torch.Tensor) else v) for k, v in out.items()}
    return res


def _codes_of(yhat, m, p, a):
    """Codes of a reconstruction: even rows around m, odd rows around the
    means the even rows give."""
    step = p.step.astype(np.float64)[None, :]
    q = np.zeros(yhat.shape, dtype=np.int64)
    q[0::2] = np.rint((yhat[0::2] - m[0::2]) / step)
    mu = ocodec.dequantize(q, m, p, a)  # odd rows: q = 0 gives their means
    q[1::2] = np.rint((yhat[1::2] - mu[1::2]) / step)
    q[:, ~p.active] = 0
    return q


def _check(params, p, rows, tok, u, got, label):
    a, b = params["nbr_weight"], params["laplace_scale"]
    y, m = orate.coefficients(rows, tok, params)
    N = y.shape[0]
    assert got["status"] == 0
    assert got["bits"].shape == (N,) and got["yhat"].shape == y.shape
    qg = _codes_of(got["yhat"].astype(np.float64), m, p, a)
    ro = orate.rate_forward(y, m, p, a, b, u)
    act = p.active
    step = p.step.astype(np.float64)
    # even rows: every disagreement is a certified tie of the oracle's residual
    qe_o, qe_g = ro.q[0::2][:, act], qg[0::2][:, act]
    res = ((y - ro.mu) / step[None, :])[0::2][:, act]
    yy = np.abs(y[0::2][:, act]) + np.abs(ro.mu[0::2][:, act])
    for n, k in np.argwhere(qe_o != qe_g):
        tie = 0.5 * (qe_o[n, k] + qe_g[n, k])
        tol = 2.0 ** -17 * yy[n, k] / step[act][k] + 1e-4
        assert abs(qe_o[n, k] - qe_g[n, k]) == 1 and abs(res[n, k] - tie) <= tol, (label, 2 * n, k)
    agree = float(np.mean(ro.q[:, act] == qg[:, act])) if N else 1.0
    gu.say("  %s: N=%d codes agree %.7f" % (label, N, agree))
    assert agree >= gu.SYMBOL_AGREEMENT
    r = orate.rate_forward(y, m, p, a, b, u, q=qg)
    # odd rows: the oracle's float32 decision around the means the GPU's even
    # codes give (as the decoder would have them); every disagreement is a
    # certified tie
    mu_o = r.mu[1::2][:, act]
    qo_o = ocodec._decide(y[1::2][:, act] - mu_o, p.step[act])
    qg_o = qg[1::2][:, act]
    res_o = (y[1::2][:, act] - mu_o) / step[act][None, :]
    yy_o = np.abs(y[1::2][:, act]) + np.abs(mu_o)
    for n, k in np.argwhere(qo_o != qg_o):
        tie = 0.5 * (qo_o[n, k] + qg_o[n, k])
        tol = 2.0 ** -17 * yy_o[n, k] / step[act][k] + 1e-4
        assert abs(qo_o[n, k] - qg_o[n, k]) == 1 and abs(res_o[n, k] - tie) <= tol, (label, 2 * n + 1, k)
    if N:
        eb = np.max(np.abs(got["bits"] - r.bits_tok) / np.maximum(r.bits_tok, 1.0))
        gu.say("  %s: bits/token %.1f, worst rel %.3g" % (label, float(np.mean(r.bits_tok)), eb))
        assert eb <= BITS_TOL
        for name, want, tol in (("yhat", r.yhat, YHAT_TOL), ("grad_y", r.g_y, GRAD_TOL),
                                ("grad_mean", r.g_m, GRAD_TOL)):
            g = got[name].astype(np.float64)
            num = np.sqrt(np.sum((g - want) ** 2, axis=1))
            den = np.sqrt(np.sum(want ** 2, axis=1))
            worst = float(np.max(num / np.maximum(den, 1e-30)))
            gu.say("  %s: %s worst row rel %.3g" % (label, name, worst))
            assert np.all(num <= tol * den + 1e-30), name
        assert np.all(got["grad_y"][:, ~act] == 0) and np.all(got["grad_mean"][:, ~act] == 0)
    # per-component sums: GRAD_TOL of the sum of the terms' magnitudes, plus
    # how far each term moves when t moves by the residual's float32 accuracy
    # tau (the bound the code ties are certified with); near the point where
    # d bits / ds changes sign that second part dominates
    odd = (np.arange(N) % 2 == 1)[:, None]
    t = (y - r.mu) / step[None, :] + u.astype(np.float64)
    s = (b.astype(np.float32).astype(np.float64) / step)[None, :]
    tau = 2.0 ** -17 * (np.abs(y) + np.abs(r.mu)) / step[None, :] + 1e-4

    def wobble(f):
        f0 = f(t, s)
        return np.maximum(np.abs(f(t + tau, s) - f0), np.abs(f(t - tau, s) - f0))

    nb = orate.neighbours(r.yhat)
    oddm = np.where(odd, 1.0, 0.0) * act[None, :]
    sa = np.sum(oddm * (GRAD_TOL * np.abs(r.g_m) + wobble(orate.dbits_dt) / step[None, :]) * np.abs(nb), axis=0)
    sb = np.sum(act[None, :] * (GRAD_TOL * np.abs(orate.dbits_ds(t, s)) + wobble(orate.dbits_ds)), axis=0) / step
    for name, want, bar in (("grad_nbr", r.g_a, sa), ("grad_scale", r.g_b, sb)):
        e = np.abs(got[name].astype(np.float64) - want)
        gu.say("  %s: %s worst %.3g of its bar" % (label, name, float(np.max(e / np.maximum(bar, 1e-30)))))
        assert np.all(e <= bar + 1e-12), name


@pytest.mark.parametrize("cfg", [0, 1], ids=["tiny-512", "prompt-4k"])
def test_rate_matches_oracle(cfg):
    req = synth.make_request(cfg)
    params = synth.world().params()
    p = gu.oracle_plan(params, req.step_scale)
    plan = gu.device_codec().plan(req.step_scale)
    N = req.T - 132
    u = synth.rate_noise(N, 2048, seed=cfg)
    gu.say("rate T=%d" % req.T)
    got = _gpu_rate(plan, req.rows, req.token_ids, u)
    _check(params, p, req.rows, req.token_ids, u, got, "cfg%d" % cfg)


@pytest.mark.parametrize("N", [0, 1, 7, 70])
def test_rate_short_requests(N):
    params = synth.world().params()
    g = synth.step_scale_for(220.0)
    p = gu.oracle_plan(params, g)
    plan = gu.device_codec().plan(g)
    T = N + 132 if N else 100
    rows, tok = synth.random_rows(T, seed=900 + N)
    u = synth.rate_noise(N, 2048, seed=50 + N)
    gu.say("rate short T=%d" % T)
    got = _gpu_rate(plan, rows, tok, u)
    _check(params, p, rows, tok, u, got, "N%d" % N)
    if N == 0:
        assert np.all(got["grad_nbr"] == 0) and np.all(got["grad_scale"] == 0)


def test_rate_with_dropped_components():
    w = synth.world()
    rng = np.random.default_rng(5)
    scale = w.laplace_scale.copy()
    scale[rng.choice(2048, size=77, replace=False)] = 1e-5
    params = gu.params_with_scales(scale)
    g = synth.step_scale_for(220.0)
    p = gu.oracle_plan(params, g)
    plan = gu.codec_with_scales(scale).plan(g)
    assert plan.c_active == p.c_active < 2048
    rows, tok = synth.random_rows(132 + 300, seed=77)
    u = synth.rate_noise(300, 2048, seed=77)
    gu.say("rate with C_a = %d" % p.c_active)
    got = _gpu_rate(plan, rows, tok, u)
    _check(params, p, rows, tok, u, got, "dropped")


def test_rate_status_of_bad_inputs():
    g = synth.step_scale_for(220.0)
    plan = gu.device_codec().plan(g)
    rows, tok = synth.random_rows(132 + 40, seed=3)
    u = synth.rate_noise(40, 2048, seed=3)
    bad_tok = tok.copy()
    bad_tok[4 + 17] = 40000
    assert _gpu_rate(plan, rows, bad_tok, u)["status"] == -1  # EINVAL
    bad_rows = rows.copy()
    bad_rows[4 + 5, 100] = 0x7F80  # +inf
    assert _gpu_rate(plan, bad_rows, tok, u)["status"] == -1  # EINVAL
    assert _gpu_rate(plan, rows, tok, u)["status"] == 0


def _check_weight_grads(params, rows, tok, gy, gm, gA, gH, label):
    """Elementwise bound: the gradients enter as two bf16 halves (relative
    error 2^-16) and the products accumulate in fp32 over K = 2 n_pad terms, so
    |error| <= (2^-16 + K 2^-24) times the product of the magnitudes."""
    wA, wH = orate.weight_grads_of(rows, tok, params, gy, gm)
    sh = ocodec.shape_of(params)
    N = rows.shape[0] - sh.keep_head - sh.keep_tail
    K = 2 * ((N + 63) // 64 * 64)
    f = 2.0 ** -16 + K * 2.0 ** -24
    # |g|^T |x|: the rows' magnitudes (bf16 values are exact in float64)
    _, _, coded_t = ocodec.split_positions(rows.shape[0], sh.keep_head, sh.keep_tail)
    X = np.abs(orate.bf16.to_f64(rows[coded_t]))
    Eg = np.abs(orate.bf16.to_f64(params["embedding"][tok[coded_t].astype(np.int64)]))
    bA = f * (np.abs(gy).T @ X)
    bH = f * (np.abs(gm).T @ Eg)
    for name, got, want, bar in (("dA", gA, wA, bA), ("dH", gH, wH, bH)):
        e = np.abs(got.astype(np.float64) - want)
        rel = float(np.linalg.norm(got - want) / np.linalg.norm(want))
        gu.say("  %s: %s rel L2 %.3g, worst %.3g of the bound" % (label, name, rel, float(np.max(e / bar))))
        assert np.all(e <= bar), name


@pytest.mark.parametrize("cfg", [0, 1], ids=["tiny-512", "prompt-4k"])
def test_rate_weight_gradients(cfg):
    import torch
    req = synth.make_request(cfg)
    params = synth.world().params()
    plan = gu.device_codec().plan(req.step_scale)
    N = req.T - 132
    rng = np.random.default_rng(300 + cfg)
    gy = (rng.standard_normal((N, 2048)) * rng.uniform(0.1, 30.0, 2048)).astype(np.float32)
    gm = (-gy + rng.standard_normal((N, 2048)).astype(np.float32)).astype(np.float32)
    gA, gH, st = gu.dk().rate_backward(plan, gu.rows_dev(req.rows), gu.to_dev(req.token_ids.astype(np.int32)),
                                       gu.to_dev(gy), gu.to_dev(gm))
    assert st == 0
    _check_weight_grads(params, req.rows, req.token_ids, gy, gm, gA.cpu().numpy(), gH.cpu().numpy(), "cfg%d" % cfg)


def test_rate_weight_gradients_edges():
    g = synth.step_scale_for(220.0)
    plan = gu.device_codec().plan(g)
    params = synth.world().params()
    # no coded rows: zero gradients
    rows, tok = synth.random_rows(100, seed=5)
    gA, gH, st = gu.dk().rate_backward(plan, gu.rows_dev(rows), gu.to_dev(tok.astype(np.int32)),
                                       gu.to_dev(np.zeros((0, 2048), np.float32)),
                                       gu.to_dev(np.zeros((0, 2048), np.float32)))
    assert st == 0 and not gA.any().item() and not gH.any().item()
    # a ragged count (one row past a multiple of 64) and a bad token id
    rows, tok = synth.random_rows(132 + 65, seed=6)
    rng = np.random.default_rng(6)
    gy = rng.standard_normal((65, 2048)).astype(np.float32)
    gm = rng.standard_normal((65, 2048)).astype(np.float32)
    gA, gH, st = gu.dk().rate_backward(plan, gu.rows_dev(rows), gu.to_dev(tok.astype(np.int32)), gu.to_dev(gy),
                                       gu.to_dev(gm))
    assert st == 0
    _check_weight_grads(params, rows, tok, gy, gm, gA.cpu().numpy(), gH.cpu().numpy(), "N65")
    bad = tok.copy()
    bad[4 + 64] = -3
    _, _, st = gu.dk().rate_backward(plan, gu.rows_dev(rows), gu.to_dev(bad.astype(np.int32)), gu.to_dev(gy),
                                     gu.to_dev(gm))
    assert st == -1  # EINVAL
