"""Pins of the rate ladder and of the modelled code length.

The DCKV digest ("How it works", Training bullet) ties one codec to one rate;
the synthetic codec gets its ladder of rates from one step scale g.  These
tests tie the oracle's rate helpers to things other than themselves: a hand
sum over a tiny stream, the bytes the (separately pinned) rANS coder really
writes for symbols drawn from the plan's own model, the ordering of fp32
values, and the bytes the full oracle encoder writes for seeded requests of
each workload.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest

from oracle import codec, plan as P, rans, rate_ladder as RL
from tests.tiny import tiny_params, tiny_rows


def _f32(x) -> np.float32:
    return np.float32(x)


def _prev_f32(g: float) -> np.float32:
    return np.nextafter(_f32(g), _f32(0.0))


# ----------------------------------------------------------------------------
# modelled code length of a stream (Evidence: stored payload vs the models'
# code length)
# ----------------------------------------------------------------------------
def test_modelled_bits_hand_sum_on_tiny_stream():
    # three components, the middle one dropped: ranks 0 and 1 are components 0 and 2
    pl = P.make_plan(_f32(1.0), np.ones(3, np.float32), np.array([0.7, 0.01, 2.5], np.float32))
    assert pl.c_active == 2 and list(pl.act_idx) == [0, 2]
    sym = np.array([[127, 128], [126, 255], [255, 127 + 40], [0, 254]], dtype=np.uint8)
    n_esc = 2
    f = [[int(v) for v in row] for row in pl.freq]
    want = 0.0
    # written out symbol by symbol: (15 - log2 f) for each coded symbol of its rank
    want += 15 - math.log2(f[0][127]) + 15 - math.log2(f[1][128])
    want += 15 - math.log2(f[0][126])
    want += 15 - math.log2(f[1][167])
    want += 15 - math.log2(f[0][0]) + 15 - math.log2(f[1][254])
    want += 64 * n_esc
    assert codec.modelled_bits(sym, pl, n_esc) == pytest.approx(want, rel=1e-12)
    assert codec.modelled_bits(sym[:0], pl, 3) == 192.0


def test_modelled_bits_against_stored_words_with_drops():
    """The coder's output (pinned by round trips elsewhere) is within a flush of
    the modelled length: per substream at most 32 bits above and 16 below."""
    prm = tiny_params(seed=11, n_coef=8)
    prm["laplace_scale"] = np.array([0.4, 0.001, 1.5, 0.02, 3.0, 0.8, 0.002, 6.0], np.float32)
    pl = P.make_plan(_f32(0.3), prm["base_step"], prm["laplace_scale"])
    assert 0 < pl.c_active < 8
    rows, tok = tiny_rows(prm, 700, seed=12, scale=0.6)
    enc = codec.encode(rows, tok, prm, pl)
    stored = 16 * sum(len(g) for g in enc.groups)
    modelled = enc.modelled_bits - 64 * len(enc.esc_flat)
    lanes = len(enc.groups) * pl.c_active
    assert -16 * lanes <= stored - modelled <= 32 * lanes + 0.01 * modelled


def _scales_for_test():
    rng = np.random.default_rng(21)
    return rng.uniform(0.05, 0.2, 64).astype(np.float32)


def test_modelled_bytes_per_token_equals_coded_bytes_of_model_draws():
    """Symbols drawn from the plan's own pmf, coded by the pinned rANS coder,
    cost what modelled_bytes_per_token says, flush included.  The scales are
    small, so the flush is about a third of the bytes and the estimate fails
    without it (or with a wrong unit)."""
    b = _scales_for_test()
    pl = P.make_plan(_f32(1.0), np.ones(b.size, np.float32), b)
    rng = np.random.default_rng(5)
    N = 256 * 16
    sym = np.empty((N, pl.c_active), np.uint8)
    for r in range(pl.c_active):
        sym[:, r] = rng.choice(255, size=N, p=pl.pmf[r])
    groups = rans.encode_all(sym, pl.freq, pl.cum)
    coded = 2 * sum(len(g) for g in groups) / N
    est = P.modelled_bytes_per_token(pl)
    assert coded == pytest.approx(est, rel=0.02)
    no_flush = P.modelled_bytes_per_token(pl, flush_bits_per_substream=0.0)
    assert abs(coded - no_flush) / coded > 0.25
    # the model part alone is the sample's modelled length per token
    assert codec.modelled_bits(sym, pl, 0) / N / 8 == pytest.approx(no_flush, rel=0.02)


def test_modelled_bytes_non_increasing_in_step_scale():
    b = _scales_for_test()
    base = np.ones(b.size, np.float32)
    gs = 2.0 ** np.linspace(-6, 3, 60)
    v = [P.modelled_bytes_per_token(P.make_plan(_f32(g), base, b)) for g in gs]
    assert all(v[i + 1] <= v[i] for i in range(len(v) - 1))
    assert v[0] > 10 * v[-1]


# ----------------------------------------------------------------------------
# the bisection
# ----------------------------------------------------------------------------
def test_smallest_scale_closed_form_thresholds():
    for thr in (0.3, 1e-3, 0.1007872, 2.0 ** -10, 3.0):
        g = RL.smallest_scale(lambda x, thr=thr: float(x) >= thr)
        # the smallest fp32 at or above thr
        want = _f32(thr)
        if float(want) < thr:
            want = np.nextafter(want, _f32(np.inf))
        assert g == float(want)
    assert RL.smallest_scale(lambda x: False) == RL.G_MAX
    assert RL.smallest_scale(lambda x: True) == float(_f32(RL.G_MIN))


def test_smallest_scale_on_a_four_component_plan():
    base = np.ones(4, np.float32)
    b = np.array([0.9, 0.3, 0.12, 0.05], np.float32)

    def bytes_at(g):
        return P.modelled_bytes_per_token(P.make_plan(_f32(g), base, b))

    for target in (0.05, 0.2, 0.6, 1.5):
        g = RL.smallest_scale(lambda x: bytes_at(x) <= target)
        assert bytes_at(g) <= target < bytes_at(_prev_f32(g))
        # direction: finer steps cost more bytes, so the answer is not the largest scale
        assert bytes_at(g * 0.5) > target
    # hand check of one rung by a linear scan over the fp32 values just below
    target = 0.6
    g = RL.smallest_scale(lambda x: bytes_at(x) <= target)
    x = _f32(g)
    for _ in range(64):
        x = _prev_f32(x)
        assert bytes_at(x) > target


# ----------------------------------------------------------------------------
# the ladder table and the workloads' achieved rates
# ----------------------------------------------------------------------------
_TABLE = os.path.join(os.path.dirname(os.path.dirname(__file__)), "dckv_synth", "step_scales.json")


@pytest.fixture(scope="module")
def world_and_sample():
    import dckv_synth as synth
    w = synth.world()
    rows, tok = synth.calibration_sample()
    return w, RL.sample_from_rows(rows, tok, w.params())


def test_coded_bytes_of_sample_non_increasing_in_step_scale(world_and_sample):
    w, s = world_and_sample
    small = RL.Sample(y=s.y[:512], m=s.m[:512], a=s.a)
    gs = [0.02, 0.03, 0.045, 0.07, 0.1, 0.15, 0.22]
    v = [RL.coded_bytes_per_token(small, P.make_plan(_f32(g), w.base_step, w.laplace_scale)) for g in gs]
    assert all(v[i + 1] <= v[i] for i in range(len(v) - 1))


def test_step_scale_table_is_the_ladder_boundary(world_and_sample):
    """Every g in the table meets its target on the calibration sample and the
    fp32 value just below it does not."""
    w, s = world_and_sample
    with open(_TABLE) as f:
        table = json.load(f)
    assert table["calibration_rows"] == s.N
    for key, g in table["step_scale"].items():
        target = table["target"][key]
        got = RL.coded_bytes_per_token(s, P.make_plan(_f32(g), w.base_step, w.laplace_scale))
        below = RL.coded_bytes_per_token(s, P.make_plan(_prev_f32(g), w.base_step, w.laplace_scale))
        assert got <= target < below, (key, got, below)
        assert got == pytest.approx(table["calibration_bytes_per_token"][key], rel=1e-12)


def _coded_bytes_per_token(req, w):
    pl = P.make_plan(_f32(req.step_scale), w.base_step, w.laplace_scale)
    enc = codec.encode(req.rows, req.token_ids, w.params(), pl)
    kept = (req.T - enc.N) * req.rows.shape[1] * 2
    return (enc.total_bytes - 64 - kept) / enc.N


def test_workloads_land_within_ten_percent_of_their_rate(world_and_sample):
    """Each workload's requests, coded by the oracle encoder, spend their rate
    target within 10 % (the 32K and batch workloads on 4,096-token prompts with
    their own seeds)."""
    import dckv_synth as synth
    w, _ = world_and_sample
    cases = [synth.make_request(0), synth.make_request(1), synth.make_request(2, T=4096)]
    seen = set()
    for i in range(synth.CONFIGS[4]["n_requests"]):
        r = synth.make_request(4, index=i, n_rows=0)
        if r.rate_target not in seen:
            seen.add(r.rate_target)
            cases.append(synth.make_request(4, index=i, T=4096))
    assert seen == set(synth.CONFIGS[4]["rates"])
    for req in cases:
        got = _coded_bytes_per_token(req, w)
        assert abs(got / req.rate_target - 1.0) <= 0.10, (req.note, req.rate_target, got)
