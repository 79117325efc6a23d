"""The linear codec on the GPU against the oracle.

The linear codec is the same codec without the synthesis-side GELU correction
(DCKV digest, Evidence: the pages compare its stored payload with DCKV's);
a plan made from parameters without w1 / w2 decodes to xhat = S yhat_b.
Bars:
  - its stream is byte-identical to the DCKV plan's stream (encoding does not
    involve the correction);
  - decoded rows within relative L2 2e-3 of the oracle's linear decode of the
    same stream, and away from the DCKV decode by the size of the correction;
  - kept rows bit-identical to the DCKV decode's; all-kept requests decode.
"""
from __future__ import annotations

import functools

import numpy as np
import pytest

import dckv_synth as synth
from oracle import bf16, codec as ocodec
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _linear_params():
    return {k: v for k, v in synth.world().params().items() if k not in ("w1", "w2")}


@functools.lru_cache(maxsize=None)
def _linear_codec():
    return gu.dk().Codec(_linear_params(), device="cuda:0")


@pytest.mark.parametrize("cfg", [0, 1])
def test_linear_codec_matches_oracle(cfg):
    req = synth.make_request(cfg)
    params = synth.world().params()
    p = gu.oracle_plan(params, req.step_scale)
    full = gu.device_codec().plan(req.step_scale)
    lin = _linear_codec().plan(req.step_scale)
    assert lin.crc == full.crc == p.crc
    gu.say("linear codec T=%d" % req.T)
    data, st = gu.gpu_encode(lin, req.rows, req.token_ids)
    assert st == 0
    data_full, st = gu.gpu_encode(full, req.rows, req.token_ids)
    assert st == 0 and data == data_full
    out, st = gu.gpu_decode(lin, data, req.token_ids)
    assert st == 0
    out_full, st = gu.gpu_decode(full, data, req.token_ids)
    assert st == 0
    dec = ocodec.decode(data, req.token_ids, _linear_params(), p)
    e = gu.rel_l2(bf16.to_f64(out), bf16.to_f64(dec.rows))
    d = gu.rel_l2(bf16.to_f64(out_full), bf16.to_f64(dec.rows))
    gu.say("  rows rel %.3g vs oracle linear; DCKV decode differs by %.3g" % (e, d))
    assert e <= gu.REL_L2_TOL
    assert d > 5 * e  # the correction is visible at this tolerance
    _, kept_t, _ = ocodec.split_positions(req.T, 4, 128)
    assert np.array_equal(out[kept_t], out_full[kept_t])


@pytest.mark.parametrize("T", [100, 133])
def test_linear_codec_short_requests(T):
    rows, tok = synth.random_rows(T, seed=2000 + T)
    g = synth.step_scale_for(220.0)
    p = gu.oracle_plan(synth.world().params(), g)
    lin = _linear_codec().plan(g)
    data, st = gu.gpu_encode(lin, rows, tok)
    assert st == 0
    out, st = gu.gpu_decode(lin, data, tok)
    assert st == 0
    dec = ocodec.decode(data, tok, _linear_params(), p)
    assert gu.rel_l2(bf16.to_f64(out), bf16.to_f64(dec.rows)) <= gu.REL_L2_TOL
