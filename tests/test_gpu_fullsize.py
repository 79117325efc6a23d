"""Single-request workloads at full size on the GPU, checked against the oracle.

The 32,768-token prompt (0.1 % of rows scaled x20, ~120 B/token) and the
131,072-token prompt (~220 B/token) each go through the launch sequence that
the benchmark times, and every coded row is checked:

  - lossless stage, every symbol: the oracle's rANS decoder reads the GPU
    stream, its encoder re-encodes those symbols to the same bytes, and the
    symbols of the GPU's rANS decoder (dckv_entropy_decode: the codec's decode
    dequantises as it decodes and keeps no symbols) equal the oracle's;
  - lossy stage, every row: the oracle's float64 transform and float32
    quantisation decision give the GPU's codes (odd rows take the GPU's
    even-row codes as neighbours, as the decoder does), >= 99.999 % equal and
    every disagreement a certified tie;
  - decode, every row: coefficients and reconstructed rows within relative L2
    2e-3 of the oracle's two-pass dequantisation, correction, synthesis and
    RoPE, each row within 4x that; kept rows bit-identical where RoPE leaves
    them so.
"""
from __future__ import annotations

import numpy as np
import pytest

import dckv_synth as synth
from oracle import codec as ocodec
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", params=[2, 3], ids=["prompt-32k", "prompt-128k"])
def run(request):
    import torch
    cfg = request.param
    gu.say("generating workload %d" % cfg)
    req = synth.make_request(cfg)
    params = synth.world().params()
    p = gu.oracle_plan(params, req.step_scale)
    codec = gu.device_codec()
    plan = codec.plan(req.step_scale)
    assert plan.crc == p.crc and plan.c_active == p.c_active
    T = req.T
    gu.say("full-size encode T=%d C_a=%d g=%.6g" % (T, p.c_active, req.step_scale))
    data, st = gu.gpu_encode(plan, req.rows, req.token_ids)
    assert st == 0
    ws = gu.dk().workspace(plan, T)
    gu.say("full-size decode")
    out, st = gu.gpu_decode(plan, data, req.token_ids, ws=ws)
    assert st == 0
    sh = ocodec.shape_of(params)
    N, kept_t, coded_t = ocodec.split_positions(T, sh.keep_head, sh.keep_tail)
    views = {}
    views["yhat_b"], _ = gu.read_view(ws, plan, T, gu.dk().VIEW_YHAT_B)
    gu.say("full-size symbols-only rANS decode")
    views["sym"], n_esc_dec, st = gu.gpu_entropy_decode(plan, data, T, N, p.c_active, ws=ws)
    assert st == 0
    torch.cuda.synchronize()
    del ws
    gu.say("oracle rANS decode of the whole GPU stream (%d bytes)" % len(data))
    h, sym_g, flat_g, qe_g, _ = gu.oracle_symbols_of_stream(data, params, p, T)
    return dict(req=req, params=params, p=p, data=data, out=out, views=views, N=N, kept_t=kept_t,
                coded_t=coded_t, sh=sh, h=h, sym_g=sym_g, flat_g=flat_g, qe_g=qe_g, n_esc_dec=n_esc_dec)


def test_fullsize_lossless_stage_bit_exact(run):
    r = run
    req, params, p, data, N = r["req"], r["params"], r["p"], r["data"], r["N"]
    h, sym_g, flat_g, qe_g = r["h"], r["sym_g"], r["flat_g"], r["qe_g"]
    assert h.N == N and h.total_bytes == len(data)
    gu.say("  %d escapes; oracle re-encode" % len(flat_g))
    assert gu.oracle_stream_from_symbols(req.rows, req.T, params, p, sym_g, flat_g, qe_g) == data
    # the GPU rANS decoder's symbols (escaped positions hold the escape sentinel)
    assert r["n_esc_dec"] == len(flat_g)
    assert np.array_equal(r["views"]["sym"], sym_g)


def test_fullsize_every_code_and_row(run):
    r = run
    req, params, p, N = r["req"], r["params"], r["p"], r["N"]
    view = r["views"]["yhat_b"].view(np.uint16).reshape(-1, p.step.size)[:N]
    gu.check_all_rows(req.rows, req.token_ids, req.T, params, p, r["sym_g"], r["flat_g"], r["qe_g"],
                      out_rows=r["out"], yhat_view=view)


def test_fullsize_kept_rows(run):
    r = run
    gu.check_kept_rows(r["req"].rows, r["req"].T, r["params"], r["out"])
