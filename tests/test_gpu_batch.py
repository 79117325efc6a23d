"""Batch calls on the GPU: a mixed batch of independent requests.

Requests come from the 16-request batch workload (Laplace / Student-t mixture
rows, each request with its own seeded ids and rate drawn from 60, 120, 220,
400 bytes/token), at shortened lengths that include ragged tiles, a request with
every row kept and a one-token request.  Bars:
  - every request's stream and decoded rows from the batch call equal those of
    the single-request calls, byte for byte;
  - two requests are also checked against the oracle directly (lossless stage
    bit-exact, codes within the symbol-agreement bar with certified ties,
    decoded rows within relative L2 2e-3);
  - a batch with one invalid request enqueues nothing.
"""
from __future__ import annotations

import numpy as np
import pytest

import dckv_synth as synth
from oracle import bf16, codec as ocodec
from tests import gpu_util as gu
from tests.test_gpu_codec import _codes, _near_tie_certified

pytestmark = pytest.mark.gpu

LENGTHS = [1037, 132, 600, 1, 900, 389, 2048, 133]


@pytest.fixture(scope="module")
def batch():
    import torch
    dk = gu.dk()
    codec = gu.device_codec()
    dev = codec.device
    reqs, plans, data = [], {}, []
    for i, T in enumerate(LENGTHS):
        r = synth.make_request(4, index=i, T=T)
        if r.step_scale not in plans:
            plans[r.step_scale] = codec.plan(r.step_scale)
        data.append(r)
    gu.say("batch of %d requests, rates %s" % (len(data), sorted({r.rate_target for r in data})))
    enc = []
    for r in data:
        plan = plans[r.step_scale]
        max_bytes, _ = plan.bytes(r.T)
        enc.append(dk.Request(plan, gu.to_dev(r.token_ids.astype(np.int32)), rows=gu.rows_dev(r.rows),
                              stream=torch.empty(max_bytes, dtype=torch.uint8, device=dev),
                              stream_bytes=torch.zeros(1, dtype=torch.int64, device=dev),
                              status=torch.full((1,), 777, dtype=torch.int32, device=dev)))
    ws = torch.empty(dk.dckv_bytes_batch(enc), dtype=torch.uint8, device=dev)
    dk.dckv_encode_batch(enc, ws)
    torch.cuda.synchronize()
    streams = []
    for e in enc:
        assert int(e.status.item()) == 0
        streams.append(e.stream[:int(e.stream_bytes.item())].clone())
    dec = [dk.Request(e.plan, e.token_ids, stream=s, capacity=s.numel(),
                      rows_out=torch.empty((int(e.token_ids.shape[0]), codec.D), dtype=torch.int16, device=dev),
                      status=torch.full((1,), 777, dtype=torch.int32, device=dev))
           for e, s in zip(enc, streams)]
    ws2 = torch.empty(dk.dckv_bytes_batch(dec), dtype=torch.uint8, device=dev)
    dk.dckv_decode_batch(dec, ws2)
    torch.cuda.synchronize()
    for d in dec:
        assert int(d.status.item()) == 0
    return dict(data=data, plans=plans, streams=[s.cpu().numpy().tobytes() for s in streams],
                rows=[d.rows_out.cpu().numpy().view(np.uint16) for d in dec])


def test_batch_equals_single_request_calls(batch):
    for r, data, rows in zip(batch["data"], batch["streams"], batch["rows"]):
        plan = batch["plans"][r.step_scale]
        gu.say("request T=%d rate %g" % (r.T, r.rate_target))
        single, st = gu.gpu_encode(plan, r.rows, r.token_ids)
        assert st == 0 and single == data
        out, st = gu.gpu_decode(plan, data, r.token_ids)
        assert st == 0 and np.array_equal(out, rows)


@pytest.mark.parametrize("k", [0, 6])
def test_batch_request_matches_oracle(batch, k):
    r, data, rows = batch["data"][k], batch["streams"][k], batch["rows"][k]
    params = synth.world().params()
    p = gu.oracle_plan(params, r.step_scale)
    gu.say("oracle check of request %d (T=%d, rate %g, C_a=%d)" % (k, r.T, r.rate_target, p.c_active))
    h, sym_g, flat_g, qe_g, _ = gu.oracle_symbols_of_stream(data, params, p, r.T)
    assert gu.oracle_stream_from_symbols(r.rows, r.T, params, p, sym_g, flat_g, qe_g) == data
    enc = ocodec.encode(r.rows, r.token_ids, params, p)
    qg = _codes(sym_g, flat_g, qe_g)
    qo = _codes(enc.sym, enc.esc_flat, enc.esc_q)
    agree = float(np.mean(qg == qo))
    gu.say("  codes agree %.7f" % agree)
    assert agree >= gu.SYMBOL_AGREEMENT and int(np.abs(qg - qo).max()) <= 1
    ok, bad = _near_tie_certified(enc, qg, qo, p, params)
    assert ok, bad
    dec = ocodec.decode(data, r.token_ids, params, p)
    e = gu.rel_l2(bf16.to_f64(rows), bf16.to_f64(dec.rows))
    gu.say("  rows rel %.3g" % e)
    assert e <= gu.REL_L2_TOL


def test_batch_with_an_invalid_request_enqueues_nothing():
    import torch
    dk = gu.dk()
    codec = gu.device_codec()
    dev = codec.device
    plan = codec.plan(synth.step_scale_for(220.0))
    reqs = []
    for i, T in enumerate([300, 400]):
        rows, tok = synth.random_rows(T, seed=90 + i)
        max_bytes, _ = plan.bytes(T)
        cap = max_bytes if i == 0 else 100  # the second one is below the stream's fixed part
        reqs.append(dk.Request(plan, gu.to_dev(tok.astype(np.int32)), rows=gu.rows_dev(rows),
                               stream=torch.empty(max(cap, 16), dtype=torch.uint8, device=dev), capacity=cap,
                               stream_bytes=torch.full((1,), 5, dtype=torch.int64, device=dev),
                               status=torch.full((1,), 777, dtype=torch.int32, device=dev)))
    ws = torch.empty(dk.dckv_bytes_batch(reqs), dtype=torch.uint8, device=dev)
    with pytest.raises(dk.DckvError) as ei:
        dk.dckv_encode_batch(reqs, ws)
    assert ei.value.code == dk.ECAPACITY and "request 1" in str(ei.value)
    torch.cuda.synchronize()
    for r in reqs:
        assert int(r.status.item()) == 777 and int(r.stream_bytes.item()) == 5
    # an empty batch is a no-op
    dk.dckv_encode_batch([], ws)
    dk.dckv_decode_batch([], ws)
