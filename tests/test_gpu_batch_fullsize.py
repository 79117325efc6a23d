"""The 16-request batch workload at full size on the GPU, against the oracle.

Sixteen independent 8,192-token requests, each with its own seeded token ids
and a rate drawn from 60, 120, 220 and 400 bytes/token; coefficients are
Laplace with a Student-t (nu = 3) fraction.  They are encoded and decoded by
one batch call each, as one launch sequence with a shared workspace.  Bars,
per request:
  - lossless stage, every symbol: the oracle's rANS decoder reads the GPU
    stream and its encoder re-encodes those symbols to the same bytes;
  - lossy stage and decode on every coded row, as for the single-request
    workloads (codes up to certified ties, rows within relative L2 2e-3);
  - kept rows;
and a few requests are also run through the single-request calls, which must
give the same bytes and rows.
"""
from __future__ import annotations

import numpy as np
import pytest

import dckv_synth as synth
from oracle import codec as ocodec
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

CFG = 4
N_REQ = 16


@pytest.fixture(scope="module")
def batch():
    import torch
    dk = gu.dk()
    codec = gu.device_codec()
    dev = codec.device
    gu.say("generating %d requests" % N_REQ)
    data = [synth.make_request(CFG, index=i) for i in range(N_REQ)]
    plans = {}
    for r in data:
        if r.step_scale not in plans:
            plans[r.step_scale] = codec.plan(r.step_scale)
    gu.say("batch encode: T=%s, rates %s" % (sorted({r.T for r in data}), sorted({r.rate_target for r in data})))
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
    for e in enc:
        e.rows = None
        e.stream = None
    gu.say("batch decode")
    dec = [dk.Request(e.plan, e.token_ids, stream=s, capacity=s.numel(),
                      rows_out=torch.empty((int(e.token_ids.shape[0]), codec.D), dtype=torch.int16, device=dev),
                      status=torch.full((1,), 777, dtype=torch.int32, device=dev))
           for e, s in zip(enc, streams)]
    del ws
    ws2 = torch.empty(dk.dckv_bytes_batch(dec), dtype=torch.uint8, device=dev)
    dk.dckv_decode_batch(dec, ws2)
    torch.cuda.synchronize()
    rows_out = []
    for d in dec:
        assert int(d.status.item()) == 0
        rows_out.append(d.rows_out.cpu().numpy().view(np.uint16))
        d.rows_out = None
    del ws2
    return dict(data=data, plans=plans, streams=[s.cpu().numpy().tobytes() for s in streams], rows=rows_out)


@pytest.mark.parametrize("i", range(N_REQ))
def test_batch_fullsize_request_matches_oracle(batch, i):
    r, data, out = batch["data"][i], batch["streams"][i], batch["rows"][i]
    params = synth.world().params()
    p = gu.oracle_plan(params, r.step_scale)
    gu.say("request %d: T=%d rate %g C_a=%d, %d bytes" % (i, r.T, r.rate_target, p.c_active, len(data)))
    h, sym_g, flat_g, qe_g, _ = gu.oracle_symbols_of_stream(data, params, p, r.T)
    assert gu.oracle_stream_from_symbols(r.rows, r.T, params, p, sym_g, flat_g, qe_g) == data
    gu.check_all_rows(r.rows, r.token_ids, r.T, params, p, sym_g, flat_g, qe_g, out_rows=out)
    gu.check_kept_rows(r.rows, r.T, params, out)


@pytest.mark.parametrize("i", [0, 5, 15])
def test_batch_fullsize_equals_single_request_calls(batch, i):
    r = batch["data"][i]
    plan = batch["plans"][r.step_scale]
    gu.say("request %d through the single-request calls" % i)
    single, st = gu.gpu_encode(plan, r.rows, r.token_ids)
    assert st == 0 and single == batch["streams"][i]
    out, st = gu.gpu_decode(plan, single, r.token_ids)
    assert st == 0 and np.array_equal(out, batch["rows"][i])
