"""Encode and decode captured in one HIP graph and replayed.

The calls only enqueue kernels on the caller's stream: no allocation, no
memset, no host synchronisation, so a serving loop can capture them.  The
decode is given the stream buffer's capacity (the parser accepts any size at
or above the stream's own total).  The graph is replayed three times with
eager codec work and synchronisations in between, and every replay must give
the eager call's stream bytes and decoded rows exactly.
"""
from __future__ import annotations

import numpy as np
import pytest

import dckv_synth as synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def test_encode_decode_graph_replays_match_eager():
    import torch
    dk = gu.dk()
    req = synth.make_request(1)
    plan = gu.device_codec().plan(req.step_scale)
    dev = gu.device_codec().device
    T = req.T
    rows = gu.rows_dev(req.rows)
    tok = gu.to_dev(req.token_ids.astype(np.int32))
    max_bytes, ws_bytes = dk.dckv_bytes(plan, T)
    gu.say("eager encode + decode, T=%d" % T)
    ref_stream, st = dk.encode(plan, rows, tok)
    assert st == 0
    ref_rows, st = dk.decode(plan, ref_stream, tok)
    assert st == 0
    ref_stream = ref_stream.clone()
    ref_rows = ref_rows.clone()

    buf = torch.zeros(max_bytes, dtype=torch.uint8, device=dev)
    nb = torch.zeros(1, dtype=torch.int64, device=dev)
    st_e = torch.full((1,), 777, dtype=torch.int32, device=dev)
    st_d = torch.full((1,), 777, dtype=torch.int32, device=dev)
    ws_e = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_d = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.zeros((T, plan.codec.D), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    gu.say("capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dk.dckv_encode(plan, rows, tok, buf, nb, st_e, ws_e)
        dk.dckv_decode(plan, buf, max_bytes, tok, out, st_d, ws_d)
    torch.cuda.synchronize()

    other_rows, other_tok = synth.random_rows(132 + 300, seed=41)
    for rep in range(3):
        # poison the outputs, then eager work of another request in between
        buf.fill_(0xAB)
        out.fill_(1.0)
        nb.fill_(0)
        st_e.fill_(777)
        st_d.fill_(777)
        s2, st2 = gu.gpu_encode(plan, other_rows, other_tok)
        assert st2 == 0
        torch.cuda.synchronize()
        gu.say("replay %d" % rep)
        g.replay()
        torch.cuda.synchronize()
        n = int(nb.item())
        assert int(st_e.item()) == 0 and int(st_d.item()) == 0
        assert n == ref_stream.numel()
        assert torch.equal(buf[:n], ref_stream)
        assert torch.equal(out.view(torch.int16), ref_rows.view(torch.int16))
