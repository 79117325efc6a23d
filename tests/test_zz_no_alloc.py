"""The allocation-free encode entry point against the workspace one.

dckv_encode_noalloc runs the kernels of dckv_encode on the library's static
scratch; its streams must equal dckv_encode's byte for byte, also on a second
call right after the first with a shorter request (the scratch keeps the
first call's contents), and a request longer than the scratch covers is
refused before anything is enqueued.
"""
from __future__ import annotations

import numpy as np
import pytest

import dckv_synth as synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _encode_both(plan, rows_bits, tok_np):
    import torch
    dk = gu.dk()
    T = rows_bits.shape[0]
    rows = gu.rows_dev(rows_bits)
    tok = gu.to_dev(tok_np.astype(np.int32))
    cap, _ = dk.dckv_bytes(plan, T)
    out = []
    for noalloc in (False, True):
        buf = torch.full((cap,), 0xA5, dtype=torch.uint8, device="cuda:0")
        nb = torch.zeros(1, dtype=torch.int64, device="cuda:0")
        st = torch.full((1,), 77, dtype=torch.int32, device="cuda:0")
        if noalloc:
            dk.dckv_encode_noalloc(plan, rows, tok, buf, nb, st)
        else:
            ws = dk.workspace(plan, T)
            dk.dckv_encode(plan, rows, tok, buf, nb, st, ws)
        torch.cuda.synchronize()
        n = int(nb.item())
        out.append((int(st.item()), n, buf[:n].cpu().numpy().tobytes()))
    return out


def test_noalloc_encode_equals_workspace_encode_twice():
    plan = gu.device_codec().plan(synth.step_scale_for(120.0))
    req = synth.make_request(2, T=8192)  # the 32K workload's seeds, outliers included, 8,192 positions
    cases = [(req.rows, req.token_ids), (req.rows[:1000], req.token_ids[:1000])]
    for T_rows, tok in cases:
        gu.say("noalloc case T=%d" % T_rows.shape[0])
        (st_a, n_a, a), (st_b, n_b, b) = _encode_both(plan, T_rows, tok)
        assert st_a == 0 and st_b == 0
        assert n_a == n_b and n_a > 0
        assert a == b


def test_noalloc_encode_rejects_requests_beyond_the_scratch():
    import torch
    dk = gu.dk()
    plan = gu.device_codec().plan(synth.step_scale_for(120.0))
    T = 16384
    rows = torch.zeros((T, synth.D), dtype=torch.int16, device="cuda:0")
    tok = torch.zeros(T, dtype=torch.int32, device="cuda:0")
    buf = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda:0")
    nb = torch.zeros(1, dtype=torch.int64, device="cuda:0")
    st = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    with pytest.raises(dk.DckvError) as e:
        dk.dckv_encode_noalloc(plan, rows, tok, buf, nb, st)
    assert e.value.code == dk.ECAPACITY
