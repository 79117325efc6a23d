"""Lossless stage on the GPU against the oracle: bit-exact bytes and symbols."""
from __future__ import annotations

import numpy as np
import pytest

import dckv_synth as synth
from oracle import codec as ocodec, rans as orans
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _entropy_encode(plan, T, sym, flat, qe, rows_bits):
    import torch
    dk = gu.dk()
    N, Ca = sym.shape
    dev = "cuda:0"
    sym_d = gu.to_dev(sym.astype(np.uint8).reshape(-1)) if sym.size else torch.zeros(1, dtype=torch.uint8,
                                                                                     device=dev)
    esc = np.empty(2 * len(flat), np.uint32)
    esc[0::2] = flat
    esc[1::2] = qe.astype(np.int64).astype(np.uint32)
    esc_d = gu.to_dev(esc.view(np.int32)) if len(flat) else torch.zeros(2, dtype=torch.int32, device=dev)
    max_bytes, _ = plan.bytes(T)
    buf = torch.empty(max_bytes, dtype=torch.uint8, device=dev)
    nb = torch.zeros(1, dtype=torch.int64, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = dk.workspace(plan, T)
    dk.dckv_entropy_encode(plan, T, sym_d, esc_d, len(flat), gu.rows_dev(rows_bits), buf, nb, st, ws)
    torch.cuda.synchronize()
    return buf[:int(nb.item())].cpu().numpy().tobytes(), int(st.item())


def _entropy_decode(plan, data, T, N, Ca):
    return gu.gpu_entropy_decode(plan, data, T, N, Ca)


@pytest.fixture(scope="module")
def c0():
    w = synth.world()
    req = synth.make_request(0)
    params = w.params()
    p = gu.oracle_plan(params, req.step_scale)
    enc = ocodec.encode(req.rows, req.token_ids, params, p)
    plan = gu.device_codec().plan(req.step_scale)
    return req, params, p, enc, plan


def test_entropy_encode_bytes_equal_oracle(c0):
    req, params, p, enc, plan = c0
    gu.say("entropy_encode c0 T=%d N=%d C_a=%d" % (req.T, enc.N, p.c_active))
    data, st = _entropy_encode(plan, req.T, enc.sym, enc.esc_flat, enc.esc_q, req.rows)
    assert st == 0
    assert data == enc.data


def test_entropy_decode_symbols_equal_oracle(c0):
    req, params, p, enc, plan = c0
    gu.say("entropy_decode c0")
    sym, n_esc, st = _entropy_decode(plan, enc.data, req.T, enc.N, p.c_active)
    assert st == 0 and n_esc == len(enc.esc_flat)
    assert np.array_equal(sym, enc.sym)


def _random_case(rng, N, Ca, esc_frac):
    sym = np.clip(np.rint(rng.laplace(127, 4.0, size=(N, Ca))), 0, 254).astype(np.uint8)
    # alphabet edges
    if N * Ca:
        sym.reshape(-1)[rng.integers(0, N * Ca, size=max(1, N * Ca // 50))] = rng.choice([0, 1, 253, 254])
    esc = rng.random((N, Ca)) < esc_frac
    sym[esc] = 255
    jj, rr = np.nonzero(esc)
    flat = (jj * Ca + rr).astype(np.int64)
    qe = (rng.integers(128, 2 ** 31 - 128, size=flat.size) * rng.choice([-1, 1], size=flat.size)).astype(np.int64)
    return sym, flat, qe


@pytest.mark.parametrize("T,n_drop,esc_frac", [
    (133, 0, 0.0), (135, 0, 0.01), (132 + 255, 0, 0.001), (132 + 256, 0, 0.0), (132 + 257, 48, 0.002),
    (132 + 600, 2011, 0.05), (132 + 300, 2047, 0.0), (40, 0, 0.0), (132 + 1100, 5, 0.05)])
def test_entropy_random_symbols_round_trip_bit_exact(T, n_drop, esc_frac):
    rng = np.random.default_rng(T * 7 + n_drop)
    w = synth.world()
    scale = w.laplace_scale.copy()
    if n_drop:
        scale[rng.choice(2048, size=n_drop, replace=False)] = 1e-6
    params = gu.params_with_scales(scale)
    g = synth.step_scale_for(220.0)
    p = gu.oracle_plan(params, g)
    assert p.c_active == 2048 - n_drop
    plan = gu.codec_with_scales(scale).plan(g)
    assert plan.c_active == p.c_active and plan.crc == p.crc
    N = max(T - 132, 0)
    sym, flat, qe = _random_case(rng, N, p.c_active, esc_frac)
    rows, _ = synth.random_rows(T, seed=T)
    gu.say("entropy random T=%d N=%d C_a=%d n_esc=%d" % (T, N, p.c_active, len(flat)))
    want = gu.oracle_stream_from_symbols(rows, T, params, p, sym, flat, qe)
    data, st = _entropy_encode(plan, T, sym, flat, qe, rows)
    assert st == 0
    assert data == want
    back, n_esc, st = _entropy_decode(plan, want, T, N, p.c_active)
    assert st == 0 and n_esc == len(flat)
    assert np.array_equal(back, sym)


def test_entropy_decode_rejects_corrupt_and_foreign_streams(c0):
    req, params, p, enc, plan = c0
    data = bytearray(enc.data)
    from oracle import stream as ostream
    h = ostream.header(enc.data)
    rans_start = h.total_bytes - h.rans_bytes
    gu.say("entropy corrupt streams")
    detected = 0
    for k in range(6):
        bad = bytearray(data)
        bad[rans_start + (k * 977) % h.rans_bytes] ^= 0x41
        sym, _, st = _entropy_decode(plan, bytes(bad), req.T, enc.N, p.c_active)
        if st == gu.dk().ECORRUPT:
            detected += 1
        else:
            assert st == 0 and not np.array_equal(sym, enc.sym)
    assert detected >= 3
    bad = bytearray(data)
    bad[8] ^= 1  # T
    _, _, st = _entropy_decode(plan, bytes(bad), req.T, enc.N, p.c_active)
    assert st == gu.dk().ECORRUPT
    other = gu.device_codec().plan(req.step_scale * 1.01)
    _, _, st = _entropy_decode(other, enc.data, req.T, enc.N, other.c_active)
    assert st == gu.dk().EPLAN
    with pytest.raises(gu.dk().DckvError):
        _entropy_decode(plan, bytes(data[:100]), req.T, enc.N, p.c_active)
