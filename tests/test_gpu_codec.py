"""Full encode/decode on the GPU against the CPU oracle.

Bars: lossless stage bit-exact (the GPU's own symbols re-encoded by the oracle
give the GPU's bytes; both decoders agree on every symbol); lossy stage
symbols agree with the oracle's on >= 99.999 % of positions; decoded
coefficients and rows within relative L2 2e-3 of the oracle's decode of the
same stream.
"""
from __future__ import annotations

import numpy as np
import pytest

import dckv_synth as synth
from oracle import bf16, codec as ocodec
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _codes(sym, flat, qe):
    q = np.ascontiguousarray(sym, dtype=np.int64) - 127
    if len(flat):
        q.reshape(-1)[flat] = qe
    return q


def _near_tie_certified(enc, qg, qo, p, params):
    """Every code disagreement sits at a rounding tie within fp32 accuracy.

    For each position where the GPU's code differs from the oracle's, the
    oracle's float64 residual, recomputed with the GPU's own even-row codes as
    the odd rows' neighbours, must round to the GPU's code or lie within the
    float32 error bound of the half-integer between the two codes.
    """
    step = p.step.astype(np.float64)
    a = params["nbr_weight"].astype(np.float64)
    N = qg.shape[0]
    jj, rr = np.nonzero(qg != qo)
    cc = p.act_idx[rr]
    y, m = enc.y, enc.m
    for j, r, c in zip(jj, rr, cc):
        mu = m[j, c]
        nb = 0.0
        if j % 2 == 1:
            for k in (j - 1, j + 1):
                if 0 <= k < N:
                    nb += m[k, c] + qg[k, r] * step[c]
            mu = mu + a[c] * nb
        res = (y[j, c] - mu) / step[c]
        if int(np.rint(res)) == qg[j, r]:
            continue
        tie = 0.5 * (qg[j, r] + qo[j, r])
        tol = 2.0 ** -17 * (abs(y[j, c]) + abs(m[j, c]) + a[c] * abs(nb)) / step[c] + 1e-4
        if not (abs(qg[j, r] - qo[j, r]) == 1 and abs(res - tie) <= tol):
            return False, (j, r, res, qg[j, r], qo[j, r], tol)
    return True, None


def _run_case(rows, tok, g, params=None, codec=None, check_rows=True, min_agree=gu.SYMBOL_AGREEMENT):
    params = params or synth.world().params()
    codec = codec or gu.device_codec()
    T = rows.shape[0]
    p = gu.oracle_plan(params, g)
    plan = codec.plan(g)
    assert plan.crc == p.crc
    gu.say("encode T=%d C_a=%d g=%.6g" % (T, p.c_active, g))
    data, st = gu.gpu_encode(plan, rows, tok)
    assert st == 0
    enc = ocodec.encode(rows, tok, params, p)
    # the GPU stream is valid for the oracle's parser and decoder
    h, sym_g, flat_g, qe_g, _ = gu.oracle_symbols_of_stream(data, params, p, T)
    N = h.N
    # lossless stage: the oracle re-encodes the GPU's symbols to the GPU's bytes
    assert gu.oracle_stream_from_symbols(rows, T, params, p, sym_g, flat_g, qe_g) == data
    # lossy stage: symbol agreement with the oracle's own quantiser
    if N and p.c_active:
        qg = _codes(sym_g, flat_g, qe_g)
        qo = _codes(enc.sym, enc.esc_flat, enc.esc_q)
        agree = float(np.mean(qg == qo))
        gu.say("  codes agree %.8f  max |dq| %d  (n_esc gpu %d oracle %d)" % (
            agree, int(np.abs(qg - qo).max()), len(flat_g), len(enc.esc_flat)))
        assert agree >= min_agree
        # a disagreement is a near-tie: the two codes are neighbours
        assert int(np.abs(qg - qo).max()) <= 1
        ok, bad = _near_tie_certified(enc, qg, qo, p, params)
        assert ok, bad
    if not check_rows:
        return data, enc, plan, p
    # decode of the GPU stream on both sides
    import torch
    ws = gu.dk().workspace(plan, T)
    gu.say("decode T=%d" % T)
    out, st = gu.gpu_decode(plan, data, tok, ws=ws)
    assert st == 0
    dec = ocodec.decode(data, tok, params, p)
    if N:
        yb, _ = gu.read_view(ws, plan, T, gu.dk().VIEW_YHAT_B)
        yb = yb.view(np.uint16).reshape(N, -1)
        e1 = gu.rel_l2(bf16.to_f64(yb), bf16.to_f64(dec.yhat_b))
        hb, _ = gu.read_view(ws, plan, T, gu.dk().VIEW_H_B)
        hb = hb.view(np.uint16).reshape(N, -1)
        e2 = gu.rel_l2(bf16.to_f64(hb), bf16.to_f64(dec.h_b))
        gu.say("  yhat_b rel %.3g (bit-equal %.5f)  h_b rel %.3g" % (e1, np.mean(yb == dec.yhat_b), e2))
        assert e1 <= gu.REL_L2_TOL and e2 <= gu.REL_L2_TOL
    e3 = gu.rel_l2(bf16.to_f64(out), bf16.to_f64(dec.rows)) if T else 0.0
    gu.say("  rows rel %.3g (bit-equal %.5f)" % (e3, np.mean(out == dec.rows) if T else 1.0))
    assert e3 <= gu.REL_L2_TOL
    # kept rows: V columns bit-identical, row 0 bit-identical
    _, kept_t, _ = ocodec.split_positions(T, 4, 128)
    D = rows.shape[1]
    vcols = np.concatenate([np.arange(l * 1024 + 512, l * 1024 + 1024) for l in range(6)])
    if len(kept_t):
        assert np.array_equal(out[kept_t][:, vcols], rows[kept_t][:, vcols])
        assert np.array_equal(out[0], rows[0])
    return data, enc, plan, p


@pytest.mark.parametrize("cfg", [0, 1])
def test_codec_matches_oracle_on_workloads(cfg):
    req = synth.make_request(cfg)
    _run_case(req.rows, req.token_ids, req.step_scale)


@pytest.mark.parametrize("T", [0, 1, 100, 132, 133, 134, 135, 136, 259, 260, 261, 388, 389, 517, 645])
def test_codec_edge_lengths(T):
    rows, tok = synth.random_rows(T, seed=1000 + T)
    _run_case(rows, tok, synth.step_scale_for(220.0))


def test_codec_escapes_and_outliers():
    rows, tok = synth.random_rows(132 + 300, seed=77)
    r64 = bf16.to_f64(rows)
    r64[10:40] *= 40.0          # many codes beyond +-127
    r64[200] *= 3000.0          # very large codes
    rows = bf16.from_f64(r64)
    # codes of |r| up to ~1e4 steps: fp32 resolves ties less finely, so the
    # agreement bar is lower and every disagreement must be a certified tie
    data, enc, plan, p = _run_case(rows, tok, synth.step_scale_for(120.0), min_agree=0.99)
    assert len(enc.esc_flat) > 100


def test_codec_many_escapes_use_global_sort():
    # more than 4096 escapes: the encoder sorts them in global memory, and row
    # tiles hold more escape records than the decoder keeps in LDS
    rows, tok = synth.random_rows(132 + 600, seed=78)
    rows = bf16.from_f64(bf16.to_f64(rows) * 60.0)
    data, enc, plan, p = _run_case(rows, tok, synth.step_scale_for(400.0), min_agree=0.99)
    assert len(enc.esc_flat) > 4096
    per_row_tile = np.bincount(enc.esc_flat // p.c_active // 256)
    assert per_row_tile.max() > 2048


def test_codec_with_dropped_components():
    w = synth.world()
    rng = np.random.default_rng(5)
    scale = w.laplace_scale.copy()
    scale[rng.choice(2048, size=77, replace=False)] = 1e-5
    params = gu.params_with_scales(scale)
    codec = gu.codec_with_scales(scale)
    rows, tok = synth.random_rows(132 + 290, seed=79)
    _run_case(rows, tok, synth.step_scale_for(220.0), params=params, codec=codec)


def test_codec_deterministic_bytes():
    req = synth.make_request(0)
    plan = gu.device_codec().plan(req.step_scale)
    a, _ = gu.gpu_encode(plan, req.rows, req.token_ids)
    b, _ = gu.gpu_encode(plan, req.rows, req.token_ids)
    assert a == b


def test_codec_cross_decode_oracle_stream():
    req = synth.make_request(0)
    params = synth.world().params()
    p = gu.oracle_plan(params, req.step_scale)
    enc = ocodec.encode(req.rows, req.token_ids, params, p)
    dec = ocodec.decode(enc.data, req.token_ids, params, p)
    plan = gu.device_codec().plan(req.step_scale)
    gu.say("gpu decode of the oracle's stream")
    out, st = gu.gpu_decode(plan, enc.data, req.token_ids)
    assert st == 0
    assert gu.rel_l2(bf16.to_f64(out), bf16.to_f64(dec.rows)) <= gu.REL_L2_TOL


def test_codec_status_codes():
    import torch
    dk = gu.dk()
    rows, tok = synth.random_rows(132 + 40, seed=80)
    plan = gu.device_codec().plan(synth.step_scale_for(220.0))
    bad = rows.copy()
    bad[20, 7] = 0x7FC0  # NaN in a coded row (coded positions are 4..43)
    gu.say("encode with a NaN row")
    _, st = gu.gpu_encode(plan, bad, tok)
    assert st == dk.EINVAL
    gu.say("encode with an out-of-range token id")
    tk = tok.copy()
    tk[20] = 40000
    _, st = gu.gpu_encode(plan, rows, tk)
    assert st == dk.EINVAL
    gu.say("encode into a too small stream buffer")
    s, st = dk.encode(plan, gu.rows_dev(rows), gu.to_dev(tok.astype(np.int32)),
                      capacity=64 + 132 * 12288 + 4 * 33 + 100)
    torch.cuda.synchronize()
    assert st == dk.ECAPACITY and s.numel() == 0
    with pytest.raises(dk.DckvError):
        dk.encode(plan, gu.rows_dev(rows), gu.to_dev(tok.astype(np.int32)), capacity=1000)
    data, st = gu.gpu_encode(plan, rows, tok)
    gu.say("decode with an out-of-range token id")
    _, st = gu.gpu_decode(plan, data, tk)
    assert st == dk.EINVAL
    gu.say("decode with the wrong plan / corrupt header")
    other = gu.device_codec().plan(synth.step_scale_for(120.0))
    _, st = gu.gpu_decode(other, data, tok)
    assert st == dk.EPLAN
    bad = bytearray(data)
    bad[20] ^= 2  # N
    _, st = gu.gpu_decode(plan, bytes(bad), tok)
    assert st == dk.ECORRUPT


def test_codec_escape_overflow_is_ecapacity():
    """More escapes than the workspace holds (max(4096, N C_a / 16) records)
    set ECAPACITY and a zero stream size; the stream bound dckv_bytes reports
    is consistent with that cap."""
    import torch
    dk = gu.dk()
    plan = gu.device_codec().plan(synth.step_scale_for(220.0))
    T = 132 + 600
    rows, tok = synth.random_rows(T, seed=81, gain=2000.0)
    max_bytes, _ = dk.dckv_bytes(plan, T)
    N, Ca = T - 132, plan.c_active
    n_blk = (N + 255) // 256
    fixed = 64 + 132 * 12288 + 4 * (n_blk * ((Ca + 63) // 64) + 1)
    cap = max(4096, N * Ca // 16)
    assert max_bytes == fixed + 2 * N * Ca + 4 * n_blk * Ca + 6 * cap
    gu.say("encode with about 3/4 of the codes escaped")
    s, st = dk.encode(plan, gu.rows_dev(rows), gu.to_dev(tok.astype(np.int32)))
    torch.cuda.synchronize()
    assert st == dk.ECAPACITY and s.numel() == 0


def test_request_length_cap():
    """Requests above 2^18 positions (a [T][6,144] bf16 operand past 3 GiB, where
    32-bit operand offsets end) are refused before anything is enqueued."""
    dk = gu.dk()
    plan = gu.device_codec().plan(synth.step_scale_for(220.0))
    max_bytes, ws = dk.dckv_bytes(plan, 1 << 18)
    assert max_bytes > 0 and ws > 0
    with pytest.raises(dk.DckvError) as e:
        dk.dckv_bytes(plan, (1 << 18) + 1)
    assert e.value.code == dk.EUNSUPPORTED
    with pytest.raises(dk.DckvError):
        dk.dckv_rate_bytes(plan, (1 << 18) + 1)
    with pytest.raises(dk.DckvError):
        dk.dckv_rate_backward_bytes(plan, (1 << 18) + 1)
    assert dk.dckv_rate_bytes(plan, 1 << 18) > 0
