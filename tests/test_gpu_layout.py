"""Cache-layout integration on the GPU: decoding into the attention layers'
head matrices, and the inverse RoPE that takes a post-RoPE cache back to the
pre-RoPE rows the codec codes (DCKV digest, "How it works", first paragraph).

Bars: dckv_decode_heads gives exactly the values of dckv_decode (bit for bit,
kept rows included, rows past N untouched in neither layout) and is within the
rows' bar of the oracle's decode of the same stream; dckv_unrope
equals the oracle's float64 inverse rotation rounded once to bf16 on every
value, in place or not, and takes a decode's post-RoPE output back to the
oracle's pre-RoPE reconstruction within the rows' bar plus one bf16 rounding;
dckv_encode_postrope writes the stream of unrope followed by encode, byte for
byte, whose codes and rows match the oracle's encode of the oracle's unrope.
"""
from __future__ import annotations

import numpy as np
import pytest

import dckv_synth as synth
from oracle import bf16, codec as ocodec
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _heads_to_rows(kv, T):
    """[2 l + kv][h][t][d] -> rows [t][((l 2 + kv) 2 + h) 256 + d]."""
    a = np.stack([k.cpu().numpy().view(np.uint16) for k in kv])  # [12][2][T][256]
    return np.ascontiguousarray(a.transpose(2, 0, 1, 3).reshape(T, -1))


@pytest.mark.parametrize("case", ["c0", "c1", "T100", "T133", "T389"])
def test_decode_heads_equals_decode(case):
    import torch
    if case.startswith("c"):
        req = synth.make_request(int(case[1]))
        rows, tok, g = req.rows, req.token_ids, req.step_scale
    else:
        T = int(case[1:])
        rows, tok = synth.random_rows(T, seed=3000 + T)
        g = synth.step_scale_for(220.0)
    plan = gu.device_codec().plan(g)
    data, st = gu.gpu_encode(plan, rows, tok)
    assert st == 0
    want, st = gu.gpu_decode(plan, data, tok)
    assert st == 0
    buf = gu.to_dev(np.frombuffer(data, dtype=np.uint8).copy())
    kv, st = gu.dk().decode_heads(plan, buf, gu.to_dev(tok.astype(np.int32)))
    torch.cuda.synchronize()
    assert st == 0
    got = _heads_to_rows(kv, len(tok))
    gu.say("%s: T=%d heads layout equal %s" % (case, len(tok), np.array_equal(got, want)))
    assert np.array_equal(got, want)
    # and against the oracle's decode of the same stream, kept rows included
    params = synth.world().params()
    p = gu.oracle_plan(params, g)
    dec = ocodec.decode(data, tok, params, p)
    e = gu.rel_l2(bf16.to_f64(got), bf16.to_f64(dec.rows))
    gu.say("  heads layout vs oracle decode: rel %.3g" % e)
    assert e <= gu.REL_L2_TOL
    gu.check_kept_rows(rows, len(tok), params, got)


def test_unrope_matches_oracle_and_inverts_decode_rope():
    import torch
    req = synth.make_request(1)
    params = synth.world().params()
    sh = ocodec.shape_of(params)
    plan = gu.device_codec().plan(req.step_scale)
    data, st = gu.gpu_encode(plan, req.rows, req.token_ids)
    assert st == 0
    post, st = gu.gpu_decode(plan, data, req.token_ids)  # post-RoPE rows
    assert st == 0
    T = post.shape[0]
    t = np.arange(T)
    want = bf16.from_f64(ocodec.unrope(bf16.to_f64(post), t, sh))
    src = gu.rows_dev(post)
    dst = torch.empty_like(src)
    gu.dk().dckv_unrope(plan, src, dst)
    gu.dk().dckv_unrope(plan, src, src)  # in place
    torch.cuda.synchronize()
    got = dst.view(torch.int16).cpu().numpy().view(np.uint16)
    got_in_place = src.view(torch.int16).cpu().numpy().view(np.uint16)
    frac = float(np.mean(got == want))
    gu.say("unrope T=%d: bit-equal %.7f" % (T, frac))
    assert np.array_equal(got, want) and np.array_equal(got_in_place, want)
    # back to the pre-RoPE reconstruction: the oracle's xhat, within the rows'
    # bar plus one more bf16 rounding (RMS 2^-8 / sqrt(12) ~ 1.1e-3 relative)
    p = gu.oracle_plan(params, req.step_scale)
    dec = ocodec.decode(data, req.token_ids, params, p)
    _, _, coded_t = ocodec.split_positions(T, sh.keep_head, sh.keep_tail)
    e = gu.rel_l2(bf16.to_f64(got[coded_t]), dec.xhat)
    gu.say("  pre-RoPE rows vs oracle xhat: rel %.3g" % e)
    assert e <= gu.REL_L2_TOL + 2.0 ** -8 / np.sqrt(12.0)


@pytest.mark.parametrize("case", ["c1", "T389", "T100"])
def test_encode_postrope_matches_unrope_then_encode(case):
    """dckv_encode_postrope of a post-RoPE cache (a decode's output) writes the
    stream dckv_encode writes for dckv_unrope of it, byte for byte, and its
    codes and decoded rows match the oracle's encode of the oracle's unrope
    (codes up to certified ties, rows within the bar)."""
    import torch
    dk = gu.dk()
    params = synth.world().params()
    sh = ocodec.shape_of(params)
    if case == "c1":
        req = synth.make_request(1)
        rows, tok, g = req.rows, req.token_ids, req.step_scale
    else:
        T = int(case[1:])
        rows, tok = synth.random_rows(T, seed=4000 + T)
        g = synth.step_scale_for(120.0)
    plan = gu.device_codec().plan(g)
    data, st = gu.gpu_encode(plan, rows, tok)
    assert st == 0
    post, st = gu.gpu_decode(plan, data, tok)  # a post-RoPE cache
    assert st == 0
    T = post.shape[0]
    tk = gu.to_dev(tok.astype(np.int32))
    src = gu.rows_dev(post)
    # the two-step GPU path
    pre = torch.empty_like(src)
    dk.dckv_unrope(plan, src, pre)
    cap, _ = dk.dckv_bytes(plan, T)
    outs = []
    for fused in (False, True):
        buf = torch.full((cap,), 0x5A, dtype=torch.uint8, device="cuda:0")
        nb = torch.zeros(1, dtype=torch.int64, device="cuda:0")
        stt = torch.full((1,), 9, dtype=torch.int32, device="cuda:0")
        if fused:
            ws = torch.empty(dk.dckv_bytes_postrope(plan, T), dtype=torch.uint8, device="cuda:0")
            dk.dckv_encode_postrope(plan, src, tk, buf, nb, stt, ws)
        else:
            ws = gu.dk().workspace(plan, T)
            dk.dckv_encode(plan, pre, tk, buf, nb, stt, ws)
        torch.cuda.synchronize()
        assert int(stt.item()) == 0
        outs.append(buf[:int(nb.item())].cpu().numpy().tobytes())
    gu.say("%s: T=%d post-RoPE encode %d bytes, equal to unrope + encode: %s" %
           (case, T, len(outs[1]), outs[0] == outs[1]))
    assert outs[0] == outs[1]
    # and against the oracle's encode of the oracle's unrope
    p = gu.oracle_plan(params, g)
    pre_o = bf16.from_f64(ocodec.unrope(bf16.to_f64(post), np.arange(T), sh))
    h, sym_g, flat_g, qe_g, _ = gu.oracle_symbols_of_stream(outs[1], params, p, T)
    assert gu.oracle_stream_from_symbols(pre_o, T, params, p, sym_g, flat_g, qe_g) == outs[1]
    out, st = gu.gpu_decode(plan, outs[1], tok)
    assert st == 0
    gu.check_all_rows(pre_o, tok, T, params, p, sym_g, flat_g, qe_g, out_rows=out)
    gu.check_kept_rows(pre_o, T, params, out)
