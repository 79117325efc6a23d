"""Shared helpers of the GPU parity tests (device setup, oracle runs)."""
from __future__ import annotations

import copy
import functools
import sys

import numpy as np

import dckv_synth as synth
from oracle import bf16, codec as ocodec, plan as oplan, rans as orans, stream as ostream

REL_L2_TOL = 2e-3          # float stages: coefficients and reconstructed rows
SYMBOL_AGREEMENT = 0.99999  # integer symbols of the lossy stage


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=None)
def dk():
    import learned_kv_cache_dckv_amd as m
    return m


@functools.lru_cache(maxsize=None)
def device_codec():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return dk().Codec(synth.world().params(), device="cuda:0")


def codec_with_scales(laplace_scale: np.ndarray):
    """Same device weights, other Laplace scales (to force dropped components)."""
    c = copy.copy(device_codec())
    c.laplace_scale = np.ascontiguousarray(laplace_scale, dtype=np.float32)
    return c


def params_with_scales(laplace_scale: np.ndarray) -> dict:
    p = dict(synth.world().params())
    p["laplace_scale"] = np.ascontiguousarray(laplace_scale, dtype=np.float32)
    return p


def oracle_plan(params: dict, g: float):
    return oplan.make_plan(np.float32(g), params["base_step"], params["laplace_scale"])


def to_dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to("cuda:0")


def rows_dev(rows_bits: np.ndarray):
    import torch
    return to_dev(rows_bits.view(np.int16)).view(torch.bfloat16)


def gpu_encode(plan, rows_bits, tok):
    import torch
    s, st = dk().encode(plan, rows_dev(rows_bits), to_dev(tok.astype(np.int32)))
    torch.cuda.synchronize()
    return s.cpu().numpy().tobytes(), st


def gpu_decode(plan, data: bytes, tok, ws=None):
    import torch
    buf = to_dev(np.frombuffer(data, dtype=np.uint8).copy()) if len(data) else torch.zeros(64, dtype=torch.uint8,
                                                                                          device="cuda:0")
    out, st = dk().decode(plan, buf[:len(data)] if len(data) else buf[:0], to_dev(tok.astype(np.int32)), ws=ws)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16), st


def gpu_entropy_decode(plan, data: bytes, T: int, N: int, Ca: int, ws=None):
    """Symbols [N][C_a] of a stream from the GPU's rANS decoder alone
    (dckv_entropy_decode), the escape count and the status."""
    import torch
    buf = to_dev(np.frombuffer(data, np.uint8).copy())
    sym = torch.full((max(N * Ca, 1),), 7, dtype=torch.uint8, device="cuda:0")
    ne = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    st = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    if ws is None:
        ws = dk().workspace(plan, T)
    dk().dckv_entropy_decode(plan, buf, len(data), T, sym, ne, st, ws)
    torch.cuda.synchronize()
    return sym[:N * Ca].cpu().numpy().reshape(N, Ca), int(ne.item()), int(st.item())


def read_view(ws, plan, T, which):
    """Bytes of one workspace view (after a call that filled it)."""
    off, nb, rs = dk().dckv_workspace_view(plan, T, which)
    return ws[off:off + nb].cpu().numpy(), rs


def tiled_symbols(buf: np.ndarray, N: int, Ca: int) -> np.ndarray:
    """Group-tiled symbol bytes -> [N][C_a]."""
    N256 = (N + 255) // 256 * 256
    G = (Ca + 63) // 64
    t = buf[:G * N256 * 64].reshape(G, N256 // 4, 64, 4)  # [g][quad][lane][row-in-quad]
    full = t.transpose(1, 3, 0, 2).reshape(N256, G * 64)
    return full[:N, :Ca]


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / den) if den > 0 else float(np.linalg.norm(a - b))


def oracle_symbols_of_stream(data: bytes, params: dict, p, T: int):
    """Parse a stream and rANS-decode it with the oracle (validates the format)."""
    h, kept, flat, qe, groups = ostream.parse(data, synth.D)
    ocodec.check_header(h, T, params, p)
    esc = np.zeros((h.N, p.c_active), dtype=bool)
    if len(flat):
        esc.reshape(-1)[flat] = True
    sym = orans.decode_all(groups, p.freq, p.cum, h.N, esc) if h.N and p.c_active else \
        np.full((h.N, p.c_active), 255, np.uint8)
    return h, sym, flat, qe, groups


def oracle_stream_from_symbols(rows, T, params, p, sym, flat, qe) -> bytes:
    sh = ocodec.shape_of(params)
    N, kept_t, _ = ocodec.split_positions(T, sh.keep_head, sh.keep_tail)
    groups = orans.encode_all(sym, p.freq, p.cum) if N and p.c_active else []
    n_blk, G, _, _ = orans.group_shape(N, p.c_active)
    h = ostream.Header(T=T, keep_head=sh.keep_head, keep_tail=sh.keep_tail, N=N, n_coef=p.step.size,
                       c_active=p.c_active, n_groups=n_blk * G, n_esc=len(flat), step_scale=float(p.step_scale),
                       plan_crc=p.crc, total_bytes=0, rans_bytes=0)
    return ostream.write(h, rows[kept_t], groups, flat, qe)


# ---------------------------------------------------------------------------
# full-size checks of every row (the oracle runs over chunks of rows)
# ---------------------------------------------------------------------------
def full_codes(sym, flat, qe, act_idx, C):
    """Codes [N][C] (int32, dropped components 0) from symbols and escapes."""
    qa = np.ascontiguousarray(sym, dtype=np.int32) - 127
    if len(flat):
        qa.reshape(-1)[flat] = qe
    q = np.zeros((sym.shape[0], C), dtype=np.int32)
    q[:, act_idx] = qa
    return q


def _rows_core(rows, tok, T, params, p, qg, js, out_rows=None, yhat_view=None):
    """Codes and decoded rows of coded rows js against the oracle (one chunk).

    The oracle's float64 transform and its float32 quantisation decision,
    with the GPU's even-row codes as the odd rows' neighbours (as the decoder
    has them), must give the GPU's codes up to certified ties (asserted here,
    for every disagreement, even and odd rows alike).  Returns the counts and
    squared-error sums the callers' aggregate bars need, and the worst
    per-row relative error of the decoded rows.
    """
    sh = ocodec.shape_of(params)
    N, _, coded_t = ocodec.split_positions(T, sh.keep_head, sh.keep_tail)
    C = p.step.size
    act = p.active
    A = bf16.to_f64(params["analysis"])
    y = bf16.to_f64(rows[coded_t[js]]) @ A.T
    need = np.unique(np.concatenate([js, js[js % 2 == 1] - 1, js[(js % 2 == 1) & (js + 1 < N)] + 1]))
    m_need = ocodec.embedding_mean(params, tok[coded_t[need]])
    pos = np.searchsorted(need, js)
    step = p.step.astype(np.float64)
    a64 = params["nbr_weight"].astype(np.float64)
    mu = m_need[pos].copy()
    odd = np.nonzero(js % 2 == 1)[0]
    if odd.size:
        jl = js[odd] - 1
        nb = m_need[np.searchsorted(need, jl)] + qg[jl] * step[None, :]
        has_r = js[odd] + 1 < N
        jr = js[odd][has_r] + 1
        nb[has_r] += m_need[np.searchsorted(need, jr)] + qg[jr] * step[None, :]
        mu[odd] += a64[None, :] * nb
    res = (y - mu) / step
    d = (y - mu)[:, act]
    qo = ocodec._decide(d, p.step[act])
    qs = qg[js][:, act].astype(np.int64)
    dis = np.argwhere(qo != qs)
    for n, k in dis:
        # a disagreement is a tie within float32 accuracy of the residual
        rr = res[n, act][k]
        tie = 0.5 * (qo[n, k] + qs[n, k])
        tol = 2.0 ** -17 * (abs(y[n, act][k]) + abs(mu[n, act][k])) / p.step[act][k] + 1e-4
        assert abs(qo[n, k] - qs[n, k]) == 1 and abs(rr - tie) <= tol, (js[n], k, rr, qo[n, k], qs[n, k])
    st = dict(n_codes=int(qo.size), n_dis=int(len(dis)), n_odd_dis=int(np.sum(js[dis[:, 0]] % 2 == 1)) if len(dis)
              else 0, yhat=(0.0, 0.0), rows=(0.0, 0.0), worst_row=0.0, rows_bit_equal=0, rows_values=0)
    yhat = mu + qg[js] * step[None, :]
    yb_bits = bf16.from_f64(yhat)
    if yhat_view is not None:
        a, b = bf16.to_f64(yhat_view[js]), bf16.to_f64(yb_bits)
        st["yhat"] = (float(np.sum((a - b) ** 2)), float(np.sum(b ** 2)))
    if out_rows is None:
        return st
    yb = bf16.to_f64(yb_bits)
    xhat = yb @ bf16.to_f64(params["synthesis"]).T
    if params.get("w1") is not None:
        hb = bf16.to_f64(bf16.from_f64(ocodec.gelu(yb @ bf16.to_f64(params["w1"]).T)))
        xhat = xhat + hb @ bf16.to_f64(params["w2"]).T
    want = bf16.from_f64(ocodec.rope(xhat, coded_t[js], sh))
    got = out_rows[coded_t[js]]
    g64, w64 = bf16.to_f64(got), bf16.to_f64(want)
    num = np.sum((g64 - w64) ** 2, axis=1)
    den = np.sum(w64 ** 2, axis=1)
    st["rows"] = (float(num.sum()), float(den.sum()))
    per = np.sqrt(num / np.maximum(den, 1e-300))
    st["worst_row"] = float(per.max())
    st["rows_bit_equal"] = int(np.sum(got == want))
    st["rows_values"] = int(got.size)
    return st


def _assert_rows_stats(st, what):
    agree = 1.0 - st["n_dis"] / max(st["n_codes"], 1)
    say("  %s codes agree %.7f (%d codes, %d ties of which %d on odd rows)" %
        (what, agree, st["n_codes"], st["n_dis"], st["n_odd_dis"]))
    assert agree >= SYMBOL_AGREEMENT
    if st["yhat"][1] > 0:
        e1 = float(np.sqrt(st["yhat"][0] / st["yhat"][1]))
        say("  %s yhat_b rel %.3g" % (what, e1))
        assert e1 <= REL_L2_TOL
    if st["rows"][1] > 0:
        e3 = float(np.sqrt(st["rows"][0] / st["rows"][1]))
        say("  %s rows rel %.3g, worst row %.3g (bit-equal %.5f)" %
            (what, e3, st["worst_row"], st["rows_bit_equal"] / max(st["rows_values"], 1)))
        assert e3 <= REL_L2_TOL
        assert st["worst_row"] <= 4 * REL_L2_TOL


def check_all_rows(rows, tok, T, params, p, sym_g, flat_g, qe_g, out_rows=None, yhat_view=None, chunk=4096):
    """Codes and decoded rows of every coded row against the oracle, in chunks
    of rows.  The bars apply to the whole request: codes >= 99.999 % equal and
    every disagreement a certified tie; coefficients (when the yhat_b view is
    given) and rows within relative L2 2e-3, every row within 4x that."""
    sh = ocodec.shape_of(params)
    N = max(T - sh.keep_head - sh.keep_tail, 0)
    qg = full_codes(sym_g, flat_g, qe_g, p.act_idx, p.step.size)
    tot = None
    for c0 in range(0, N, chunk):
        js = np.arange(c0, min(c0 + chunk, N), dtype=np.int64)
        st = _rows_core(rows, tok, T, params, p, qg, js, out_rows, yhat_view)
        if tot is None:
            tot = st
        else:
            for k in ("n_codes", "n_dis", "n_odd_dis", "rows_bit_equal", "rows_values"):
                tot[k] += st[k]
            for k in ("yhat", "rows"):
                tot[k] = (tot[k][0] + st[k][0], tot[k][1] + st[k][1])
            tot["worst_row"] = max(tot["worst_row"], st["worst_row"])
    if tot is not None:
        _assert_rows_stats(tot, "all %d rows:" % N)
    return tot


def check_kept_rows(rows, T, params, out_rows):
    """Kept rows: RoPE'd keys within the float bar, values and row 0 bit-identical."""
    sh = ocodec.shape_of(params)
    _, kept_t, _ = ocodec.split_positions(T, sh.keep_head, sh.keep_tail)
    if not len(kept_t):
        return
    want = bf16.from_f64(ocodec.rope(bf16.to_f64(rows[kept_t]), kept_t, sh))
    got = out_rows[kept_t]
    assert rel_l2(bf16.to_f64(got), bf16.to_f64(want)) <= REL_L2_TOL
    vcols = np.concatenate([np.arange(l * 1024 + 512, l * 1024 + 1024) for l in range(sh.n_layers)])
    assert np.array_equal(got[:, vcols], rows[kept_t][:, vcols])
    assert np.array_equal(out_rows[0], rows[0])
