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
# full-size checks on sampled rows (the oracle computes them one by one)
# ---------------------------------------------------------------------------
def full_codes(sym, flat, qe, act_idx, C):
    """Codes [N][C] (int32, dropped components 0) from symbols and escapes."""
    qa = np.ascontiguousarray(sym, dtype=np.int32) - 127
    if len(flat):
        qa.reshape(-1)[flat] = qe
    q = np.zeros((sym.shape[0], C), dtype=np.int32)
    q[:, act_idx] = qa
    return q


def sample_rows(N: int, rows_coded: np.ndarray, seed: int = 4242, n_random: int = 48, n_outliers: int = 12):
    """Tile and block edges, the first and last rows, the rows of largest norm
    (outliers, when the workload has them) and seeded random rows."""
    fixed = [0, 1, 2, 3, 126, 127, 128, 129, 254, 255, 256, 257, 511, 512, 513, 32767, 32768,
             N - 4, N - 3, N - 2, N - 1]
    rng = np.random.default_rng(seed)
    rand = rng.choice(N, size=min(n_random, N), replace=False)
    norms = np.concatenate([np.linalg.norm(bf16.to_f64(rows_coded[i:i + 4096]), axis=1)
                            for i in range(0, N, 4096)])
    outl = np.argsort(norms)[-n_outliers:]
    js = np.unique(np.concatenate([np.array([j for j in fixed if 0 <= j < N]), rand, outl]))
    return js.astype(np.int64)


def check_sampled_rows(rows, tok, T, params, p, sym_g, flat_g, qe_g, js, out_rows=None, yhat_view=None):
    """Codes and decoded rows of sampled coded rows js against the oracle.

    The oracle's float64 transform and its float32 quantisation decision,
    with the GPU's even-row codes as the odd rows' neighbours (as the decoder
    has them), must give the GPU's codes up to certified ties; the oracle's
    two-pass dequantisation, correction, synthesis and RoPE of the GPU's codes
    must match the GPU's rows (and the yhat_b view, if given) within the
    float bar, in aggregate and row by row.
    """
    sh = ocodec.shape_of(params)
    N, _, coded_t = ocodec.split_positions(T, sh.keep_head, sh.keep_tail)
    C = p.step.size
    act = p.active
    qg = full_codes(sym_g, flat_g, qe_g, p.act_idx, C)
    A = bf16.to_f64(params["analysis"])
    y = bf16.to_f64(rows[coded_t[js]]) @ A.T
    need = np.unique(np.concatenate([js, js[js % 2 == 1] - 1, js[(js % 2 == 1) & (js + 1 < N)] + 1]))
    m_need = ocodec.embedding_mean(params, tok[coded_t[need]])
    pos = {int(j): i for i, j in enumerate(need)}
    step = p.step.astype(np.float64)
    a64 = params["nbr_weight"].astype(np.float64)
    mu = np.empty((len(js), C))
    for n, j in enumerate(js):
        m = m_need[pos[int(j)]].copy()
        if j % 2 == 1:
            nb = m_need[pos[int(j - 1)]] + qg[j - 1] * step
            if j + 1 < N:
                nb = nb + m_need[pos[int(j + 1)]] + qg[j + 1] * step
            m = m + a64 * nb
        mu[n] = m
    res = (y - mu) / step
    d = (y - mu)[:, act]
    qo = ocodec._decide(d, p.step[act])
    qs = qg[js][:, act].astype(np.int64)
    agree = float(np.mean(qo == qs))
    say("  sampled codes agree %.7f (%d codes)" % (agree, qo.size))
    assert agree >= SYMBOL_AGREEMENT
    for n, k in np.argwhere(qo != qs):
        # a disagreement is a tie within float32 accuracy of the residual
        rr = res[n, act][k]
        tie = 0.5 * (qo[n, k] + qs[n, k])
        tol = 2.0 ** -17 * (abs(y[n, act][k]) + abs(mu[n, act][k])) / p.step[act][k] + 1e-4
        assert abs(qo[n, k] - qs[n, k]) == 1 and abs(rr - tie) <= tol, (js[n], k, rr, qo[n, k], qs[n, k])
    yhat = mu + qg[js] * step[None, :]
    yb_bits = bf16.from_f64(yhat)
    if yhat_view is not None:
        e1 = rel_l2(bf16.to_f64(yhat_view[js]), bf16.to_f64(yb_bits))
        say("  sampled yhat_b rel %.3g (bit-equal %.5f)" % (e1, np.mean(yhat_view[js] == yb_bits)))
        assert e1 <= REL_L2_TOL
    if out_rows is None:
        return
    yb = bf16.to_f64(yb_bits)
    hb = bf16.to_f64(bf16.from_f64(ocodec.gelu(yb @ bf16.to_f64(params["w1"]).T)))
    xhat = yb @ bf16.to_f64(params["synthesis"]).T + hb @ bf16.to_f64(params["w2"]).T
    want = bf16.from_f64(ocodec.rope(xhat, coded_t[js], sh))
    got = out_rows[coded_t[js]]
    e3 = rel_l2(bf16.to_f64(got), bf16.to_f64(want))
    say("  sampled rows rel %.3g (bit-equal %.5f)" % (e3, np.mean(got == want)))
    assert e3 <= REL_L2_TOL
    for n in range(len(js)):
        assert rel_l2(bf16.to_f64(got[n]), bf16.to_f64(want[n])) <= 4 * REL_L2_TOL, js[n]


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
