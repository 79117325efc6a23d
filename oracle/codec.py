"""Encode and decode of one request's prompt KV cache (CPU, float64).

Sources: DCKV digest page (trove.briskstack.com, "DCKV: Learned Transform
Coding of the Prompt KV Cache in Hybrid Language Models"), section "How it
works" with its Transform, Coding and Conditional entropy models bullets, and
the paper abstract (entropy models conditioned on the prompt tokens and on
already decoded neighbouring positions).

Readings taken where the pages are silent (each is used below):
  * Row layout: column ((l*2 + kv)*n_kv_heads + h)*head_dim + d, kv = 0 for
    keys.  Kept positions are t < keep_head or t >= T - keep_tail; they travel
    verbatim (pre-RoPE).  If T <= keep_head + keep_tail every row is kept.
    Coded row j is position t = j + keep_head.
  * Conditional mean of coded row j: mu_j = H E[tok_t] for even j; for odd j
    mu_j = H E[tok_t] + a * (yhat_{j-1} + yhat_{j+1}) with yhat_N = 0 (the
    right neighbour of the last row is missing).  Neighbours are the decoded
    coefficients yhat = mu + q * step; the encoder uses the same reconstructed
    values the decoder will have (closed loop).  Even rows first, then odd
    rows: two passes at any length.
  * The quantisation decision is taken in float32, the precision of the GPU
    kernel: d = fp32(y - mu), r = fp32(d / step) (IEEE division),
    q = round-half-even(r), clamped to +-(2^31 - 128).  Components that are
    dropped are not coded: q = 0, yhat = mu.
  * |q| > 127 is an escape: symbol slot 255 (skipped by rANS) plus a record
    {flat = j*C_a + rank, q}, records in ascending flat order.
  * Decode side: yhat_b = bf16(yhat); h = GELU(W1 yhat_b) with the exact erf
    GELU, h_b = bf16(h); xhat = S yhat_b + W2 h_b; RoPE (rotate-half,
    w_i = theta^(-i/(head_dim/2)), angle t*w_i in float64) on the key columns;
    output bf16.  Kept rows get the same RoPE, so the output is a uniform
    post-RoPE cache.
  * The linear codec (Evidence section, which compares its stored payload
    with DCKV's) is read as the same codec without the nonlinear correction:
    params without "w1" / "w2" decode to xhat = S yhat_b.  Encoding does not
    involve the correction, so both codecs write the same stream.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
from scipy.special import erf

from . import bf16, rans, stream
from .plan import ESC, PREC_BITS, Plan

Q_LIMIT = 2147483520.0  # 2^31 - 128, the largest float32 below 2^31


class NonFinite(ValueError):
    pass


@dataclass
class Shape:
    n_layers: int
    n_kv_heads: int
    head_dim: int
    keep_head: int
    keep_tail: int
    rope_theta: float

    @property
    def D(self) -> int:
        return self.n_layers * 2 * self.n_kv_heads * self.head_dim


def shape_of(params: dict) -> Shape:
    return Shape(params["n_layers"], params["n_kv_heads"], params["head_dim"], params["keep_head"],
                 params["keep_tail"], params["rope_theta"])


def split_positions(T: int, keep_head: int, keep_tail: int):
    """(N, kept positions, coded positions)."""
    N = max(T - keep_head - keep_tail, 0)
    t = np.arange(T)
    coded = t[keep_head:keep_head + N] if N > 0 else t[:0]
    kept = np.setdiff1d(t, coded)
    return N, kept, coded


@dataclass
class Encoded:
    data: bytes
    N: int
    y: np.ndarray          # float64 [N][C] analysis coefficients
    m: np.ndarray          # float64 [N][C] embedding mean
    yhat: np.ndarray       # float64 [N][C] reconstructed coefficients
    q: np.ndarray          # int64 [N][C] codes (0 for dropped)
    sym: np.ndarray        # uint8 [N][C_a] (255 at escapes)
    esc_flat: np.ndarray
    esc_q: np.ndarray
    groups: list = field(repr=False, default_factory=list)
    modelled_bits: float = 0.0

    @property
    def total_bytes(self) -> int:
        return len(self.data)


def embedding_mean(params: dict, tok_coded: np.ndarray) -> np.ndarray:
    """H E[tok] for each coded row (float64)."""
    E = bf16.to_f64(params["embedding"][np.asarray(tok_coded, dtype=np.int64)])
    H = bf16.to_f64(params["mean_head"])
    return E @ H.T


def _neighbour_sum(yhat: np.ndarray, js: np.ndarray) -> np.ndarray:
    N = yhat.shape[0]
    nb = yhat[js - 1].copy()
    right = js + 1 < N
    nb[right] += yhat[js[right] + 1]
    return nb


def _decide(d64: np.ndarray, step32: np.ndarray) -> np.ndarray:
    """Quantisation decision in float32: q = rint(fp32(d) / step)."""
    with np.errstate(over="ignore", invalid="ignore"):
        d32 = d64.astype(np.float32)
        r32 = (d32 / step32[None, :]).astype(np.float32)
        q = np.rint(r32)
    q = np.clip(q, -Q_LIMIT, Q_LIMIT)
    return q.astype(np.int64)


def quantize(y: np.ndarray, m: np.ndarray, p: Plan, a: np.ndarray):
    """Two-pass checkerboard quantisation.  Returns (q, yhat)."""
    N, C = y.shape
    step = p.step.astype(np.float64)
    act = p.active
    q = np.zeros((N, C), dtype=np.int64)
    yhat = np.zeros((N, C), dtype=np.float64)
    a64 = np.asarray(a, dtype=np.float32).astype(np.float64)
    for parity in (0, 1):
        js = np.arange(parity, N, 2)
        if js.size == 0:
            continue
        mu = m[js]
        if parity == 1:
            mu = mu + a64[None, :] * _neighbour_sum(yhat, js)
        d = y[js][:, act] - mu[:, act]
        if not np.all(np.isfinite(d)):
            raise NonFinite("non-finite coefficient residual")
        qa = _decide(d, p.step[act])
        qj = np.zeros((js.size, C), dtype=np.int64)
        qj[:, act] = qa
        q[js] = qj
        yhat[js] = mu + qj * step[None, :]
    return q, yhat


def dequantize(q: np.ndarray, m: np.ndarray, p: Plan, a: np.ndarray) -> np.ndarray:
    """Two decode passes: even rows from the embedding mean, odd rows add neighbours."""
    N, C = q.shape
    step = p.step.astype(np.float64)
    a64 = np.asarray(a, dtype=np.float32).astype(np.float64)
    yhat = np.zeros((N, C), dtype=np.float64)
    for parity in (0, 1):
        js = np.arange(parity, N, 2)
        if js.size == 0:
            continue
        mu = m[js]
        if parity == 1:
            mu = mu + a64[None, :] * _neighbour_sum(yhat, js)
        yhat[js] = mu + q[js] * step[None, :]
    return yhat


def symbols(q: np.ndarray, p: Plan):
    """Code -> symbol slot (q + 127), 255 for escapes; escape records in flat order."""
    qa = np.ascontiguousarray(q[:, p.act_idx])
    esc = np.abs(qa) > 127
    sym = np.ascontiguousarray(np.where(esc, ESC, qa + 127), dtype=np.uint8)
    jj, rr = np.nonzero(esc)
    flat = jj * p.c_active + rr
    return sym, flat.astype(np.int64), qa[jj, rr].astype(np.int64)


def modelled_bits(sym: np.ndarray, p: Plan, n_esc: int) -> float:
    """Code length the tables assign: sum of (15 - log2 f) plus 64 bits per escape."""
    if sym.size == 0:
        return 64.0 * n_esc
    ok = sym != ESC
    r = np.broadcast_to(np.arange(sym.shape[1])[None, :], sym.shape)
    f = p.freq[r[ok], sym[ok].astype(np.int64)]
    return float(np.sum(PREC_BITS - np.log2(f.astype(np.float64))) + 64.0 * n_esc)


def encode(rows: np.ndarray, tok: np.ndarray, params: dict, p: Plan) -> Encoded:
    sh = shape_of(params)
    T, D = rows.shape
    assert D == sh.D
    N, kept_t, coded_t = split_positions(T, sh.keep_head, sh.keep_tail)
    C = params["analysis"].shape[0]
    if N > 0:
        X = bf16.to_f64(rows[coded_t])
        A = bf16.to_f64(params["analysis"])
        y = X @ A.T
        m = embedding_mean(params, tok[coded_t])
        q, yhat = quantize(y, m, p, params["nbr_weight"])
    else:
        y = m = yhat = np.zeros((0, C))
        q = np.zeros((0, C), dtype=np.int64)
    sym, flat, qe = symbols(q, p)
    groups = rans.encode_all(sym, p.freq, p.cum) if N > 0 and p.c_active > 0 else []
    n_blk, G, _, _ = rans.group_shape(N, p.c_active)
    assert len(groups) == n_blk * G
    h = stream.Header(T=T, keep_head=sh.keep_head, keep_tail=sh.keep_tail, N=N, n_coef=C,
                      c_active=p.c_active, n_groups=n_blk * G, n_esc=len(flat),
                      step_scale=float(p.step_scale), plan_crc=p.crc, total_bytes=0, rans_bytes=0)
    data = stream.write(h, rows[kept_t], groups, flat, qe)
    return Encoded(data=data, N=N, y=y, m=m, yhat=yhat, q=q, sym=sym, esc_flat=flat, esc_q=qe,
                   groups=groups, modelled_bits=modelled_bits(sym, p, len(flat)))


def gelu(u: np.ndarray) -> np.ndarray:
    """Exact (erf) GELU: 0.5 u (1 + erf(u / sqrt 2))."""
    return 0.5 * u * (1.0 + erf(u / np.sqrt(2.0)))


def rope(x: np.ndarray, t: np.ndarray, sh: Shape) -> np.ndarray:
    """Rotate-half RoPE on the key columns of rows x (float64) at positions t."""
    out = x.copy()
    half = sh.head_dim // 2
    w = np.power(float(sh.rope_theta), -np.arange(half, dtype=np.float64) / half)
    ang = np.asarray(t, dtype=np.float64)[:, None] * w[None, :]
    c, s = np.cos(ang), np.sin(ang)
    for l in range(sh.n_layers):
        for h in range(sh.n_kv_heads):
            base = (l * 2 * sh.n_kv_heads + h) * sh.head_dim
            lo = x[:, base:base + half]
            hi = x[:, base + half:base + sh.head_dim]
            out[:, base:base + half] = lo * c - hi * s
            out[:, base + half:base + sh.head_dim] = hi * c + lo * s
    return out


def unrope(x: np.ndarray, t: np.ndarray, sh: Shape) -> np.ndarray:
    """The inverse of rope(): the key columns rotated back by the angles of
    positions t (float64).  Encoding a post-RoPE cache takes its rows through
    this first (first paragraph of "How it works": keys are coded before
    RoPE)."""
    return rope(x, -np.asarray(t, dtype=np.float64), sh)


@dataclass
class Decoded:
    rows: np.ndarray     # uint16 bf16 [T][D]
    sym: np.ndarray      # uint8 [N][C_a]
    q: np.ndarray        # int64 [N][C]
    yhat: np.ndarray     # float64 [N][C]
    yhat_b: np.ndarray   # uint16 bf16 [N][C]
    h_b: np.ndarray      # uint16 bf16 [N][hidden]
    xhat: np.ndarray     # float64 [N][D] before RoPE


def check_header(h: stream.Header, T: int, params: dict, p: Plan):
    sh = shape_of(params)
    N = max(T - sh.keep_head - sh.keep_tail, 0)
    C = params["analysis"].shape[0]
    n_blk, G, _, _ = rans.group_shape(N, p.c_active)
    if h.plan_crc != p.crc or h.c_active != p.c_active or h.n_coef != C:
        raise stream.PlanMismatch("stream was written under another plan")
    if (h.T != T or h.N != N or h.keep_head != sh.keep_head or h.keep_tail != sh.keep_tail
            or h.n_groups != n_blk * G):
        raise stream.StreamError("header does not match the request")


def decode(data: bytes, tok: np.ndarray, params: dict, p: Plan) -> Decoded:
    sh = shape_of(params)
    D = sh.D
    h, kept, flat, qe, groups = stream.parse(data, D)
    T = int(len(tok))
    check_header(h, T, params, p)
    N = h.N
    C = params["analysis"].shape[0]
    _, kept_t, coded_t = split_positions(T, sh.keep_head, sh.keep_tail)
    esc = np.zeros((N, p.c_active), dtype=bool)
    if len(flat):
        esc.reshape(-1)[flat] = True
    sym = rans.decode_all(groups, p.freq, p.cum, N, esc) if N > 0 and p.c_active > 0 else \
        np.full((N, p.c_active), ESC, np.uint8)
    qa = np.ascontiguousarray(sym, dtype=np.int64) - 127
    if len(flat):
        qa.reshape(-1)[flat] = qe
    q = np.zeros((N, C), dtype=np.int64)
    q[:, p.act_idx] = qa
    out = np.zeros((T, D), dtype=np.uint16)
    linear = params.get("w1") is None
    hid = 0 if linear else params["w1"].shape[0]
    if N > 0:
        m = embedding_mean(params, tok[coded_t])
        yhat = dequantize(q, m, p, params["nbr_weight"])
        yb_bits = bf16.from_f64(yhat)
        yb = bf16.to_f64(yb_bits)
        S = bf16.to_f64(params["synthesis"])
        xhat = yb @ S.T
        if linear:
            hb_bits = np.zeros((N, 0), np.uint16)
        else:
            W1 = bf16.to_f64(params["w1"])
            hb_bits = bf16.from_f64(gelu(yb @ W1.T))
            W2 = bf16.to_f64(params["w2"])
            xhat = xhat + bf16.to_f64(hb_bits) @ W2.T
        out[coded_t] = bf16.from_f64(rope(xhat, coded_t, sh))
    else:
        yhat = np.zeros((0, C))
        yb_bits = np.zeros((0, C), np.uint16)
        hb_bits = np.zeros((0, hid), np.uint16)
        xhat = np.zeros((0, D))
    if len(kept_t):
        out[kept_t] = bf16.from_f64(rope(bf16.to_f64(kept), kept_t, sh))
    return Decoded(rows=out, sym=sym, q=q, yhat=yhat, yhat_b=yb_bits, h_b=hb_bits, xhat=xhat)
