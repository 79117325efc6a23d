"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test ties one part of the oracle to something other than itself: a
number printed on the DCKV digest page, a closed form, an invariant, a library
routine the step reduces to, or brute force on tiny inputs.
"""
from __future__ import annotations

import json
import os
import struct
import zlib
from fractions import Fraction
import itertools

import numpy as np
import pytest
from scipy.stats import laplace

from oracle import bf16, codec, plan as P, rans, stream
from tests.tiny import tiny_params, tiny_rows

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")))


# ----------------------------------------------------------------------------
# sizes fixed by the pages
# ----------------------------------------------------------------------------
def test_sizes_from_pages():
    layers, kv, heads, hd = GOLD["full_attention_layers"]["value"], 2, 2, 256
    row = layers * kv * heads * hd
    assert row == GOLD["row_dim"]["value"]
    assert row * 2 == GOLD["kv_bytes_per_token_bf16"]["value"]
    assert 4096 * 12288 == GOLD["kv_bytes_4k_tokens_MiB"]["value"] * 2 ** 20
    assert 131072 * 12288 == GOLD["kv_bytes_128k_tokens_GiB"]["value"] * 2 ** 30
    kept = (GOLD["keep_head"]["value"] + GOLD["keep_tail"]["value"]) * 12288
    assert kept == 1622016
    assert round(kept / 2 ** 20, 2) == GOLD["kept_MiB"]["value"]
    # the linear codec (analysis + synthesis, fp32) is exactly 96 MiB
    assert 2 * 6144 * 2048 * 4 == GOLD["linear_codec_MiB_fp32"]["value"] * 2 ** 20


def test_kept_rows_verbatim_and_positions():
    prm = tiny_params(seed=3)
    pl = P.make_plan(np.float32(0.3), prm["base_step"], prm["laplace_scale"])
    for T in (0, 1, 2, 3, 4, 5, 9, 40):
        rows, tok = tiny_rows(prm, T, seed=T)
        enc = codec.encode(rows, tok, prm, pl)
        h, kept, *_ = stream.parse(enc.data, rows.shape[1])
        N = max(T - 3, 0)
        assert h.N == N and enc.N == N
        keep_t = [t for t in range(T) if t < 1 or t >= T - 2] if T > 3 else list(range(T))
        assert np.array_equal(kept, rows[keep_t])
        dec = codec.decode(enc.data, tok, prm, pl)
        # V columns of kept rows are bit-identical, and so is every column at t = 0
        D = rows.shape[1]
        vcols = np.arange(D // 2, D)
        assert np.array_equal(dec.rows[keep_t][:, vcols], rows[keep_t][:, vcols])
        if T:
            assert np.array_equal(dec.rows[0], rows[0])


# ----------------------------------------------------------------------------
# bf16 rounding: exact rational nearest-even
# ----------------------------------------------------------------------------
def _bf16_exact(x: float) -> int:
    if x == 0:
        return 0x8000 if np.signbit(x) else 0
    fx = Fraction(x)
    best = None
    # candidates: neighbours of the float32 truncation
    f32 = np.float32(x)
    bits = int(np.array(f32).view(np.uint32)) >> 16
    for b in range(max(bits - 2, 0), bits + 3):
        for sgn in (0, 0x8000):
            bb = (b & 0x7FFF) | sgn
            if (bb & 0x7F80) == 0x7F80:
                continue
            v = Fraction(float(np.array(bb << 16, dtype=np.uint32).view(np.float32)))
            d = abs(v - fx)
            key = (d, bb & 1)
            if best is None or key < best[0]:
                best = (key, bb)
    return best[1]


def test_bf16_round_nearest_even_exact():
    rng = np.random.default_rng(5)
    xs = list(rng.standard_normal(3000) * 10.0 ** rng.integers(-30, 30, 3000))
    # exact ties and near-ties between bf16 neighbours, including double-rounding traps
    for b in rng.integers(0x0080, 0x7F00, 400):
        lo = float(np.array(int(b) << 16, dtype=np.uint32).view(np.float32))
        hi = float(np.array((int(b) + 1) << 16, dtype=np.uint32).view(np.float32))
        mid = (lo + hi) / 2
        xs += [mid, np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf), -mid,
               mid + (hi - lo) * 2.0 ** -30, mid - (hi - lo) * 2.0 ** -30]
    got = bf16.from_f64(np.array(xs))
    want = np.array([_bf16_exact(float(x)) for x in xs], dtype=np.uint16)
    assert np.array_equal(got, want)
    # round trip of every finite bf16 value is exact
    allb = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    fin = (allb & 0x7F80) != 0x7F80
    assert np.array_equal(bf16.from_f64(bf16.to_f64(allb[fin])), allb[fin])


# ----------------------------------------------------------------------------
# tables
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("s", [0.05, 0.0501, 0.1, 0.37, 1.0, 3.3, 17.0, 250.0, 5000.0])
def test_table_invariants_and_laplace_cdf(s):
    f, cum, pn = P.laplace_tables(np.array([s]))
    f, cum, pn = f[0], cum[0], pn[0]
    assert f.sum() == P.M and f.min() >= 1 and cum[-1] == P.M and cum[0] == 0
    assert np.array_equal(f, f[::-1])                       # symmetric
    assert np.all(np.diff(f[127:]) <= 0)                    # non-increasing in |k|
    # float part is the Laplace(0, s) mass of [k-1/2, k+1/2], renormalised to +-127
    k = np.arange(-127, 128)
    mass = laplace.cdf(k + 0.5, scale=s) - laplace.cdf(k - 0.5, scale=s)
    np.testing.assert_allclose(pn, mass / mass.sum(), rtol=1e-9, atol=1e-15)


def test_drop_rule_threshold():
    base = np.ones(4, np.float32)
    g = np.float32(0.5)
    b = np.array([0.025, np.nextafter(np.float32(0.025), np.float32(0)), 0.03, 0.0], np.float32)
    pl = P.make_plan(g, base, b)
    # s = b / step; 0.025 / 0.5 = 0.05 is kept (drop only strictly below 0.05 steps)
    assert list(pl.active) == [True, False, True, False]
    assert list(pl.act_idx) == [0, 2] and list(pl.rank) == [0, -1, 1, -1]


def _crc32_bitwise(data: bytes) -> int:
    crc = 0xFFFFFFFF
    for byte in data:
        crc ^= byte
        for _ in range(8):
            crc = (crc >> 1) ^ (0xEDB88320 if crc & 1 else 0)
    return crc ^ 0xFFFFFFFF


def test_plan_crc_layout():
    base = np.ones(5, np.float32)
    b = np.array([0.3, 0.001, 0.2, 0.9, 0.05], np.float32)
    pl = P.make_plan(np.float32(0.25), base, b)
    blob = b"".join(struct.pack("<f", float(v)) for v in pl.step)
    blob += bytes(int(a) for a in pl.active)
    blob += b"".join(struct.pack("<H", int(v)) for v in pl.freq.reshape(-1))
    assert pl.crc == _crc32_bitwise(blob)
    assert _crc32_bitwise(b"123456789") == 0xCBF43926  # CRC-32 check value


def test_steps_are_fp32_products():
    g = np.float32(0.1007872)
    d = np.array([1.0, 0.3, 7.7, 1e-3], np.float32)
    st = P.steps(g, d)
    for gi, di, si in zip([g] * 4, d, st):
        exact = Fraction(float(gi)) * Fraction(float(di))
        # the float32 nearest to the exact product
        cands = [np.float32(float(si)), np.nextafter(si, np.float32(np.inf)), np.nextafter(si, np.float32(0))]
        errs = [abs(Fraction(float(c)) - exact) for c in cands]
        assert errs[0] == min(errs)


# ----------------------------------------------------------------------------
# rANS
# ----------------------------------------------------------------------------
def _tables(scales):
    f, cum, _ = P.laplace_tables(np.asarray(scales, dtype=np.float64))
    return f, cum


def test_rans_exhaustive_tiny_groups():
    f, cum = _tables([0.05, 0.9, 40.0])
    alphabet = [0, 1, 126, 127, 128, 253, 254]
    count = 0
    for Lb in (1, 2):
        for n in (1, 2, 3):
            for combo in itertools.product(alphabet, repeat=Lb * n):
                sym = np.array(combo).reshape(Lb, n)
                w = rans.encode_group(sym, f[:n], cum[:n])
                assert len(w) >= 2 * n
                back = rans.decode_group(w, f[:n], cum[:n], Lb)
                assert np.array_equal(np.array(back), sym)
                count += 1
    assert count > 500


def test_rans_extreme_tables_and_end_state():
    # f_0 = 2^15 - 254 (all other symbols have frequency 1) and a flat-ish table
    f, cum = _tables([1e-4, 1e4])
    assert f[0][127] == P.M - 254
    rng = np.random.default_rng(0)
    for trial in range(30):
        Lb = int(rng.integers(1, 40))
        sym = rng.integers(0, 255, size=(Lb, 2))
        if trial % 3 == 0:
            sym[:, 0] = 127
        w = rans.encode_group(sym, f, cum)
        assert np.array_equal(np.array(rans.decode_group(w, f, cum, Lb)), sym)
        # end state: re-running the decoder's state machine ends at L with all words used
        with pytest.raises(rans.CorruptStream):
            rans.decode_group(w + [0], f, cum, Lb)
        if len(w) > 4:
            bad = list(w)
            bad[-1] ^= 0x5A5A
            try:
                out = rans.decode_group(bad, f, cum, Lb)
                assert not np.array_equal(np.array(out), sym)
            except rans.CorruptStream:
                pass


def test_rans_escape_mask_skips_positions():
    f, cum = _tables([0.3, 0.7, 2.0, 9.0])
    rng = np.random.default_rng(7)
    sym = rng.integers(100, 155, size=(20, 4))
    mask = rng.random((20, 4)) < 0.3
    s2 = np.where(mask, 255, sym)
    w = rans.encode_group(s2, f, cum)
    back = np.array(rans.decode_group(w, f, cum, 20, esc_mask=mask))
    assert np.array_equal(back, s2)


def test_rans_lockstep_equals_scalar_and_roundtrips():
    rng = np.random.default_rng(11)
    for N, Ca in [(1, 1), (3, 70), (257, 5), (300, 130), (511, 64)]:
        scales = rng.uniform(0.05, 30.0, Ca)
        f, cum = _tables(scales)
        sym = np.clip(np.rint(rng.laplace(127, 3, (N, Ca))), 0, 254).astype(np.uint8)
        esc = rng.random((N, Ca)) < 0.01
        sym[esc] = 255
        groups = rans.encode_all(sym, f, cum)
        n_blk, G, Lb, nl = rans.group_shape(N, Ca)
        assert len(groups) == n_blk * G
        for gid in range(0, len(groups), max(1, len(groups) // 7)):
            b, g = divmod(gid, G)
            blk = sym[256 * b:256 * b + Lb[b], 64 * g:64 * g + nl[g]]
            assert list(groups[gid]) == rans.encode_group(blk, f[64 * g:64 * g + nl[g]],
                                                          cum[64 * g:64 * g + nl[g]])
        back = rans.decode_all(groups, f, cum, N, esc)
        assert np.array_equal(back, sym)


def test_rans_stored_close_to_modelled():
    """Per group: -16*lanes <= stored bits - modelled bits <= 32*lanes + 1% of modelled."""
    rng = np.random.default_rng(3)
    scales = rng.uniform(0.1, 8.0, 64)
    f, cum = _tables(scales)
    pmf = f / P.M
    N = 256
    sym = np.empty((N, 64), np.uint8)
    for c in range(64):
        sym[:, c] = rng.choice(255, size=N, p=pmf[c])
    (w,) = rans.encode_all(sym, f, cum)
    modelled = sum((15 - np.log2(f[c, sym[:, c]])).sum() for c in range(64))
    stored = 16 * len(w)
    assert -16 * 64 <= stored - modelled <= 32 * 64 + 0.01 * modelled


# ----------------------------------------------------------------------------
# quantiser, escapes, checkerboard
# ----------------------------------------------------------------------------
def test_quantizer_brute_force_nearest_lattice():
    rng = np.random.default_rng(2)
    y = rng.laplace(0, 10, (64, 5))
    m = rng.normal(0, 1, (64, 5))
    base = np.ones(5, np.float32)
    pl = P.make_plan(np.float32(0.07), base, np.full(5, 1.0, np.float32))
    q, yhat = codec.quantize(y, m, pl, np.zeros(5, np.float32))   # a = 0: every row is "even"
    step = pl.step.astype(np.float64)
    ks = np.arange(-4000, 4001)
    for j in range(64):
        for c in range(5):
            d = y[j, c] - m[j, c]
            best = ks[np.argmin(np.abs(d - ks * step[c]))]
            frac = abs(d / step[c] - np.floor(d / step[c]) - 0.5)
            if frac > 1e-5:  # away from a tie the lattice point is unique
                assert q[j, c] == best
            assert yhat[j, c] == m[j, c] + q[j, c] * step[c]


def test_escape_cost_is_64_bits_per_code():
    prm = tiny_params(seed=4, n_coef=8)
    pl = P.make_plan(np.float32(0.5), prm["base_step"], prm["laplace_scale"])
    rows, tok = tiny_rows(prm, 40, seed=9, scale=0.2)
    enc = codec.encode(rows, tok, prm, pl)
    base_bytes = enc.total_bytes
    assert len(enc.esc_flat) == 0
    # push one code from 127 to 128: exactly 8 more escape bytes, one fewer rANS symbol
    q = enc.q.copy()
    j, c = 6, int(pl.act_idx[2])
    sizes = {}
    for v in (127, 128, -128, 2 ** 31 - 128, -(2 ** 31 - 128)):
        q[j, c] = v
        sym, flat, qe = codec.symbols(q, pl)
        groups = rans.encode_all(sym, pl.freq, pl.cum)
        words = sum(len(g) for g in groups)
        sizes[v] = (len(flat), words)
        # decode of the escape recovers the code exactly
        esc = np.zeros(sym.shape, bool)
        esc.reshape(-1)[flat] = True
        back = rans.decode_all(groups, pl.freq, pl.cum, sym.shape[0], esc)
        qa = back.astype(np.int64) - 127
        qa.reshape(-1)[flat] = qe
        assert qa[j, pl.rank[c]] == v
    assert sizes[127][0] == 0 and sizes[128][0] == 1 and sizes[-128][0] == 1
    bits_127 = 15 - np.log2(pl.freq[pl.rank[c], 254])
    # the rANS part shrinks by about that symbol's code length (within flush granularity)
    assert abs((sizes[127][1] - sizes[128][1]) * 16 - bits_127) <= 16 + 1e-9
    assert base_bytes > 0


def test_checkerboard_locality_and_two_passes():
    prm = tiny_params(seed=6, n_coef=8)
    pl = P.make_plan(np.float32(0.2), prm["base_step"], prm["laplace_scale"])
    rows, tok = tiny_rows(prm, 30, seed=10)
    enc = codec.encode(rows, tok, prm, pl)
    N = enc.N
    a = prm["nbr_weight"]
    y0 = codec.dequantize(enc.q, enc.m, pl, a)
    assert np.array_equal(y0, enc.yhat)
    # perturbing an odd code leaves every even yhat bit-identical and touches only that row
    q1 = enc.q.copy()
    q1[5, pl.act_idx[0]] += 3
    y1 = codec.dequantize(q1, enc.m, pl, a)
    assert np.array_equal(y1[0::2], y0[0::2])
    diff_rows = np.nonzero(np.any(y1 != y0, axis=1))[0]
    assert list(diff_rows) == [5]
    # perturbing the even code at j changes yhat only at j-1, j, j+1
    for j in (0, 8, N - 1 if (N - 1) % 2 == 0 else N - 2):
        q2 = enc.q.copy()
        q2[j, pl.act_idx[1]] -= 2
        y2 = codec.dequantize(q2, enc.m, pl, a)
        rows_changed = set(np.nonzero(np.any(y2 != y0, axis=1))[0].tolist())
        assert j in rows_changed and rows_changed <= {j - 1, j, j + 1}
    # the odd mean uses yhat_N = 0 at the right edge: closed form for the last row
    if (N - 1) % 2 == 1:
        c = 0
        step = float(pl.step[c])
        want = enc.m[N - 1, c] + float(a[c]) * y0[N - 2, c] + enc.q[N - 1, c] * step
        assert y0[N - 1, c] == want


def test_embedding_mean_is_gathered_matmul():
    prm = tiny_params(seed=8, emb_dim=4, n_coef=8)
    tok = np.array([3, 0, 15, 3], np.int32)
    E = bf16.to_f64(prm["embedding"])
    H = bf16.to_f64(prm["mean_head"])
    m = codec.embedding_mean(prm, tok)
    for r, t in enumerate(tok):
        for c in range(8):
            assert m[r, c] == pytest.approx(sum(H[c, k] * E[t, k] for k in range(4)), rel=1e-14, abs=1e-15)


# ----------------------------------------------------------------------------
# decode-side float stages
# ----------------------------------------------------------------------------
def test_gelu_matches_torch_exact_gelu():
    import torch
    u = np.linspace(-8, 8, 2001)
    ref = torch.nn.functional.gelu(torch.from_numpy(u), approximate="none").numpy()
    np.testing.assert_allclose(codec.gelu(u), ref, rtol=1e-12, atol=1e-15)


def test_rope_closed_forms():
    sh = codec.Shape(n_layers=2, n_kv_heads=2, head_dim=8, keep_head=0, keep_tail=0, rope_theta=1e7)
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, sh.D))
    # t = 0 is the identity; V columns never move
    assert np.array_equal(codec.rope(x, np.zeros(5), sh), x)
    t1, t2 = np.array([3.0, 17.0, 131071.0, 5.0, 1.0]), np.array([1.0, 4.0, 2.0, 65536.0, 0.0])
    r1 = codec.rope(x, t1, sh)
    # composition R(t1) R(t2) = R(t1 + t2)
    np.testing.assert_allclose(codec.rope(r1, t2, sh), codec.rope(x, t1 + t2, sh), atol=1e-9)
    # complex form (x_i + i x_{i+half}) e^{i t w_i} on every key head
    half = sh.head_dim // 2
    w = 1e7 ** (-np.arange(half) / half)
    for l in range(2):
        for h in range(2):
            base = (l * 4 + h) * sh.head_dim
            z = x[:, base:base + half] + 1j * x[:, base + half:base + 2 * half]
            zr = z * np.exp(1j * t1[:, None] * w[None, :])
            np.testing.assert_allclose(r1[:, base:base + half], zr.real, atol=1e-12)
            np.testing.assert_allclose(r1[:, base + half:base + 2 * half], zr.imag, atol=1e-12)
            vb = (l * 4 + 2 + h) * sh.head_dim
            assert np.array_equal(r1[:, vb:vb + sh.head_dim], x[:, vb:vb + sh.head_dim])
    # per-pair norm preserved
    for l in range(2):
        for h in range(2):
            base = (l * 4 + h) * sh.head_dim
            n0 = x[:, base:base + half] ** 2 + x[:, base + half:base + 2 * half] ** 2
            n1 = r1[:, base:base + half] ** 2 + r1[:, base + half:base + 2 * half] ** 2
            np.testing.assert_allclose(n0, n1, rtol=1e-12)


def test_unrope_inverts_rope_and_leaves_values():
    prm = tiny_params(seed=14, n_layers=2, n_kv_heads=2, head_dim=8)
    sh = codec.shape_of(prm)
    rng = np.random.default_rng(5)
    x = rng.normal(0, 1, (9, sh.D))
    t = np.arange(100, 109)
    np.testing.assert_allclose(codec.unrope(codec.rope(x, t, sh), t, sh), x, rtol=0, atol=1e-12)
    np.testing.assert_allclose(codec.rope(codec.unrope(x, t, sh), t, sh), x, rtol=0, atol=1e-12)
    u = codec.unrope(x, t, sh)
    # value columns are untouched; the rotation keeps each key pair's norm
    for l in range(2):
        vb = (l * 2 + 1) * 2 * 8
        np.testing.assert_array_equal(u[:, vb:vb + 16], x[:, vb:vb + 16])
        kb = l * 2 * 2 * 8
        pairs = lambda a: a[:, kb:kb + 4] ** 2 + a[:, kb + 4:kb + 8] ** 2
        np.testing.assert_allclose(pairs(u), pairs(x), rtol=1e-12)


def test_matmul_orientation_against_triple_loop():
    prm = tiny_params(seed=12, n_coef=4, head_dim=2, n_layers=1, n_kv_heads=1)
    X = np.random.default_rng(0).standard_normal((3, 4))
    A = bf16.to_f64(prm["analysis"])
    y = X @ A.T
    for j in range(3):
        for c in range(4):
            assert y[j, c] == pytest.approx(sum(A[c, k] * X[j, k] for k in range(4)), rel=1e-13)


def test_end_to_end_closed_form_error_bound():
    """x in span(S), W2 = 0, no drops, no escapes: |xhat - x| <= sqrt(sum (step/2)^2) + bf16 slack."""
    prm = tiny_params(seed=13, n_coef=16, head_dim=8, n_layers=1, n_kv_heads=1, w2_zero=True,
                      keep_head=0, keep_tail=0)
    D = 16
    pl = P.make_plan(np.float32(0.05), prm["base_step"], np.full(16, 1.0, np.float32))
    assert pl.c_active == 16
    S = bf16.to_f64(prm["synthesis"])
    rng = np.random.default_rng(2)
    coef = rng.normal(0, 0.5, (40, 16))
    rows = bf16.from_f64(coef @ S.T)
    tok = rng.integers(0, 16, 40).astype(np.int32)
    enc = codec.encode(rows, tok, prm, pl)
    assert len(enc.esc_flat) == 0
    dec = codec.decode(enc.data, tok, prm, pl)
    x = bf16.to_f64(rows)
    bound = np.sqrt(np.sum((pl.step.astype(np.float64) / 2) ** 2))
    err = np.linalg.norm(dec.xhat - x, axis=1)
    slack = 0.02 * np.linalg.norm(x, axis=1) + 0.01  # bf16 basis and bf16 yhat
    assert np.all(err <= bound + slack)


def test_linear_codec_drops_exactly_the_correction():
    """The linear codec (no w1 / w2) writes the same stream and decodes to the
    DCKV reconstruction minus W2 h_b: the pre-RoPE difference equals W2 h_b
    computed here from the DCKV decode's own h_b."""
    prm = tiny_params(seed=21, n_coef=8, head_dim=8, n_layers=1, n_kv_heads=1, keep_head=1, keep_tail=2)
    lin = {k: v for k, v in prm.items() if k not in ("w1", "w2")}
    pl = P.make_plan(np.float32(0.3), prm["base_step"], prm["laplace_scale"])
    rows, tok = tiny_rows(prm, 30, seed=4)
    enc = codec.encode(rows, tok, prm, pl)
    assert codec.encode(rows, tok, lin, pl).data == enc.data
    full = codec.decode(enc.data, tok, prm, pl)
    part = codec.decode(enc.data, tok, lin, pl)
    assert np.array_equal(part.yhat_b, full.yhat_b)
    assert part.h_b.shape[1] == 0
    corr = bf16.to_f64(full.h_b) @ bf16.to_f64(prm["w2"]).T
    assert np.max(np.abs(corr)) > 1e-3  # the correction is not trivially zero here
    np.testing.assert_allclose(full.xhat - part.xhat, corr, rtol=1e-12, atol=1e-12)
    # kept rows do not depend on the codec
    _, kept_t, _ = codec.split_positions(30, 1, 2)
    assert np.array_equal(full.rows[kept_t], part.rows[kept_t])


# ----------------------------------------------------------------------------
# stream validation
# ----------------------------------------------------------------------------
def test_stream_errors_detected():
    prm = tiny_params(seed=14, n_coef=8)
    pl = P.make_plan(np.float32(0.3), prm["base_step"], prm["laplace_scale"])
    rows, tok = tiny_rows(prm, 50, seed=3)
    enc = codec.encode(rows, tok, prm, pl)
    data = bytearray(enc.data)
    with pytest.raises(stream.StreamError):
        codec.decode(bytes(data[:-2]), tok, prm, pl)
    bad = bytearray(data)
    bad[0] = ord("X")
    with pytest.raises(stream.StreamError):
        codec.decode(bytes(bad), tok, prm, pl)
    other = P.make_plan(np.float32(0.31), prm["base_step"], prm["laplace_scale"])
    with pytest.raises(stream.PlanMismatch):
        codec.decode(enc.data, tok, prm, other)
    with pytest.raises(stream.StreamError):
        codec.decode(enc.data, tok[:-1], prm, pl)
    # flip bits inside the rANS section: either detected, or the symbols differ
    h = stream.header(enc.data)
    rans_start = h.total_bytes - h.rans_bytes
    hits = 0
    for k in range(20):
        b2 = bytearray(data)
        b2[rans_start + (k * 7) % h.rans_bytes] ^= 0x10
        try:
            d2 = codec.decode(bytes(b2), tok, prm, pl)
            assert not np.array_equal(d2.sym, enc.sym)
        except rans.CorruptStream:
            hits += 1
    assert hits > 10


def test_drop_path_and_degenerate_plans():
    prm = tiny_params(seed=15, n_coef=8)
    b = prm["laplace_scale"].copy()
    b[[1, 4, 6]] = 0.001
    prm["laplace_scale"] = b
    pl = P.make_plan(np.float32(0.5), prm["base_step"], b)
    assert pl.c_active == 5
    rows, tok = tiny_rows(prm, 33, seed=4)
    enc = codec.encode(rows, tok, prm, pl)
    dec = codec.decode(enc.data, tok, prm, pl)
    assert np.all(enc.q[:, [1, 4, 6]] == 0)
    assert np.array_equal(dec.yhat, enc.yhat)
    # dropped components decode to their conditional mean exactly
    a = prm["nbr_weight"].astype(np.float64)
    for c in (1, 4, 6):
        mu = enc.m[:, c].copy()
        ev = dec.yhat[0::2, c]
        assert np.array_equal(ev, mu[0::2])
        for j in range(1, enc.N, 2):
            nb = dec.yhat[j - 1, c] + (dec.yhat[j + 1, c] if j + 1 < enc.N else 0.0)
            assert dec.yhat[j, c] == mu[j] + a[c] * nb
    # every component dropped: no groups, the stream still round-trips the kept rows
    pl0 = P.make_plan(np.float32(1e4), prm["base_step"], b)
    assert pl0.c_active == 0
    enc0 = codec.encode(rows, tok, prm, pl0)
    assert stream.header(enc0.data).n_groups == 0
    dec0 = codec.decode(enc0.data, tok, prm, pl0)
    assert dec0.rows.shape == rows.shape
    # C_a not a multiple of 64 with many components
    prm2 = tiny_params(seed=16, n_coef=100, head_dim=64)
    pl2 = P.make_plan(np.float32(0.3), prm2["base_step"], prm2["laplace_scale"])
    assert pl2.c_active == 100
    rows2, tok2 = tiny_rows(prm2, 300, seed=5)
    enc2 = codec.encode(rows2, tok2, prm2, pl2)
    dec2 = codec.decode(enc2.data, tok2, prm2, pl2)
    assert np.array_equal(dec2.sym, enc2.sym)


def test_nonfinite_input_rejected():
    prm = tiny_params(seed=17)
    pl = P.make_plan(np.float32(0.3), prm["base_step"], prm["laplace_scale"])
    rows, tok = tiny_rows(prm, 20, seed=6)
    rows[7, 3] = 0x7FC0
    with pytest.raises(codec.NonFinite):
        codec.encode(rows, tok, prm, pl)


def test_rans_word_order_closed_form():
    """One lane, one symbol: x = (L div f) M + (L mod f) + c, stored low word first."""
    f, cum = _tables([0.7])
    for s in (0, 100, 127, 200, 254):
        fs, cs = int(f[0, s]), int(cum[0, s])
        x = (65536 // fs) * 32768 + 65536 % fs + cs
        assert rans.encode_group([[s]], f, cum) == [x & 0xFFFF, x >> 16]
    # two lanes, one token: lane 0's flush words come first after reversal
    s0, s1 = 127, 130
    x0 = (65536 // int(f[0, s0])) * 32768 + 65536 % int(f[0, s0]) + int(cum[0, s0])
    f2, c2 = _tables([0.7, 0.7])
    assert rans.encode_group([[s0, s1]], f2, c2)[:2] == [x0 & 0xFFFF, x0 >> 16]


def test_stream_header_offsets():
    prm = tiny_params(seed=18, n_coef=8)
    pl = P.make_plan(np.float32(0.3), prm["base_step"], prm["laplace_scale"])
    rows, tok = tiny_rows(prm, 12, seed=2)
    enc = codec.encode(rows, tok, prm, pl)
    d = enc.data
    assert d[0:4] == b"DCKV"
    assert int.from_bytes(d[4:6], "little") == 1 and int.from_bytes(d[6:8], "little") == 64
    u32 = lambda o: int.from_bytes(d[o:o + 4], "little")
    assert [u32(8), u32(12), u32(16), u32(20), u32(24), u32(28)] == [12, 1, 2, 9, 8, pl.c_active]
    assert u32(32) == 1 and u32(36) == len(enc.esc_flat)          # one block x one group
    assert struct.unpack("<f", d[40:44])[0] == np.float32(0.3) and u32(44) == pl.crc
    assert int.from_bytes(d[48:56], "little") == len(d)
    D = rows.shape[1]
    kept_end = 64 + 3 * D * 2
    assert d[64:kept_end] == rows[[0, 10, 11]].astype("<u2").tobytes()
    assert u32(kept_end) == 0 and u32(kept_end + 4) == int.from_bytes(d[56:64], "little")
