"""Seeded synthetic inputs for the DCKV prompt-KV-cache codec.

This module is the only code shared by the CPU oracle (``oracle/``) and the HIP
path's callers (tests, ``bench.py``).  It draws random numbers and builds the
synthetic codec parameters; it contains none of the codec's encode or decode
arithmetic (no quantiser, no entropy tables, no rANS, no RoPE, no GELU).

What the pages fix (DCKV digest, trove.briskstack.com, "How it works"):
  * the stacked row is the pre-RoPE K and V of the 6 full-attention layers,
    6,144 values per token in bf16 (12,288 bytes);
  * the first 4 and the last 128 positions are kept in bf16;
  * the transform maps a row to 2,048 coefficients, and the correction has one
    hidden layer of 256 GELU units.
Everything else here is a seeded stand-in, because the language model, the
trained codec weights and the evaluation suites are not available:
  * rows x = U z + e, U a seeded orthonormal 6144x6144 basis,
    z_k ~ Laplace(0, 0.5 (k+1)^-0.7), e ~ N(0, 0.001^2);
  * the analysis/synthesis basis is the top-2048 (uncentred) PCA of a separate
    seeded calibration batch of 2,048 rows ("the basis starts from PCA");
  * W1, W2 ~ N(0, 0.01^2); embedding table and mean head ~ N(0, 0.02^2);
    neighbour weights a_c ~ U(0, 0.5); base steps delta_c = 1;
  * the per-component Laplace scale b_c is the maximum-likelihood fit (mean
    absolute residual) on the calibration batch, with the conditional mean
    taken open loop (unquantised neighbours).  This is parameter synthesis run
    once per codec, not part of encode or decode; both sides receive the same
    fitted vector as an input.
"N(0, s)" always means standard deviation s.
"""
from __future__ import annotations

import json
import os
from dataclasses import dataclass, field

import numpy as np

CODEC_SEED = 20261027

N_LAYERS = 6
N_KV_HEADS = 2
HEAD_DIM = 256
D = N_LAYERS * 2 * N_KV_HEADS * HEAD_DIM  # 6144
N_COEF = 2048
N_HIDDEN = 256
EMB_DIM = 2048
VOCAB = 32768
KEEP_HEAD = 4
KEEP_TAIL = 128
ROPE_THETA = 1.0e7
CALIB_ROWS = 2048
ROW_CHUNK = 4096

_HERE = os.path.dirname(os.path.abspath(__file__))
_CACHE_DIR = os.path.join(os.path.dirname(_HERE), ".dckv_cache")
_WORLD_VERSION = "world-v1"


# --------------------------------------------------------------------------
# bf16 helpers (input preparation only)
# --------------------------------------------------------------------------
def to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# codec world
# --------------------------------------------------------------------------
@dataclass
class World:
    """Synthetic codec parameters (bf16 matrices as uint16 bits, fp32 vectors)."""

    analysis: np.ndarray   # A  [N_COEF][D]      bf16 bits
    synthesis: np.ndarray  # S  [D][N_COEF]      bf16 bits
    w1: np.ndarray         # W1 [N_HIDDEN][N_COEF]
    w2: np.ndarray         # W2 [D][N_HIDDEN]
    embedding: np.ndarray  # E  [VOCAB][EMB_DIM]
    mean_head: np.ndarray  # H  [N_COEF][EMB_DIM]
    nbr_weight: np.ndarray     # a_c  fp32 [N_COEF]
    laplace_scale: np.ndarray  # b_c  fp32 [N_COEF]
    base_step: np.ndarray      # delta_c fp32 [N_COEF]
    U: np.ndarray = field(repr=False)  # float32 [D][D] orthonormal row basis

    def params(self) -> dict:
        return dict(
            analysis=self.analysis, synthesis=self.synthesis, w1=self.w1, w2=self.w2,
            embedding=self.embedding, mean_head=self.mean_head,
            nbr_weight=self.nbr_weight, laplace_scale=self.laplace_scale,
            base_step=self.base_step, n_layers=N_LAYERS, n_kv_heads=N_KV_HEADS,
            head_dim=HEAD_DIM, keep_head=KEEP_HEAD, keep_tail=KEEP_TAIL,
            rope_theta=ROPE_THETA,
        )


def z_scales(d: int = D) -> np.ndarray:
    """Per-direction Laplace scale of the row model: 0.5 (k+1)^-0.7."""
    return 0.5 * (np.arange(d, dtype=np.float64) + 1.0) ** -0.7


def _orthonormal(rng: np.random.Generator, d: int) -> np.ndarray:
    import torch

    g = rng.standard_normal((d, d), dtype=np.float32)
    q, r = torch.linalg.qr(torch.from_numpy(g))
    q = q.numpy()
    sign = np.sign(np.diag(r.numpy()))
    sign[sign == 0] = 1.0
    return np.ascontiguousarray(q * sign[None, :], dtype=np.float32)


def _rows_from_z(U: np.ndarray, z: np.ndarray, e: np.ndarray) -> np.ndarray:
    import torch

    x = torch.from_numpy(np.ascontiguousarray(z, dtype=np.float32)) @ torch.from_numpy(U).T
    return x.numpy() + e.astype(np.float32)


def _build_world() -> World:
    ss = np.random.SeedSequence(CODEC_SEED)
    (s_u, s_cz, s_ce, s_ct, s_w1, s_w2, s_e, s_h, s_a) = ss.spawn(9)
    U = _orthonormal(np.random.default_rng(s_u), D)

    # calibration batch, same row model as the requests
    sig = z_scales()
    zc = np.random.default_rng(s_cz).laplace(0.0, 1.0, size=(CALIB_ROWS, D)) * sig[None, :]
    ec = np.random.default_rng(s_ce).normal(0.0, 1e-3, size=(CALIB_ROWS, D))
    xc = bf16_bits_to_f32(to_bf16_bits(_rows_from_z(U, zc, ec))).astype(np.float64)
    tok_c = np.random.default_rng(s_ct).integers(0, VOCAB, size=CALIB_ROWS)

    # basis: uncentred PCA of the calibration rows
    _, _, vt = np.linalg.svd(xc, full_matrices=False)
    B = vt[:N_COEF].T.copy()  # [D][N_COEF], orthonormal columns
    idx = np.argmax(np.abs(B), axis=0)
    sgn = np.sign(B[idx, np.arange(N_COEF)])
    sgn[sgn == 0] = 1.0
    B *= sgn[None, :]
    A_bits = to_bf16_bits(B.T.astype(np.float32))
    S_bits = to_bf16_bits(B.astype(np.float32))

    W1 = to_bf16_bits(np.random.default_rng(s_w1).normal(0.0, 0.01, size=(N_HIDDEN, N_COEF)).astype(np.float32))
    W2 = to_bf16_bits(np.random.default_rng(s_w2).normal(0.0, 0.01, size=(D, N_HIDDEN)).astype(np.float32))
    E = to_bf16_bits(np.random.default_rng(s_e).normal(0.0, 0.02, size=(VOCAB, EMB_DIM)).astype(np.float32))
    H = to_bf16_bits(np.random.default_rng(s_h).normal(0.0, 0.02, size=(N_COEF, EMB_DIM)).astype(np.float32))
    a = np.random.default_rng(s_a).uniform(0.0, 0.5, size=N_COEF).astype(np.float32)
    delta = np.ones(N_COEF, dtype=np.float32)

    # Laplace scale fit on the calibration batch (open loop, parameter synthesis)
    Af = bf16_bits_to_f32(A_bits).astype(np.float64)
    Hf = bf16_bits_to_f32(H).astype(np.float64)
    Ef = bf16_bits_to_f32(E[tok_c]).astype(np.float64)
    y = xc @ Af.T
    m = Ef @ Hf.T
    nb = np.zeros_like(y)
    nb[1:] += y[:-1]
    nb[:-1] += y[1:]
    resid = y - m
    odd = np.arange(CALIB_ROWS) % 2 == 1
    resid[odd] -= a.astype(np.float64)[None, :] * nb[odd]
    b = np.maximum(np.mean(np.abs(resid), axis=0), 1e-12).astype(np.float32)

    return World(analysis=A_bits, synthesis=S_bits, w1=W1, w2=W2, embedding=E, mean_head=H,
                 nbr_weight=a, laplace_scale=b, base_step=delta, U=U)


_WORLD: World | None = None


def world(use_cache: bool = True) -> World:
    """The seeded synthetic codec (built once per process, cached on disk)."""
    global _WORLD
    if _WORLD is not None:
        return _WORLD
    path = os.path.join(_CACHE_DIR, _WORLD_VERSION + ".npz")
    if use_cache and os.path.exists(path):
        with np.load(path, allow_pickle=False) as z:
            _WORLD = World(**{k: z[k] for k in z.files})
        return _WORLD
    w = _build_world()
    if use_cache:
        try:
            os.makedirs(_CACHE_DIR, exist_ok=True)
            tmp = path + ".tmp.npz"
            np.savez(tmp, **{k: getattr(w, k) for k in w.__dataclass_fields__})
            os.replace(tmp, path)
        except OSError:
            pass
    _WORLD = w
    return w


# --------------------------------------------------------------------------
# requests
# --------------------------------------------------------------------------
@dataclass
class Request:
    rows: np.ndarray       # uint16 bf16 bits [T][D], pre-RoPE
    token_ids: np.ndarray  # int32 [T]
    step_scale: float      # rate setting g
    rate_target: float     # bytes per coded token the step scale was chosen for
    T: int
    note: str = ""


_STEP_SCALES_FILE = os.path.join(_HERE, "step_scales.json")


def step_scale_for(rate_bytes_per_token: float) -> float:
    """Step scale g for a rate target, from the table the rate ladder script wrote."""
    with open(_STEP_SCALES_FILE) as f:
        table = json.load(f)
    key = "%g" % rate_bytes_per_token
    if key not in table["step_scale"]:
        raise KeyError("no step scale for rate %s B/token; rerun oracle/rate_ladder.py" % key)
    return float(table["step_scale"][key])


CONFIGS = {
    0: dict(name="tiny-512", T=512, rate=220.0, seed=1000),
    1: dict(name="prompt-4k-55x", T=4096, rate=12288.0 / 55.0, seed=1001),
    2: dict(name="prompt-32k-100x-outliers", T=32768, rate=120.0, seed=1002, outlier_frac=0.001,
            outlier_gain=20.0),
    3: dict(name="prompt-128k", T=131072, rate=220.0, seed=1003),
    4: dict(name="batch-16x8k-mixed", T=8192, rate=None, seed=1004, n_requests=16,
            rates=(60.0, 120.0, 220.0, 400.0), t3_frac=0.1),
}

RATE_TARGETS = (60.0, 120.0, 220.0, 12288.0 / 55.0, 400.0)


def _draw_rows(w: World, T: int, ss: np.random.SeedSequence, outlier_frac=0.0, outlier_gain=1.0,
               t3_frac=0.0, n_rows: int | None = None):
    """Rows x = U z + e for positions 0..T-1 (or the first n_rows of them)."""
    s_z, s_e, s_tok, s_out, s_mix = ss.spawn(5)
    n = T if n_rows is None else min(T, n_rows)
    sig = z_scales()
    n_chunks = (T + ROW_CHUNK - 1) // ROW_CHUNK
    zc = s_z.spawn(n_chunks)
    ecs = s_e.spawn(n_chunks)
    mcs = s_mix.spawn(n_chunks)
    N = max(T - KEEP_HEAD - KEEP_TAIL, 0)
    gain = np.ones(T, dtype=np.float32)
    if outlier_frac > 0 and N > 0:
        k = int(round(outlier_frac * N))
        pick = np.random.default_rng(s_out).choice(N, size=k, replace=False) + KEEP_HEAD
        gain[pick] = outlier_gain
    out = np.empty((n, D), dtype=np.uint16)
    for c in range((n + ROW_CHUNK - 1) // ROW_CHUNK):
        r0 = c * ROW_CHUNK
        r1 = min(r0 + ROW_CHUNK, T)
        rows = r1 - r0
        eps = np.random.default_rng(zc[c]).laplace(0.0, 1.0, size=(rows, D))
        if t3_frac > 0:
            rm = np.random.default_rng(mcs[c])
            use_t = rm.random(size=(rows, D)) < t3_frac
            tv = rm.standard_t(3.0, size=(rows, D))
            eps = np.where(use_t, tv, eps)
        z = eps * sig[None, :]
        e = np.random.default_rng(ecs[c]).normal(0.0, 1e-3, size=(rows, D))
        x = _rows_from_z(w.U, z, e) * gain[r0:r1, None]
        take = min(rows, n - r0)
        if take <= 0:
            break
        out[r0:r0 + take] = to_bf16_bits(x[:take])
    tok = np.random.default_rng(s_tok).integers(0, VOCAB, size=T).astype(np.int32)
    return out, tok[:n] if n_rows is not None else tok


def make_request(cfg: int, index: int = 0, T: int | None = None, n_rows: int | None = None) -> Request:
    """The seeded request of a workload.

    cfg 0..3 are single prompts, cfg 4 is the 16-request batch (``index`` picks
    the request).  ``T`` overrides the prompt length (same seeds, shorter
    prompt); ``n_rows`` generates only the first rows of the prompt (a bounded
    sample of the same workload).
    """
    c = CONFIGS[cfg]
    w = world()
    TT = c["T"] if T is None else int(T)
    if cfg == 4:
        ss = np.random.SeedSequence(c["seed"]).spawn(c["n_requests"])[index]
        s_rows, s_rate = ss.spawn(2)
        rate = c["rates"][int(np.random.default_rng(s_rate).integers(len(c["rates"])))]
        rows, tok = _draw_rows(w, TT, s_rows, t3_frac=c["t3_frac"], n_rows=n_rows)
        note = "t3-mixture request %d" % index
    else:
        s_rows, _ = np.random.SeedSequence(c["seed"]).spawn(2)
        rate = c["rate"]
        rows, tok = _draw_rows(w, TT, s_rows, outlier_frac=c.get("outlier_frac", 0.0),
                               outlier_gain=c.get("outlier_gain", 1.0), n_rows=n_rows)
        note = c["name"]
    return Request(rows=rows, token_ids=tok, step_scale=step_scale_for(rate), rate_target=rate, T=TT,
                   note=note)


RATE_CALIB_ROWS = 4096


def calibration_sample(n_rows: int = RATE_CALIB_ROWS):
    """Rows and token ids of the held-out sample the rate ladder is calibrated
    on: the row model with a seed of its own (neither a workload nor the batch
    the basis and scales were fitted on)."""
    w = world()
    return _draw_rows(w, n_rows, np.random.SeedSequence([CODEC_SEED, 1]))


def random_rows(T: int, seed: int, gain: float = 1.0):
    """Rows and token ids from the row model with an arbitrary seed (edge-case tests)."""
    w = world()
    rows, tok = _draw_rows(w, T, np.random.SeedSequence(seed), outlier_frac=0.0)
    if gain != 1.0:
        rows = to_bf16_bits(bf16_bits_to_f32(rows) * np.float32(gain))
    return rows, tok


def rate_noise(n_rows: int, n_coef: int, seed: int) -> np.ndarray:
    """Uniform noise in [-1/2, 1/2) steps, float32 [n_rows][n_coef] (the
    additive noise of the training rate, drawn by the caller)."""
    rng = np.random.default_rng(np.random.SeedSequence([CODEC_SEED, 77, int(seed)]))
    return (rng.random((n_rows, n_coef), dtype=np.float32) - np.float32(0.5)).astype(np.float32)
