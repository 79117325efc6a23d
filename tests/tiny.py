"""Tiny codec parameters for brute-force oracle tests (dimension-generic)."""
from __future__ import annotations

import numpy as np

from oracle import bf16


def tiny_params(seed=0, n_layers=1, n_kv_heads=1, head_dim=8, n_coef=8, n_hidden=4, emb_dim=4,
                vocab=16, keep_head=1, keep_tail=2, rope_theta=100.0, orthonormal=True, w2_zero=False):
    rng = np.random.default_rng(seed)
    D = n_layers * 2 * n_kv_heads * head_dim
    if orthonormal:
        q, _ = np.linalg.qr(rng.standard_normal((D, D)))
        B = q[:, :n_coef]
    else:
        B = rng.standard_normal((D, n_coef)) * 0.3
    p = dict(
        analysis=bf16.from_f64(B.T), synthesis=bf16.from_f64(B),
        w1=bf16.from_f64(rng.normal(0, 0.3, (n_hidden, n_coef))),
        w2=bf16.from_f64(np.zeros((D, n_hidden)) if w2_zero else rng.normal(0, 0.3, (D, n_hidden))),
        embedding=bf16.from_f64(rng.normal(0, 0.5, (vocab, emb_dim))),
        mean_head=bf16.from_f64(rng.normal(0, 0.5, (n_coef, emb_dim))),
        nbr_weight=rng.uniform(0, 0.5, n_coef).astype(np.float32),
        laplace_scale=rng.uniform(0.05, 1.0, n_coef).astype(np.float32),
        base_step=np.ones(n_coef, dtype=np.float32),
        n_layers=n_layers, n_kv_heads=n_kv_heads, head_dim=head_dim, keep_head=keep_head,
        keep_tail=keep_tail, rope_theta=rope_theta)
    return p


def tiny_rows(params, T, seed=1, scale=1.0):
    rng = np.random.default_rng(seed)
    D = params["analysis"].shape[1]
    rows = bf16.from_f64(rng.laplace(0, scale, (T, D)))
    tok = rng.integers(0, params["embedding"].shape[0], T).astype(np.int32)
    return rows, tok
