"""Rate plan: quantisation steps, dropped components, integer Laplace tables.

Sources (DCKV digest page, "How it works"):
  * Transform bullet: per-component quantisation steps; components whose
    Laplace scale is below 0.05 quantisation steps are dropped.
  * Coding bullet: codes are rANS-coded under Laplace distributions.
  * "What it claims"/Training: steps are trained per component and one trained
    codec gives one rate.
  * "Limits": table selection needs encoder and decoder to compute identical
    predictions.

Readings taken where the pages are silent:
  * The rate setting is one scalar g: step_c = fp32(g * delta_c) (IEEE float32
    product), so one set of trained base steps gives a ladder of rates.
  * Scale in steps s_c = b_c / step_c in float64; component c is dropped when
    s_c < 0.05 (strictly below).  Active components are ranked by ascending c.
  * The conditional mean shifts the quantisation grid (codes are taken around
    the predicted mean), so the code pmf is a zero-mean discretised Laplace of
    scale s_c: one static table per component.  Encoder and decoder therefore
    share tables that do not depend on any float prediction.
  * The alphabet is the 255 codes -127..127 (index k+127); codes beyond +-127
    leave the alphabet (escaped).  Table precision is 15 bits (M = 2^15).
  * Integer table of component c, from the discretised Laplace restricted to
    the alphabet and renormalised:
        p_0 = 1 - exp(-0.5/s),  p_k = (exp(-(|k|-0.5)/s) - exp(-(|k|+0.5)/s))/2
        total = p_-127 + ... + p_127, summed in that index order
        f_k = 1 + floor(p_k/total * (M - 255)),  then f_0 += M - sum(f)
        cum_0 = 0, cum_{i+1} = cum_i + f_i  (index order)
  * Plan CRC: CRC-32 (zlib polynomial) over the steps (fp32, little endian),
    the active flags (one byte each) and the frequencies of the active
    components in rank order (u16 little endian).
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass

import numpy as np

PREC_BITS = 15
M = 1 << PREC_BITS
N_SYM = 255          # codes -127..127
ESC = 255            # marks an escaped position in a symbol array
DROP_BELOW = 0.05    # steps


@dataclass
class Plan:
    step_scale: np.float32
    step: np.ndarray      # fp32 [C]
    active: np.ndarray    # bool [C]
    act_idx: np.ndarray   # int64 [C_a]  component of each rank
    rank: np.ndarray      # int64 [C]    rank of each component, -1 if dropped
    freq: np.ndarray      # int64 [C_a][255]
    cum: np.ndarray       # int64 [C_a][256]  (cum[:, 255] == M)
    pmf: np.ndarray       # float64 [C_a][255] renormalised model pmf
    crc: int

    @property
    def c_active(self) -> int:
        return int(self.act_idx.size)


def steps(step_scale, base_step) -> np.ndarray:
    """step_c = fp32(g * delta_c): IEEE float32 product, round to nearest even."""
    return (np.float32(step_scale) * np.asarray(base_step, dtype=np.float32)).astype(np.float32)


def laplace_tables(s: np.ndarray):
    """Integer frequency tables for Laplace scales ``s`` (in steps), float64."""
    s = np.asarray(s, dtype=np.float64)
    k = np.arange(-127, 128, dtype=np.float64)[None, :]
    ak = np.maximum(np.abs(k), 1.0)  # the k = 0 entry is set below
    ss = s[:, None]
    p = 0.5 * np.exp(-(ak - 0.5) / ss) - 0.5 * np.exp(-(ak + 0.5) / ss)
    p[:, 127] = 1.0 - np.exp(-0.5 / s)
    total = np.zeros(s.shape[0], dtype=np.float64)
    for i in range(N_SYM):  # index order, sequential
        total = total + p[:, i]
    pn = p / total[:, None]
    f = 1 + np.floor(pn * (M - N_SYM)).astype(np.int64)
    f[:, 127] += M - f.sum(axis=1)
    cum = np.zeros((s.shape[0], N_SYM + 1), dtype=np.int64)
    cum[:, 1:] = np.cumsum(f, axis=1)
    return f, cum, pn


def plan_crc(step: np.ndarray, active: np.ndarray, freq: np.ndarray) -> int:
    blob = (np.asarray(step, dtype="<f4").tobytes()
            + np.asarray(active, dtype=np.uint8).tobytes()
            + np.asarray(freq, dtype="<u2").tobytes())
    return zlib.crc32(blob) & 0xFFFFFFFF


def make_plan(step_scale, base_step, laplace_scale) -> Plan:
    step = steps(step_scale, base_step)
    s = np.asarray(laplace_scale, dtype=np.float32).astype(np.float64) / step.astype(np.float64)
    active = s >= DROP_BELOW
    act_idx = np.nonzero(active)[0]
    rank = -np.ones(step.shape[0], dtype=np.int64)
    rank[act_idx] = np.arange(act_idx.size)
    if act_idx.size:
        f, cum, pn = laplace_tables(s[act_idx])
    else:
        f = np.zeros((0, N_SYM), np.int64)
        cum = np.zeros((0, N_SYM + 1), np.int64)
        pn = np.zeros((0, N_SYM))
    return Plan(step_scale=np.float32(step_scale), step=step, active=active, act_idx=act_idx, rank=rank,
                freq=f, cum=cum, pmf=pn, crc=plan_crc(step, active, f))


def modelled_bytes_per_token(p: Plan, flush_bits_per_substream: float = 24.0,
                             block: int = 256) -> float:
    """Expected coded bytes per token under the plan's own model.

    Sum over active components of the model cross-entropy (15 - log2 f_k)
    weighted by the model pmf, plus the per-substream flush (about 24 bits per
    (component, 256-token block) substream), in bytes.
    """
    if p.c_active == 0:
        return 0.0
    bits = (p.pmf * (PREC_BITS - np.log2(p.freq))).sum()
    return float(bits / 8.0 + p.c_active * flush_bits_per_substream / 8.0 / block)
