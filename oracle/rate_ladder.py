"""Rate ladder: the step scale g that meets a bytes-per-token target.

Test infrastructure (CPU, float64): part of the oracle.  Only the tests, the
smoke check, the benchmark's CPU-baseline leg and this script itself use it.

One trained codec gives one rate (DCKV digest, "How it works", Training
bullet: the rate-distortion weight is fixed per codec, and rescaling the steps
of a trained codec costs bytes or quality).  The synthetic codec here gets its
ladder of rates by scaling every base step with one scalar g
(step_c = fp32(g * delta_c)).

Reading taken where the pages are silent: a target of B bytes per coded token
is met on data, not on the plan's own Laplace model.  g is the smallest fp32
value for which the encoder's stream over a held-out seeded calibration sample
(rows of the same row model, neither a workload nor the batch the basis was
fitted on) spends at most B bytes per coded token: group offsets, escape
records and rANS words, i.e. everything but the header and the kept rows.
The plan's a-priori estimate (``plan.modelled_bytes_per_token``) is not used
for this: on the synthetic rows the residuals of the tail components are close
to Gaussian, so a Laplace of the same mean absolute value puts several times
too much mass outside the zero bin at coarse steps, and the estimate
overstates the coded bytes (by about 40 % at 120 bytes per token).

Run as a script, it writes ``dckv_synth/step_scales.json``, the table the
seeded workloads read their rate setting from:

    python -m oracle.rate_ladder
"""
from __future__ import annotations

import json
import os
import sys
from dataclasses import dataclass

import numpy as np

from . import bf16, codec, rans, stream
from .plan import Plan, make_plan, modelled_bytes_per_token

G_MIN = 2.0 ** -16
G_MAX = 16.0


def smallest_scale(meets, lo: float = G_MIN, hi: float = G_MAX) -> float:
    """Smallest fp32 g in [lo, hi] with ``meets(g)``.

    ``meets`` must be false below some threshold and true from it on (coded
    bytes do not grow as the steps grow).  Positive fp32 values are ordered
    like their bit patterns, so the search bisects over the integers those
    patterns spell and ends on two neighbouring fp32 values: ``meets`` is
    false at the lower one and true at the returned one.  If ``meets(hi)`` is
    false, hi is returned; if ``meets(lo)`` is true, lo.
    """
    a = int(np.float32(lo).view(np.int32))
    b = int(np.float32(hi).view(np.int32))

    def val(k: int) -> np.float32:
        return np.array([k], dtype=np.int32).view(np.float32)[0]

    if not meets(val(b)):
        return float(val(b))
    if meets(val(a)):
        return float(val(a))
    while b - a > 1:
        mid = (a + b) // 2
        if meets(val(mid)):
            b = mid
        else:
            a = mid
    return float(val(b))


@dataclass
class Sample:
    """Coefficients of a calibration sample taken as N consecutive coded rows."""

    y: np.ndarray    # float64 [N][C] analysis coefficients A x
    m: np.ndarray    # float64 [N][C] embedding means H E[tok]
    a: np.ndarray    # fp32 [C] neighbour weights

    @property
    def N(self) -> int:
        return int(self.y.shape[0])


def sample_from_rows(rows: np.ndarray, tok: np.ndarray, params: dict) -> Sample:
    """y = A x and the embedding means of rows that are all coded (float64)."""
    X = bf16.to_f64(rows)
    A = bf16.to_f64(params["analysis"])
    return Sample(y=X @ A.T, m=codec.embedding_mean(params, tok),
                  a=np.asarray(params["nbr_weight"], dtype=np.float32))


def coded_bytes(s: Sample, p: Plan) -> int:
    """Bytes the encoder writes for the sample's coded rows under plan p: the
    stream without its header and kept rows (u32 group offsets, 8-byte escape
    records, the rANS words)."""
    q, _ = codec.quantize(s.y, s.m, p, s.a)
    sym, flat, qe = codec.symbols(q, p)
    groups = rans.encode_all(sym, p.freq, p.cum) if s.N > 0 and p.c_active > 0 else []
    n_blk, G, _, _ = rans.group_shape(s.N, p.c_active)
    h = stream.Header(T=s.N, keep_head=0, keep_tail=0, N=s.N, n_coef=s.y.shape[1],
                      c_active=p.c_active, n_groups=n_blk * G, n_esc=len(flat),
                      step_scale=float(p.step_scale), plan_crc=p.crc, total_bytes=0, rans_bytes=0)
    kept = np.zeros((0, 1), dtype=np.uint16)
    return len(stream.write(h, kept, groups, flat, qe)) - stream.HEADER_BYTES


def coded_bytes_per_token(s: Sample, p: Plan) -> float:
    return coded_bytes(s, p) / s.N if s.N else 0.0


def step_scale_for_rate(target: float, s: Sample, base_step, laplace_scale) -> float:
    """Smallest fp32 g whose stream over the sample spends at most ``target``
    bytes per coded token."""
    def meets(g):
        return coded_bytes_per_token(s, make_plan(np.float32(g), base_step, laplace_scale)) <= target

    return smallest_scale(meets)


def main(argv=None) -> int:
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    import dckv_synth as synth

    w = synth.world()
    rows, tok = synth.calibration_sample()
    s = sample_from_rows(rows, tok, w.params())
    out = {"calibration_rows": s.N, "target": {}, "step_scale": {}, "calibration_bytes_per_token": {},
           "modelled_bytes_per_token": {}}
    for rate in synth.RATE_TARGETS:
        g = step_scale_for_rate(rate, s, w.base_step, w.laplace_scale)
        p = make_plan(np.float32(g), w.base_step, w.laplace_scale)
        key = "%g" % rate
        out["target"][key] = rate
        out["step_scale"][key] = g
        out["calibration_bytes_per_token"][key] = coded_bytes_per_token(s, p)
        out["modelled_bytes_per_token"][key] = modelled_bytes_per_token(p)
        print("rate %8.3f B/token -> g = %.9g  (C_a = %d, sample %.3f, a-priori model %.3f)" %
              (rate, g, p.c_active, out["calibration_bytes_per_token"][key],
               out["modelled_bytes_per_token"][key]), flush=True)
    path = os.path.join(root, "dckv_synth", "step_scales.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
