"""Rate ladder: the step scale g that meets a bytes-per-token target.

One trained codec gives one rate (DCKV digest, "How it works", Training); the
synthetic codec here gets its rate ladder by scaling every base step with one
scalar g.  For a target B bytes per coded token, g is the smallest value (by
bisection on log2 g in [-16, 4], 60 steps) whose modelled bytes per token (the
plan's own cross-entropy plus the per-substream flush) do not exceed B.

Run as a script, it writes ``dckv_synth/step_scales.json``, the table the
seeded workloads read their rate setting from:

    python -m oracle.rate_ladder
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

from .plan import make_plan, modelled_bytes_per_token


def step_scale_for_rate(target: float, base_step, laplace_scale, iters: int = 60) -> float:
    lo, hi = -16.0, 4.0  # log2 g; bytes decrease as g grows

    def bytes_at(lg):
        return modelled_bytes_per_token(make_plan(np.float32(2.0 ** lg), base_step, laplace_scale))

    if bytes_at(hi) > target:
        return float(np.float32(2.0 ** hi))
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if bytes_at(mid) <= target:
            hi = mid
        else:
            lo = mid
    g = np.float32(2.0 ** hi)
    if bytes_at(np.log2(float(g))) > target:  # rounding to fp32 must not overshoot the target
        g = np.nextafter(g, np.float32(np.inf))
    return float(g)


def main(argv=None) -> int:
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    import dckv_synth as synth

    w = synth.world()
    out = {"step_scale": {}, "modelled_bytes_per_token": {}}
    for rate in synth.RATE_TARGETS:
        g = step_scale_for_rate(rate, w.base_step, w.laplace_scale)
        p = make_plan(np.float32(g), w.base_step, w.laplace_scale)
        key = "%g" % rate
        out["step_scale"][key] = g
        out["modelled_bytes_per_token"][key] = modelled_bytes_per_token(p)
        print("rate %8.3f B/token -> g = %.9g  (C_a = %d, modelled %.3f)" %
              (rate, g, p.c_active, out["modelled_bytes_per_token"][key]))
    path = os.path.join(root, "dckv_synth", "step_scales.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
