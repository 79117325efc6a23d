"""The plan's embedding-mean table on the GPU against the oracle.

The code means of a position come from its token's input embedding (DCKV
digest, "How it works", Conditional entropy models); the mean of every
coefficient depends on the token id alone, so the plan holds H E[v] for the
whole vocabulary.  Bars:
  - columns: the active components in rank order, then the dropped ones in
    ascending order (a permutation of all components);
  - sampled rows (first, last, seeded random ids) within relative L2 1e-5 of
    the oracle's float64 mean of the same bf16 inputs (fp32 accumulation over
    2,048 bf16 products), every row on its own;
  - the same with dropped components, whose columns follow the active ones;
  - plans with the same embedding, mean head and active set share one table
    (reference-counted; the last plan frees it).
"""
from __future__ import annotations

import numpy as np
import pytest

import dckv_synth as synth
from oracle import codec as ocodec
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

TOL = 1e-5


def _check_plan(plan, params, p):
    dk = gu.dk()
    tab, cols = dk.mean_table(plan)
    vocab, C = tab.shape
    assert vocab == params["embedding"].shape[0] and C == p.step.size
    # column order
    assert np.array_equal(np.sort(cols), np.arange(C))
    assert np.array_equal(cols[:p.c_active], p.act_idx)
    assert np.array_equal(cols[p.c_active:], np.flatnonzero(~p.active))
    rng = np.random.default_rng(31)
    ids = np.unique(np.concatenate([[0, 1, 255, 256, vocab - 1], rng.choice(vocab, size=64, replace=False)]))
    got = tab[ids].cpu().numpy().astype(np.float64)
    want = ocodec.embedding_mean(params, ids)[:, cols]
    for n, v in enumerate(ids):
        e = gu.rel_l2(got[n], want[n])
        assert e <= TOL, (int(v), e)
    gu.say("  %d table rows, worst rel %.3g" % (len(ids), max(gu.rel_l2(got[n], want[n]) for n in range(len(ids)))))


def test_mean_table_matches_oracle():
    params = synth.world().params()
    g = synth.step_scale_for(220.0)
    plan = gu.device_codec().plan(g)
    gu.say("mean table, C_a = %d" % plan.c_active)
    _check_plan(plan, params, gu.oracle_plan(params, g))


def test_mean_table_with_dropped_components():
    w = synth.world()
    rng = np.random.default_rng(5)
    scale = w.laplace_scale.copy()
    scale[rng.choice(2048, size=77, replace=False)] = 1e-5
    params = gu.params_with_scales(scale)
    g = synth.step_scale_for(220.0)
    p = gu.oracle_plan(params, g)
    plan = gu.codec_with_scales(scale).plan(g)
    assert plan.c_active == p.c_active < 2048
    gu.say("mean table, C_a = %d" % plan.c_active)
    _check_plan(plan, params, p)


def test_plans_share_one_mean_table():
    """Plans with the same embedding, mean head and active set (here: the four
    rates of the batch workload, all with every component active) hold one
    table; a plan with dropped components gets its own; the last plan to go
    frees it, and a plan made after that builds a fresh, correct one."""
    import torch
    dk = gu.dk()
    params = synth.world().params()
    codec = gu.device_codec()
    rates = (60.0, 120.0, 220.0, 400.0)
    plans = [codec.plan(synth.step_scale_for(r)) for r in rates]
    ptrs = {dk.dckv_plan_mean_table(p)[0] for p in plans}
    mem = [dk.dckv_plan_memory(p) for p in plans]
    gu.say("  4 rates: %d table(s); users %s; plan block %d B, table %d B" %
           (len(ptrs), [m["mean_table_users"] for m in mem], mem[0]["table_bytes"], mem[0]["mean_table_bytes"]))
    assert all(p.c_active == 2048 for p in plans)
    assert len(ptrs) == 1
    assert all(m["mean_table_users"] >= 4 for m in mem)
    assert mem[0]["mean_table_bytes"] == params["embedding"].shape[0] * 2048 * 4
    # a plan with dropped components: another column order, another table
    scale = synth.world().laplace_scale.copy()
    scale[::3] = 1e-5
    other = gu.codec_with_scales(scale).plan(synth.step_scale_for(220.0))
    assert dk.dckv_plan_mean_table(other)[0] not in ptrs
    assert dk.dckv_plan_memory(other)["mean_table_users"] == 1
    # freeing all but one keeps the table; the survivor still codes correctly
    n_before = dk.dckv_plan_memory(plans[0])["mean_table_users"]
    for p in plans[1:]:
        p.free()
    assert dk.dckv_plan_memory(plans[0])["mean_table_users"] == n_before - 3
    req = synth.make_request(0)
    g = synth.step_scale_for(60.0)
    data, st = gu.gpu_encode(plans[0], req.rows, req.token_ids)
    assert st == 0
    enc = ocodec.encode(req.rows, req.token_ids, params, gu.oracle_plan(params, g))
    sym = gu.oracle_symbols_of_stream(data, params, gu.oracle_plan(params, g), req.T)[1]
    agree = float(np.mean(sym == enc.sym))
    gu.say("  survivor plan: symbol agreement %.7f" % agree)
    assert agree >= gu.SYMBOL_AGREEMENT
    plans[0].free()
    other.free()
    torch.cuda.synchronize()
    # a new plan after the table was released builds a correct one again
    fresh = codec.plan(synth.step_scale_for(220.0))
    _check_plan(fresh, params, gu.oracle_plan(params, synth.step_scale_for(220.0)))
    fresh.free()
