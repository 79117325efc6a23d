"""A paged attention cache on either side of the codec, on the GPU (DCKV
digest, "How it works", first paragraph: keys are coded before RoPE and RoPE
is reapplied after decoding; abstract page: the cache is stored or moved to be
reused).

The pools hold the request's positions in shuffled blocks (block table a
seeded permutation of a larger pool, block sizes that do and do not divide T);
every other row of the pools holds a sentinel.  Bars:
  - dckv_encode_paged writes dckv_encode's stream of the same rows, byte for
    byte (post_rope = 0), and dckv_encode_postrope's stream of the same
    post-RoPE rows (post_rope = 1);
  - dckv_decode_paged writes exactly dckv_decode's rows into the request's
    rows of the pools and leaves every other row untouched; those rows are
    within the rows' bar of the oracle's decode of the same stream;
  - a block table entry outside the pool gives DCKV_EINVAL on the device
    (encode: size 0), with nothing read from or written to the pools.
"""
from __future__ import annotations

import numpy as np
import pytest

import dckv_synth as synth
from oracle import bf16, codec as ocodec
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FC1  # a bf16 NaN pattern the codec never writes


def _layout(T, bs, extra, seed):
    """Block table of a request of T positions in a pool with `extra` spare blocks."""
    n_log = (T + bs - 1) // bs
    n_blocks = n_log + extra
    rng = np.random.default_rng(seed)
    table = rng.permutation(n_blocks)[:n_log].astype(np.int32)
    return table, n_blocks


def _physical_rows(T, bs, table):
    t = np.arange(T)
    return table[t // bs].astype(np.int64) * bs + t % bs


def _pools_from_rows(rows, T, bs, table, n_blocks):
    """numpy pools [12][n_blocks * bs][2][256] (uint16) holding rows at their physical rows."""
    pools = np.full((12, n_blocks * bs, 2, 256), SENTINEL, np.uint16)
    phys = _physical_rows(T, bs, table)
    r = rows.reshape(T, 12, 2, 256)  # column block (l 2 + kv), head, dim
    for i in range(12):
        pools[i, phys] = r[:, i]
    return pools


def _dev_cache(pools, table, bs, n_blocks):
    import torch
    tens = [gu.to_dev(pools[i].reshape(n_blocks, bs, 2, 256).view(np.int16)) for i in range(12)]
    return gu.dk().PagedKV(tens, gu.to_dev(table), bs), tens


def _pools_back(tens):
    return np.stack([t.cpu().numpy().view(np.uint16).reshape(-1, 2, 256) for t in tens])


def _encode_paged(plan, cache, post_rope, tok):
    import torch
    dk = gu.dk()
    T = len(tok)
    cap, _ = dk.dckv_bytes(plan, T)
    buf = torch.empty(cap, dtype=torch.uint8, device="cuda:0")
    nb = torch.zeros(1, dtype=torch.int64, device="cuda:0")
    st = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    ws = torch.empty(dk.dckv_bytes_paged(plan, T), dtype=torch.uint8, device="cuda:0")
    dk.dckv_encode_paged(plan, cache, post_rope, gu.to_dev(tok.astype(np.int32)), buf, nb, st, ws)
    torch.cuda.synchronize()
    n = int(nb.item())
    return buf[:n].cpu().numpy().tobytes(), int(st.item())


def _decode_paged(plan, data, tok, cache):
    import torch
    dk = gu.dk()
    T = len(tok)
    buf = gu.to_dev(np.frombuffer(data, dtype=np.uint8).copy())
    st = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    ws = torch.empty(dk.dckv_bytes_paged(plan, T), dtype=torch.uint8, device="cuda:0")
    dk.dckv_decode_paged(plan, buf, len(data), gu.to_dev(tok.astype(np.int32)), cache, st, ws)
    torch.cuda.synchronize()
    return int(st.item())


def _request(case):
    if case.startswith("c"):
        req = synth.make_request(int(case[1]))
        return req.rows, req.token_ids, req.step_scale
    T = int(case[1:])
    rows, tok = synth.random_rows(T, seed=5000 + T)
    return rows, tok, synth.step_scale_for(220.0)


@pytest.mark.parametrize("case,bs", [("c0", 16), ("c1", 16), ("c1", 48), ("T100", 16), ("T389", 7)])
def test_paged_encode_and_decode_equal_contiguous(case, bs):
    rows, tok, g = _request(case)
    T = len(tok)
    plan = gu.device_codec().plan(g)
    table, n_blocks = _layout(T, bs, extra=5, seed=77 + T + bs)
    gu.say("%s: T=%d block_size %d, %d of %d blocks" % (case, T, bs, len(table), n_blocks))
    want, st = gu.gpu_encode(plan, rows, tok)
    assert st == 0
    cache, _ = _dev_cache(_pools_from_rows(rows, T, bs, table, n_blocks), table, bs, n_blocks)
    got, st = _encode_paged(plan, cache, False, tok)
    assert st == 0 and got == want
    # decode into fresh pools: the request's rows equal dckv_decode's, the rest untouched
    dec, st = gu.gpu_decode(plan, want, tok)
    assert st == 0
    empty = np.full((12, n_blocks * bs, 2, 256), SENTINEL, np.uint16)
    cache2, tens = _dev_cache(empty, table, bs, n_blocks)
    assert _decode_paged(plan, want, tok, cache2) == 0
    back = _pools_back(tens)
    expect = _pools_from_rows(dec, T, bs, table, n_blocks)
    gu.say("  decode into the pools equal %s" % np.array_equal(back, expect))
    assert np.array_equal(back, expect)
    if case in ("c0", "T389"):
        params = synth.world().params()
        p = gu.oracle_plan(params, g)
        o = ocodec.decode(want, tok, params, p)
        phys = _physical_rows(T, bs, table)
        got_rows = np.ascontiguousarray(back[:, phys].transpose(1, 0, 2, 3).reshape(T, -1))
        e = gu.rel_l2(bf16.to_f64(got_rows), bf16.to_f64(o.rows))
        gu.say("  paged rows vs oracle decode: rel %.3g" % e)
        assert e <= gu.REL_L2_TOL


@pytest.mark.parametrize("case,bs", [("c1", 16), ("T389", 32)])
def test_paged_encode_of_a_post_rope_cache(case, bs):
    import torch
    rows, tok, g = _request(case)
    T = len(tok)
    plan = gu.device_codec().plan(g)
    data, st = gu.gpu_encode(plan, rows, tok)
    assert st == 0
    post, st = gu.gpu_decode(plan, data, tok)  # keys carry RoPE
    assert st == 0
    dk = gu.dk()
    # the contiguous post-RoPE encode of the same rows
    cap, _ = dk.dckv_bytes(plan, T)
    buf = torch.empty(cap, dtype=torch.uint8, device="cuda:0")
    nb = torch.zeros(1, dtype=torch.int64, device="cuda:0")
    stt = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    ws = torch.empty(dk.dckv_bytes_postrope(plan, T), dtype=torch.uint8, device="cuda:0")
    dk.dckv_encode_postrope(plan, gu.rows_dev(post), gu.to_dev(tok.astype(np.int32)), buf, nb, stt, ws)
    torch.cuda.synchronize()
    assert int(stt.item()) == 0
    want = buf[:int(nb.item())].cpu().numpy().tobytes()
    table, n_blocks = _layout(T, bs, extra=3, seed=91 + T)
    cache, _ = _dev_cache(_pools_from_rows(post, T, bs, table, n_blocks), table, bs, n_blocks)
    got, st = _encode_paged(plan, cache, True, tok)
    gu.say("%s: post-RoPE paged encode equal %s" % (case, got == want))
    assert st == 0 and got == want


def test_paged_block_table_out_of_range():
    rows, tok, g = _request("T389")
    T, bs = len(tok), 16
    plan = gu.device_codec().plan(g)
    table, n_blocks = _layout(T, bs, extra=2, seed=5)
    for bad in (n_blocks, -1):
        t2 = table.copy()
        t2[len(t2) // 2] = bad
        cache, _ = _dev_cache(_pools_from_rows(rows, T, bs, table, n_blocks), t2, bs, n_blocks)
        data, st = _encode_paged(plan, cache, False, tok)
        assert st == gu.dk().EINVAL and len(data) == 0
    data, st = gu.gpu_encode(plan, rows, tok)
    assert st == 0
    t2 = table.copy()
    t2[0] = n_blocks + 3
    empty = np.full((12, n_blocks * bs, 2, 256), SENTINEL, np.uint16)
    cache, tens = _dev_cache(empty, t2, bs, n_blocks)
    assert _decode_paged(plan, data, tok, cache) == gu.dk().EINVAL
    assert np.array_equal(_pools_back(tens), empty)  # nothing written


def test_paged_argument_errors():
    import torch
    dk = gu.dk()
    rows, tok, g = _request("T100")
    plan = gu.device_codec().plan(g)
    table, n_blocks = _layout(len(tok), 16, extra=0, seed=1)
    cache, _ = _dev_cache(_pools_from_rows(rows, len(tok), 16, table, n_blocks), table, 16, n_blocks)
    cache.block_size = 0
    with pytest.raises(dk.DckvError) as e:
        _encode_paged(plan, cache, False, tok)
    assert e.value.code == dk.EINVAL
