"""C ABI checks that need no GPU: exported symbols and the host plan tables."""
from __future__ import annotations

import os
import re

import numpy as np
import pytest

import dckv_synth as synth
from oracle import plan as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    import learned_kv_cache_dckv_amd as dk
    return dk


def test_library_exports_every_declared_symbol():
    dk = _lib()
    header = open(os.path.join(ROOT, "include", "dckv.h")).read()
    body = re.sub(r"/\*.*?\*/", "", header, flags=re.S)
    declared = set(re.findall(r"\b(dckv_[a-z_]+)\s*\(", body))
    assert declared == set(dk.EXPORTS)
    for name in declared:
        assert hasattr(dk.lib(), name)


def _compare(base, scale, g):
    dk = _lib()
    got = dk.dckv_plan_tables(base, scale, g)
    want = P.make_plan(np.float32(g), base, scale)
    assert np.array_equal(got["step"].view(np.uint32), want.step.view(np.uint32))
    assert np.array_equal(got["active"], want.active)
    assert got["c_active"] == want.c_active
    assert np.array_equal(got["freq"].astype(np.int64), want.freq)
    assert got["crc"] == want.crc


@pytest.mark.parametrize("rate", list(synth.RATE_TARGETS))
def test_plan_tables_bit_exact_for_workload_rates(rate):
    w = synth.world()
    _compare(w.base_step, w.laplace_scale, synth.step_scale_for(rate))


def test_plan_tables_bit_exact_random_and_edges():
    rng = np.random.default_rng(0)
    for trial in range(20):
        n = int(rng.integers(1, 300))
        base = rng.uniform(0.2, 3.0, n).astype(np.float32)
        scale = (10.0 ** rng.uniform(-4, 1, n)).astype(np.float32)
        _compare(base, scale, float(10.0 ** rng.uniform(-3, 0.5)))
    # exactly at the drop threshold, all dropped, none dropped
    base = np.ones(4, np.float32)
    _compare(base, np.array([0.025, 0.0249999, 1.0, 0.0], np.float32), 0.5)
    _compare(base, np.zeros(4, np.float32), 0.5)
    _compare(base, np.full(4, 1e4, np.float32), 1e-3)


def test_plan_tables_rejects_bad_input():
    dk = _lib()
    with pytest.raises(dk.DckvError):
        dk.dckv_plan_tables(np.ones(3, np.float32), np.ones(3, np.float32), 0.0)
    with pytest.raises(dk.DckvError):
        dk.dckv_plan_tables(np.array([1.0, -1.0], np.float32), np.ones(2, np.float32), 0.1)
    with pytest.raises(dk.DckvError):
        dk.dckv_plan_tables(np.ones(2, np.float32), np.array([1.0, np.nan], np.float32), 0.1)


def test_fit_workspace_size_and_bounds():
    dk = _lib()
    with pytest.raises(dk.DckvError):
        dk.dckv_fit_bytes(1)
    with pytest.raises(dk.DckvError):
        dk.dckv_fit_bytes((1 << 18) + 1)
    # per row: fp32 coefficients and means (16 KiB), two bf16 halves of the
    # coefficients and the gathered embeddings (12 KiB), the checked id; fixed:
    # Gram and right-hand sides (32 MiB), bf16 head (8 MiB), partial sums,
    # (512 row chunks), the diagonal, the inverses of the 32 diagonal blocks
    n = 4096
    got = dk.dckv_fit_bytes(n)
    per_row = 2048 * 4 * 2 + 2048 * 2 * 3 + 4
    fixed = 2048 * 2048 * 4 * 2 + 2048 * 2048 * 2 + 512 * 2 * 2048 * 8 + 2048 * 4 + 32 * 64 * 64 * 4
    assert fixed + per_row * n <= got <= fixed + per_row * n + 12 * 256


def test_plan_rejects_vocab_beyond_32bit_mean_table_offsets():
    """A vocabulary of 2^19 rows would make the mean table 4 GiB, past the
    encoder's 32-bit offsets: the plan refuses it before touching a device."""
    import ctypes
    dk = _lib()
    n = 2048
    vec = np.ones(n, np.float32)
    for vocab, want in ((1 << 19, dk.EUNSUPPORTED), ((1 << 19) + 7, dk.EUNSUPPORTED)):
        prm = dk._Params(6, 2, 256, n, 256, 2048, vocab, 4, 128, 1e7,
                         8, 8, 8, 8, 8, 8, vec.ctypes.data, vec.ctypes.data, vec.ctypes.data)
        h = ctypes.c_void_p()
        rc = dk.lib().dckv_plan(ctypes.byref(prm), 0.1, ctypes.byref(h))
        assert rc == want and not h.value
        assert "vocab" in dk.dckv_last_error()
