"""Shared helpers of the GPU parity tests (device setup, oracle runs)."""
from __future__ import annotations

import copy
import functools
import sys

import numpy as np

import dckv_synth as synth
from oracle import bf16, codec as ocodec, plan as oplan, rans as orans, stream as ostream

REL_L2_TOL = 2e-3          # float stages: coefficients and reconstructed rows
SYMBOL_AGREEMENT = 0.99999  # integer symbols of the lossy stage


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=None)
def dk():
    import learned_kv_cache_dckv_amd as m
    return m


@functools.lru_cache(maxsize=None)
def device_codec():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return dk().Codec(synth.world().params(), device="cuda:0")


def codec_with_scales(laplace_scale: np.ndarray):
    """Same device weights, other Laplace scales (to force dropped components)."""
    c = copy.copy(device_codec())
    c.laplace_scale = np.ascontiguousarray(laplace_scale, dtype=np.float32)
    return c


def params_with_scales(laplace_scale: np.ndarray) -> dict:
    p = dict(synth.world().params())
    p["laplace_scale"] = np.ascontiguousarray(laplace_scale, dtype=np.float32)
    return p


def oracle_plan(params: dict, g: float):
    return oplan.make_plan(np.float32(g), params["base_step"], params["laplace_scale"])


def to_dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to("cuda:0")


def rows_dev(rows_bits: np.ndarray):
    import torch
    return to_dev(rows_bits.view(np.int16)).view(torch.bfloat16)


def gpu_encode(plan, rows_bits, tok):
    import torch
    s, st = dk().encode(plan, rows_dev(rows_bits), to_dev(tok.astype(np.int32)))
    torch.cuda.synchronize()
    return s.cpu().numpy().tobytes(), st


def gpu_decode(plan, data: bytes, tok, ws=None):
    import torch
    buf = to_dev(np.frombuffer(data, dtype=np.uint8).copy()) if len(data) else torch.zeros(64, dtype=torch.uint8,
                                                                                          device="cuda:0")
    out, st = dk().decode(plan, buf[:len(data)] if len(data) else buf[:0], to_dev(tok.astype(np.int32)), ws=ws)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16), st


def read_view(ws, plan, T, which):
    """Bytes of one workspace view (after a call that filled it)."""
    off, nb, rs = dk().dckv_workspace_view(plan, T, which)
    return ws[off:off + nb].cpu().numpy(), rs


def tiled_symbols(buf: np.ndarray, N: int, Ca: int) -> np.ndarray:
    """Group-tiled symbol bytes -> [N][C_a]."""
    N256 = (N + 255) // 256 * 256
    G = (Ca + 63) // 64
    t = buf[:G * N256 * 64].reshape(G, N256 // 4, 64, 4)  # [g][quad][lane][row-in-quad]
    full = t.transpose(1, 3, 0, 2).reshape(N256, G * 64)
    return full[:N, :Ca]


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / den) if den > 0 else float(np.linalg.norm(a - b))


def oracle_symbols_of_stream(data: bytes, params: dict, p, T: int):
    """Parse a stream and rANS-decode it with the oracle (validates the format)."""
    h, kept, flat, qe, groups = ostream.parse(data, synth.D)
    ocodec.check_header(h, T, params, p)
    esc = np.zeros((h.N, p.c_active), dtype=bool)
    if len(flat):
        esc.reshape(-1)[flat] = True
    sym = orans.decode_all(groups, p.freq, p.cum, h.N, esc) if h.N and p.c_active else \
        np.full((h.N, p.c_active), 255, np.uint8)
    return h, sym, flat, qe, groups


def oracle_stream_from_symbols(rows, T, params, p, sym, flat, qe) -> bytes:
    sh = ocodec.shape_of(params)
    N, kept_t, _ = ocodec.split_positions(T, sh.keep_head, sh.keep_tail)
    groups = orans.encode_all(sym, p.freq, p.cum) if N and p.c_active else []
    n_blk, G, _, _ = orans.group_shape(N, p.c_active)
    h = ostream.Header(T=T, keep_head=sh.keep_head, keep_tail=sh.keep_tail, N=N, n_coef=p.step.size,
                       c_active=p.c_active, n_groups=n_blk * G, n_esc=len(flat), step_scale=float(p.step_scale),
                       plan_crc=p.crc, total_bytes=0, rans_bytes=0)
    return ostream.write(h, rows[kept_t], groups, flat, qe)
