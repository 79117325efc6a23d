"""Byte-stream layout of one encoded request (writer and validating parser).

The pages define no format (the DCKV digest only says the payload is "stored"
and compares it with the code length the models predict, "Evidence"); this
layout is the project's own, version 1.  All fields are little endian and the
sections follow each other without padding:

  offset 0   "DCKV", u16 version = 1, u16 header_bytes = 64
  offset 8   u32 T, keep_head, keep_tail, N, n_coef, C_a, n_groups, n_esc
  offset 40  f32 step_scale, u32 plan_crc
  offset 48  u64 total_bytes, u64 rans_bytes
  offset 64  kept rows: bf16 pre-RoPE rows of the kept positions, in position
             order, (T - N) * D values
  then       u32 group_offset[n_groups + 1]: byte offsets into the rANS
             section, [0] = 0 and [n_groups] = rans_bytes, non-decreasing
  then       n_esc escape records {u32 flat = j*C_a + rank, i32 code},
             strictly ascending flat
  then       the rANS section: group id = b*G + g in order, each a sequence of
             u16 words
"""
from __future__ import annotations

import struct
from dataclasses import dataclass

import numpy as np

MAGIC = b"DCKV"
VERSION = 1
HEADER_BYTES = 64
_HDR = struct.Struct("<4sHHIIIIIIIIfIQQ")
assert _HDR.size == HEADER_BYTES


class StreamError(ValueError):
    """Malformed stream (maps to a corrupt-stream status)."""


class PlanMismatch(ValueError):
    """Stream was written under another plan (maps to a plan-mismatch status)."""


@dataclass
class Header:
    T: int
    keep_head: int
    keep_tail: int
    N: int
    n_coef: int
    c_active: int
    n_groups: int
    n_esc: int
    step_scale: float
    plan_crc: int
    total_bytes: int
    rans_bytes: int


def write(h: Header, kept_rows: np.ndarray, group_words: list, esc_flat: np.ndarray,
          esc_q: np.ndarray) -> bytes:
    lens = np.array([2 * len(w) for w in group_words], dtype=np.int64)
    offs = np.zeros(len(group_words) + 1, dtype=np.int64)
    offs[1:] = np.cumsum(lens)
    rans = b"".join(np.asarray(w, dtype="<u2").tobytes() for w in group_words)
    kept = np.ascontiguousarray(kept_rows, dtype="<u2").tobytes()
    esc = np.empty(len(esc_flat), dtype=[("flat", "<u4"), ("q", "<i4")])
    esc["flat"] = esc_flat
    esc["q"] = esc_q
    body = kept + offs.astype("<u4").tobytes() + esc.tobytes() + rans
    total = HEADER_BYTES + len(body)
    hdr = _HDR.pack(MAGIC, VERSION, HEADER_BYTES, h.T, h.keep_head, h.keep_tail, h.N, h.n_coef,
                    h.c_active, len(group_words), len(esc_flat), float(np.float32(h.step_scale)),
                    h.plan_crc, total, len(rans))
    return hdr + body


def header(buf: bytes) -> Header:
    if len(buf) < HEADER_BYTES:
        raise StreamError("stream shorter than its header")
    (magic, ver, hb, T, kh, kt, N, nc, ca, ng, ne, g, crc, total, rb) = _HDR.unpack_from(buf, 0)
    if magic != MAGIC or ver != VERSION or hb != HEADER_BYTES:
        raise StreamError("bad magic/version")
    return Header(T, kh, kt, N, nc, ca, ng, ne, g, crc, total, rb)


def parse(buf: bytes, D: int):
    """Split a stream into its sections, checking every size and offset."""
    h = header(buf)
    n_kept = h.T - h.N
    if h.N > h.T or n_kept < 0:
        raise StreamError("N > T")
    pos = HEADER_BYTES
    kept_end = pos + n_kept * D * 2
    offs_end = kept_end + 4 * (h.n_groups + 1)
    esc_end = offs_end + 8 * h.n_esc
    if h.total_bytes != len(buf) or esc_end + h.rans_bytes != h.total_bytes:
        raise StreamError("section sizes do not add up")
    kept = np.frombuffer(buf, dtype="<u2", count=n_kept * D, offset=pos).reshape(n_kept, D)
    offs = np.frombuffer(buf, dtype="<u4", count=h.n_groups + 1, offset=kept_end).astype(np.int64)
    if offs[0] != 0 or offs[-1] != h.rans_bytes or np.any(np.diff(offs) < 0) or np.any(offs % 2):
        raise StreamError("bad group offsets")
    esc = np.frombuffer(buf, dtype=[("flat", "<u4"), ("q", "<i4")], count=h.n_esc, offset=offs_end)
    flat = esc["flat"].astype(np.int64)
    q = esc["q"].astype(np.int64)
    if h.n_esc and (np.any(np.diff(flat) <= 0) or flat[-1] >= h.N * h.c_active):
        raise StreamError("bad escape records")
    words_all = np.frombuffer(buf, dtype="<u2", count=h.rans_bytes // 2, offset=esc_end)
    groups = [words_all[offs[i] // 2: offs[i + 1] // 2] for i in range(h.n_groups)]
    return h, kept, flat, q, groups
