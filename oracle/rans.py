"""Interleaved 32-bit rANS over (component, 256-token block) substreams.

Source: DCKV digest page, "How it works", Coding bullet (an asymmetric-numeral
coder over discretised-Laplace symbol models; a code outside [-127, 127] is
stored as a 64-bit record instead).
The pages fix neither the coder's parameters nor a byte format; the readings
taken here are:
  * state x is 32 bits, renormalisation moves 16-bit words, L = 2^16, table
    precision 15 bits (M = 2^15);
  * a substream is one active component over one block of up to 256 coded
    tokens; up to 64 substreams of one block (active ranks 64g .. 64g+63) are
    interleaved into one word sequence, a "group";
  * escaped positions carry no rANS symbol (their code travels in a 64-bit
    record of its own) and are skipped by both coder directions.

Encoder of a group with lanes l = 0..n-1 and tokens i = 0..L_b-1:
  every lane starts at x = L; tokens are taken from last to first and, inside
  a token, lanes from last to first; before coding symbol s with frequency f
  and cumulative frequency c a lane whose x >= f * 2^17 emits x mod 2^16 and
  shifts x right by 16; then x = (x div f) * M + (x mod f) + c.  Finally each
  lane, from last to first, emits x div 2^16 then x mod 2^16.  The group's
  words are the emitted sequence reversed.
Decoder: read x = w0 | w1 << 16 for each lane in order; then for tokens first
  to last and lanes first to last: slot = x mod M, s is the symbol with
  cum_s <= slot < cum_{s+1}, x = f_s * (x >> 15) + slot - cum_s, and while the
  state is below L it takes the next word: x = (x << 16) | w.  A valid group
  ends with every lane back at L and every word consumed.

Two implementations follow: a scalar one (plain loops, for small inputs and
exhaustive tests) and a lock-step one that runs all groups of a request at
once with numpy (for full-size requests).  They are cross-checked in tests.
"""
from __future__ import annotations

import numpy as np

from .plan import ESC, M, PREC_BITS

L = 1 << 16
BLOCK = 256
LANES = 64


class CorruptStream(ValueError):
    pass


# --------------------------------------------------------------------------
# scalar coder (one group)
# --------------------------------------------------------------------------
def encode_group(sym, freq, cum) -> list:
    """sym: [L_b][n] ints (255 = escaped/skip); freq [n][255]; cum [n][256]."""
    sym = [[int(v) for v in row] for row in sym]
    Lb = len(sym)
    n = len(freq)
    x = [L] * n
    pushed = []
    for i in range(Lb - 1, -1, -1):
        for l in range(n - 1, -1, -1):
            s = sym[i][l]
            if s == ESC:
                continue
            f = int(freq[l][s])
            c = int(cum[l][s])
            if x[l] >= (f << 17):
                pushed.append(x[l] & 0xFFFF)
                x[l] >>= 16
            x[l] = (x[l] // f) * M + (x[l] % f) + c
    for l in range(n - 1, -1, -1):
        pushed.append(x[l] >> 16)
        pushed.append(x[l] & 0xFFFF)
    pushed.reverse()
    return pushed


def decode_group(words, freq, cum, Lb: int, esc_mask=None):
    """Inverse of :func:`encode_group`; raises CorruptStream on a bad group."""
    n = len(freq)
    w = [int(v) for v in words]
    if len(w) < 2 * n:
        raise CorruptStream("group shorter than its flush")
    x = []
    ptr = 0
    for _ in range(n):
        x.append(w[ptr] | (w[ptr + 1] << 16))
        ptr += 2
    out = [[ESC] * n for _ in range(Lb)]
    for i in range(Lb):
        for l in range(n):
            if esc_mask is not None and esc_mask[i][l]:
                continue
            slot = x[l] & (M - 1)
            c = cum[l]
            s = 0
            while not (int(c[s]) <= slot < int(c[s + 1])):
                s += 1
            x[l] = int(freq[l][s]) * (x[l] >> PREC_BITS) + slot - int(c[s])
            if x[l] < L:
                if ptr >= len(w):
                    raise CorruptStream("group ran out of words")
                x[l] = (x[l] << 16) | w[ptr]
                ptr += 1
            out[i][l] = s
    if ptr != len(w) or any(v != L for v in x):
        raise CorruptStream("group end state check failed")
    return out


# --------------------------------------------------------------------------
# lock-step coder (all groups of a request)
# --------------------------------------------------------------------------
def group_shape(N: int, c_active: int):
    """Blocks, component groups, and per-group token count / lane count."""
    n_blk = (N + BLOCK - 1) // BLOCK
    G = (c_active + LANES - 1) // LANES
    Lb = np.array([min(BLOCK, N - BLOCK * b) for b in range(n_blk)], dtype=np.int64)
    nl = np.array([min(LANES, c_active - LANES * g) for g in range(G)], dtype=np.int64)
    return n_blk, G, Lb, nl


def encode_all(sym: np.ndarray, freq: np.ndarray, cum: np.ndarray):
    """Encode every group of a request.

    sym: uint8 [N][C_a] (255 = escaped).  Returns a list of uint16 arrays, one
    per group, in group order id = b*G + g.
    """
    N, Ca = sym.shape
    n_blk, G, Lb, nl = group_shape(N, Ca)
    ng = n_blk * G
    if ng == 0:
        return []
    lane = np.arange(LANES)
    b_of = np.repeat(np.arange(n_blk), G)
    g_of = np.tile(np.arange(G), n_blk)
    comp = g_of[:, None] * LANES + lane[None, :]          # rank of each lane
    lane_ok = lane[None, :] < nl[g_of][:, None]
    compc = np.minimum(comp, max(Ca - 1, 0))
    x = np.full((ng, LANES), L, dtype=np.uint64)
    cap = LANES * (BLOCK + 2)
    out = np.zeros((ng, cap), dtype=np.uint16)
    cnt = np.zeros(ng, dtype=np.int64)
    rows = np.arange(ng)
    for i in range(BLOCK - 1, -1, -1):
        tok_ok = i < Lb[b_of]
        if not tok_ok.any():
            continue
        j = np.minimum(b_of * BLOCK + i, N - 1)
        s = sym[j[:, None], compc].astype(np.int64)
        act = lane_ok & tok_ok[:, None] & (s != 255)
        sc = np.where(act, s, 0)
        f = freq[compc, sc].astype(np.uint64)
        c = cum[compc, sc].astype(np.uint64)
        emit = act & (x >= (f << np.uint64(17)))
        # descending-lane push order: lanes above l that emit come first
        above = np.cumsum(emit[:, ::-1], axis=1)[:, ::-1] - emit
        pos = cnt[:, None] + above
        r_e, l_e = np.nonzero(emit)
        out[r_e, pos[r_e, l_e]] = (x[r_e, l_e] & np.uint64(0xFFFF)).astype(np.uint16)
        cnt += emit.sum(axis=1)
        x = np.where(emit, x >> np.uint64(16), x)
        fa = np.where(act, f, np.uint64(1))
        xn = (x // fa) * np.uint64(M) + (x % fa) + c
        x = np.where(act, xn, x)
    # flush, lanes descending: high word then low word
    ln = nl[g_of]
    res = []
    for r in range(ng):
        n = int(ln[r])
        k = int(cnt[r])
        seq = out[r, :k].tolist()
        for l in range(n - 1, -1, -1):
            seq.append(int(x[r, l]) >> 16)
            seq.append(int(x[r, l]) & 0xFFFF)
        seq.reverse()
        res.append(np.array(seq, dtype=np.uint16))
    return res


def slot_lut(cum: np.ndarray) -> np.ndarray:
    """Per-component slot -> symbol table (uint8 [C_a][M])."""
    Ca = cum.shape[0]
    lut = np.zeros((Ca, M), dtype=np.uint8)
    for r in range(Ca):
        lut[r] = np.repeat(np.arange(255, dtype=np.uint8), np.diff(cum[r]))
    return lut


def decode_all(words: list, freq: np.ndarray, cum: np.ndarray, N: int, esc_mask: np.ndarray | None = None):
    """Decode every group; returns uint8 [N][C_a] (255 at escaped positions).

    words: list of uint16 arrays in group order.  esc_mask: bool [N][C_a].
    Raises CorruptStream if any group fails its end-state check.
    """
    Ca = freq.shape[0]
    n_blk, G, Lb, nl = group_shape(N, Ca)
    ng = n_blk * G
    sym = np.full((N, Ca), 255, dtype=np.uint8)
    if ng == 0:
        return sym
    lut = slot_lut(cum)
    lens = np.array([len(w) for w in words], dtype=np.int64)
    off = np.zeros(ng + 1, dtype=np.int64)
    off[1:] = np.cumsum(lens)
    flat = np.concatenate([np.asarray(w, dtype=np.uint64) for w in words] + [np.zeros(1, np.uint64)])
    lane = np.arange(LANES)
    b_of = np.repeat(np.arange(n_blk), G)
    g_of = np.tile(np.arange(G), n_blk)
    comp = g_of[:, None] * LANES + lane[None, :]
    ln = nl[g_of]
    lane_ok = lane[None, :] < ln[:, None]
    if np.any(lens < 2 * ln):
        raise CorruptStream("group shorter than its flush")
    compc = np.minimum(comp, Ca - 1)
    base = off[:-1]
    ptr = 2 * ln.copy()
    lo = flat[np.minimum(base[:, None] + 2 * lane[None, :], flat.size - 1)]
    hi = flat[np.minimum(base[:, None] + 2 * lane[None, :] + 1, flat.size - 1)]
    x = np.where(lane_ok, lo | (hi << np.uint64(16)), np.uint64(L))
    for i in range(BLOCK):
        tok_ok = i < Lb[b_of]
        if not tok_ok.any():
            break
        j = np.minimum(b_of * BLOCK + i, N - 1)
        act = lane_ok & tok_ok[:, None]
        if esc_mask is not None:
            act &= ~esc_mask[j[:, None], compc]
        slot = (x & np.uint64(M - 1)).astype(np.int64)
        s = lut[compc, slot].astype(np.int64)
        f = freq[compc, s].astype(np.uint64)
        c = cum[compc, s].astype(np.uint64)
        xn = f * (x >> np.uint64(PREC_BITS)) + slot.astype(np.uint64) - c
        need = act & (xn < np.uint64(L))
        below = np.cumsum(need, axis=1) - need
        idx = ptr[:, None] + below
        over = need & (idx >= lens[:, None])
        if over.any():
            raise CorruptStream("group ran out of words")
        w = flat[np.minimum(base[:, None] + idx, flat.size - 1)]
        xn = np.where(need, (xn << np.uint64(16)) | w, xn)
        x = np.where(act, xn, x)
        ptr += need.sum(axis=1)
        r_a, l_a = np.nonzero(act)
        sym[j[r_a], comp[r_a, l_a]] = s[r_a, l_a]
    if np.any(ptr != lens) or np.any(np.where(lane_ok, x, np.uint64(L)) != np.uint64(L)):
        raise CorruptStream("group end state check failed")
    return sym
