"""DCKV prompt-KV-cache codec for AMD Instinct MI355X (gfx950).

A thin ctypes binding of ``libdckv.so``: every function here only marshals
arguments for the C ABI declared in ``include/dckv.h``; every step of encode
and decode runs in the library's HIP kernels.  PyTorch provides device memory
and the current HIP stream.

The library must be built first (``python learned_kv_cache_dckv_amd/build.py``);
importing this package without it raises ImportError.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdckv.so")

OK, EINVAL, ENOMEM, ECAPACITY, ECORRUPT, EPLAN, EHIP, EUNSUPPORTED = 0, -1, -2, -3, -4, -5, -6, -7
STATUS_NAMES = {0: "OK", -1: "EINVAL", -2: "ENOMEM", -3: "ECAPACITY", -4: "ECORRUPT", -5: "EPLAN",
                -6: "EHIP", -7: "EUNSUPPORTED"}
VIEW_SYMBOLS, VIEW_YHAT_B, VIEW_H_B = 0, 1, 2

# every symbol include/dckv.h declares
EXPORTS = ("dckv_plan_tables", "dckv_plan", "dckv_plan_free", "dckv_plan_info", "dckv_plan_mean_table",
           "dckv_plan_memory",
           "dckv_bytes", "dckv_encode", "dckv_encode_noalloc", "dckv_bytes_postrope", "dckv_encode_postrope",
           "dckv_decode", "dckv_decode_heads", "dckv_unrope", "dckv_bytes_paged", "dckv_encode_paged",
           "dckv_decode_paged", "dckv_bytes_batch", "dckv_encode_batch", "dckv_decode_batch", "dckv_entropy_encode",
           "dckv_entropy_decode", "dckv_workspace_view", "dckv_profile_enable", "dckv_profile_only", "dckv_profile_reset",
           "dckv_profile_read", "dckv_fit_bytes", "dckv_fit", "dckv_rate_bytes", "dckv_rate_forward",
           "dckv_rate_backward_bytes", "dckv_rate_backward", "dckv_last_error")


class DckvError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("%s (%d): %s" % (STATUS_NAMES.get(code, "?"), code, msg))
        self.code = code


class _Params(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("n_coef", ctypes.c_int32), ("n_hidden", ctypes.c_int32), ("emb_dim", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("keep_head", ctypes.c_int32), ("keep_tail", ctypes.c_int32),
                ("rope_theta", ctypes.c_float),
                ("analysis", ctypes.c_void_p), ("synthesis", ctypes.c_void_p), ("w1", ctypes.c_void_p),
                ("w2", ctypes.c_void_p), ("embedding", ctypes.c_void_p), ("mean_head", ctypes.c_void_p),
                ("nbr_weight", ctypes.c_void_p), ("laplace_scale", ctypes.c_void_p),
                ("base_step", ctypes.c_void_p)]


class _PagedKV(ctypes.Structure):
    _fields_ = [("kv", ctypes.c_void_p * 12), ("block_table", ctypes.c_void_p), ("block_size", ctypes.c_int32),
                ("n_blocks", ctypes.c_int64)]


class _Req(ctypes.Structure):
    """One request of a batch call (struct dckv_req)."""
    _fields_ = [("plan", ctypes.c_void_p), ("rows", ctypes.c_void_p), ("token_ids", ctypes.c_void_p),
                ("T", ctypes.c_int64), ("stream", ctypes.c_void_p), ("capacity", ctypes.c_uint64),
                ("stream_bytes", ctypes.c_void_p), ("rows_out", ctypes.c_void_p), ("status", ctypes.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libdckv.so is not built: run `python learned_kv_cache_dckv_amd/build.py` "
                          "(expected at %s)" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, U64, I64, I32, U32, F = (ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32,
                                ctypes.c_uint32, ctypes.c_float)
    sig = {
        "dckv_plan_tables": [P, P, I32, F, P, P, P, P, P],
        "dckv_plan": [P, F, P],
        "dckv_plan_free": [P],
        "dckv_plan_info": [P, P, P, P, P, P],
        "dckv_plan_mean_table": [P, P, P, P],
        "dckv_plan_memory": [P, P, P, P],
        "dckv_bytes": [P, I64, P, P],
        "dckv_encode": [P, P, P, I64, P, U64, P, P, P, U64, P],
        "dckv_encode_noalloc": [P, P, P, I64, P, U64, P, P, P],
        "dckv_bytes_postrope": [P, I64, P],
        "dckv_encode_postrope": [P, P, P, I64, P, U64, P, P, P, U64, P],
        "dckv_decode": [P, P, U64, P, I64, P, P, P, U64, P],
        "dckv_decode_heads": [P, P, U64, P, I64, P, P, P, U64, P],
        "dckv_unrope": [P, P, I64, P, P],
        "dckv_bytes_paged": [P, I64, P],
        "dckv_encode_paged": [P, P, I32, P, I64, P, U64, P, P, P, U64, P],
        "dckv_decode_paged": [P, P, U64, P, I64, P, P, P, U64, P],
        "dckv_bytes_batch": [P, I32, P],
        "dckv_encode_batch": [P, I32, P, U64, P],
        "dckv_decode_batch": [P, I32, P, U64, P],
        "dckv_entropy_encode": [P, I64, P, P, U32, P, P, U64, P, P, P, U64, P],
        "dckv_entropy_decode": [P, P, U64, I64, P, P, P, P, U64, P],
        "dckv_workspace_view": [P, I64, I32, P, P, P],
        "dckv_profile_enable": [I32],
        "dckv_profile_only": [ctypes.c_char_p],
        "dckv_profile_reset": [],
        "dckv_profile_read": [ctypes.c_char_p, P, P],
        "dckv_fit_bytes": [I64, P],
        "dckv_fit": [P, P, P, I64, F, P, P, P, P, P, P, U64, P],
        "dckv_rate_bytes": [P, I64, P],
        "dckv_rate_forward": [P, P, P, I64, P, P, P, P, P, P, P, P, P, U64, P],
        "dckv_rate_backward_bytes": [P, I64, P],
        "dckv_rate_backward": [P, P, P, I64, P, P, P, P, P, P, U64, P],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.dckv_last_error.argtypes = []
    lib.dckv_last_error.restype = ctypes.c_char_p
    return lib


_lib = _load()


def lib():
    return _lib


def dckv_last_error() -> str:
    return (_lib.dckv_last_error() or b"").decode()


def _check(rc: int):
    if rc != 0:
        raise DckvError(rc, dckv_last_error())


def _ptr(x) -> int:
    """Address of a torch tensor (device) or numpy array (host); None -> 0."""
    if x is None:
        return 0
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    return x.data_ptr()


def _stream_handle(stream=None) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _as_bits(t):
    """bf16 tensor or int16/uint16 bit tensor -> int16 tensor view of the bits."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16)
    if t.dtype in (torch.int16, torch.uint16):
        return t.view(torch.int16)
    raise TypeError("expected bf16 data as torch.bfloat16 or 16-bit integer bits, got %s" % t.dtype)


# ---------------------------------------------------------------------------
# plan
# ---------------------------------------------------------------------------
def dckv_plan_tables(base_step, laplace_scale, step_scale: float):
    """Host-only plan tables: dict(step, active, freq[C_a][255], c_active, crc)."""
    bs = np.ascontiguousarray(base_step, dtype=np.float32)
    ls = np.ascontiguousarray(laplace_scale, dtype=np.float32)
    n = bs.size
    step = np.empty(n, np.float32)
    active = np.empty(n, np.uint8)
    freq = np.empty((n, 255), np.uint16)
    ca = ctypes.c_int32()
    crc = ctypes.c_uint32()
    _check(_lib.dckv_plan_tables(_ptr(bs), _ptr(ls), n, float(step_scale), _ptr(step), _ptr(active), _ptr(freq),
                                 ctypes.byref(ca), ctypes.byref(crc)))
    return dict(step=step, active=active.astype(bool), freq=freq[:ca.value].copy(), c_active=ca.value,
                crc=crc.value)


class Codec:
    """Codec parameters resident in device memory (bf16 matrices as bit tensors)."""

    def __init__(self, params: dict, device="cuda"):
        import torch
        self.device = torch.device(device)

        def dev(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(self.device)

        self.analysis = dev(params["analysis"])
        self.synthesis = dev(params["synthesis"])
        # without w1 / w2: the linear codec (no correction on the synthesis side)
        self.linear = params.get("w1") is None
        self.w1 = None if self.linear else dev(params["w1"])
        self.w2 = None if self.linear else dev(params["w2"])
        self.embedding = dev(params["embedding"])
        self.mean_head = dev(params["mean_head"])
        self.nbr_weight = np.ascontiguousarray(params["nbr_weight"], dtype=np.float32)
        self.laplace_scale = np.ascontiguousarray(params["laplace_scale"], dtype=np.float32)
        self.base_step = np.ascontiguousarray(params["base_step"], dtype=np.float32)
        self.shape = dict(n_layers=params.get("n_layers", 6), n_kv_heads=params.get("n_kv_heads", 2),
                          head_dim=params.get("head_dim", 256), keep_head=params.get("keep_head", 4),
                          keep_tail=params.get("keep_tail", 128), rope_theta=params.get("rope_theta", 1e7))
        self.n_coef = self.analysis.shape[0]
        self.D = self.analysis.shape[1]
        self.n_hidden = 256 if self.linear else self.w1.shape[0]
        self.vocab, self.emb_dim = self.embedding.shape

    def c_params(self) -> _Params:
        s = self.shape
        return _Params(s["n_layers"], s["n_kv_heads"], s["head_dim"], self.n_coef, self.n_hidden, self.emb_dim,
                       self.vocab, s["keep_head"], s["keep_tail"], float(s["rope_theta"]),
                       _ptr(self.analysis), _ptr(self.synthesis), _ptr(self.w1), _ptr(self.w2),
                       _ptr(self.embedding), _ptr(self.mean_head), _ptr(self.nbr_weight),
                       _ptr(self.laplace_scale), _ptr(self.base_step))

    def plan(self, step_scale: float) -> "Plan":
        return dckv_plan(self, step_scale)


class Plan:
    def __init__(self, handle: int, codec: Codec, step_scale: float):
        self.handle = handle
        self.codec = codec
        self.step_scale = float(np.float32(step_scale))
        info = dckv_plan_info(self)
        self.c_active = info["c_active"]
        self.crc = info["crc"]

    def free(self):
        if self.handle:
            dckv_plan_free(self)

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass

    def bytes(self, T: int):
        return dckv_bytes(self, T)


def dckv_plan(codec: Codec, step_scale: float) -> Plan:
    prm = codec.c_params()
    h = ctypes.c_void_p()
    _check(_lib.dckv_plan(ctypes.byref(prm), float(step_scale), ctypes.byref(h)))
    return Plan(h.value, codec, step_scale)


def dckv_plan_free(plan: Plan):
    h, plan.handle = plan.handle, 0
    _check(_lib.dckv_plan_free(h))


def dckv_plan_info(plan: Plan) -> dict:
    n = plan.codec.n_coef
    step = np.empty(n, np.float32)
    active = np.empty(n, np.uint8)
    ca = ctypes.c_int32()
    crc = ctypes.c_uint32()
    _check(_lib.dckv_plan_info(plan.handle, _ptr(step), _ptr(active), 0, ctypes.byref(ca), ctypes.byref(crc)))
    freq = np.empty((max(ca.value, 1), 255), np.uint16)
    _check(_lib.dckv_plan_info(plan.handle, 0, 0, _ptr(freq), None, None))
    return dict(step=step, active=active.astype(bool), freq=freq[:ca.value], c_active=ca.value, crc=crc.value)


def dckv_plan_memory(plan: Plan) -> dict:
    """Device bytes the plan holds and how many plans share its mean table."""
    tb, mb, users = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_int32()
    _check(_lib.dckv_plan_memory(plan.handle, ctypes.byref(tb), ctypes.byref(mb), ctypes.byref(users)))
    return dict(table_bytes=tb.value, mean_table_bytes=mb.value, mean_table_users=users.value)


def dckv_plan_mean_table(plan: Plan):
    """(device address of the table, rows, col_component[n_coef]): the plan's
    embedding-mean table, fp32 [rows][n_coef]."""
    tab = ctypes.c_void_p()
    rows = ctypes.c_int64()
    cols = np.empty(plan.codec.n_coef, np.int32)
    _check(_lib.dckv_plan_mean_table(plan.handle, ctypes.byref(tab), ctypes.byref(rows), _ptr(cols)))
    return tab.value or 0, rows.value, cols


class _DeviceArray:
    """A device address with shape and dtype, for torch.as_tensor (no copy)."""

    def __init__(self, addr: int, shape, typestr: str):
        self.__cuda_array_interface__ = {"shape": tuple(shape), "typestr": typestr, "data": (int(addr), False),
                                         "version": 2, "strides": None}


def mean_table(plan: Plan):
    """The plan's embedding-mean table as a torch float32 tensor [vocab][n_coef]
    sharing the plan's memory (read only; valid while the plan lives), and
    col_component: the component of each column."""
    import torch
    addr, rows, cols = dckv_plan_mean_table(plan)
    t = torch.as_tensor(_DeviceArray(addr, (rows, plan.codec.n_coef), "<f4"), device=plan.codec.device)
    return t, cols


def dckv_bytes(plan: Plan, T: int):
    """(max stream bytes, workspace bytes) for a request of T tokens."""
    ms = ctypes.c_uint64()
    ws = ctypes.c_uint64()
    _check(_lib.dckv_bytes(plan.handle, int(T), ctypes.byref(ms), ctypes.byref(ws)))
    return ms.value, ws.value


def workspace(plan: Plan, T: int):
    import torch
    _, ws = dckv_bytes(plan, T)
    return torch.empty(max(ws, 256), dtype=torch.uint8, device=plan.codec.device)


# ---------------------------------------------------------------------------
# encode / decode
# ---------------------------------------------------------------------------
def dckv_encode(plan: Plan, rows, token_ids, stream_buf, stream_bytes, status, ws, stream=None):
    """Enqueue an encode.  rows [T][D] bf16 (device), token_ids [T] int32,
    stream_buf uint8 [capacity], stream_bytes int64 [1], status int32 [1]."""
    T = int(rows.shape[0])
    rows = _as_bits(rows)
    _check(_lib.dckv_encode(plan.handle, _ptr(rows), _ptr(token_ids), T, _ptr(stream_buf), stream_buf.numel(),
                            _ptr(stream_bytes), _ptr(status), _ptr(ws), ws.numel(), _stream_handle(stream)))


def dckv_encode_noalloc(plan: Plan, rows, token_ids, stream_buf, stream_bytes, status, stream=None):
    """Enqueue an encode that uses the library's own static scratch instead of a
    workspace (requests up to 8,192 positions)."""
    T = int(rows.shape[0])
    rows = _as_bits(rows)
    _check(_lib.dckv_encode_noalloc(plan.handle, _ptr(rows), _ptr(token_ids), T, _ptr(stream_buf),
                                    stream_buf.numel(), _ptr(stream_bytes), _ptr(status), _stream_handle(stream)))


def dckv_bytes_postrope(plan: Plan, T: int) -> int:
    """Workspace bytes of dckv_encode_postrope for a request of T tokens."""
    v = ctypes.c_uint64()
    _check(_lib.dckv_bytes_postrope(plan.handle, int(T), ctypes.byref(v)))
    return v.value


def dckv_encode_postrope(plan: Plan, rows, token_ids, stream_buf, stream_bytes, status, ws, stream=None):
    """Enqueue an encode of post-RoPE rows [T][D] (keys rotated back inside)."""
    T = int(rows.shape[0])
    rows = _as_bits(rows)
    _check(_lib.dckv_encode_postrope(plan.handle, _ptr(rows), _ptr(token_ids), T, _ptr(stream_buf),
                                     stream_buf.numel(), _ptr(stream_bytes), _ptr(status), _ptr(ws), ws.numel(),
                                     _stream_handle(stream)))


class PagedKV:
    """A paged attention cache: pools[2 l + kv] (layer l, kv = 0 keys, 1 values) are device
    tensors [n_blocks][block_size][n_kv_heads][head_dim] (bf16 or int16 bits); block_table is
    a device int32 tensor of the request's physical blocks."""

    def __init__(self, pools, block_table, block_size: int):
        assert len(pools) == 12
        self.pools = [_as_bits(t) for t in pools]
        self.block_table = block_table
        self.block_size = int(block_size)
        self.n_blocks = int(self.pools[0].shape[0])

    def c_struct(self) -> _PagedKV:
        c = _PagedKV()
        for i, t in enumerate(self.pools):
            c.kv[i] = _ptr(t)
        c.block_table = _ptr(self.block_table)
        c.block_size = self.block_size
        c.n_blocks = self.n_blocks
        return c


def dckv_bytes_paged(plan: Plan, T: int) -> int:
    """Workspace bytes of dckv_encode_paged / dckv_decode_paged for T tokens."""
    v = ctypes.c_uint64()
    _check(_lib.dckv_bytes_paged(plan.handle, int(T), ctypes.byref(v)))
    return v.value


def dckv_encode_paged(plan: Plan, cache: PagedKV, post_rope: bool, token_ids, stream_buf, stream_bytes, status,
                      ws, stream=None):
    """Enqueue an encode of the request held in a paged cache."""
    T = int(token_ids.shape[0])
    c = cache.c_struct()
    _check(_lib.dckv_encode_paged(plan.handle, ctypes.byref(c), 1 if post_rope else 0, _ptr(token_ids), T,
                                  _ptr(stream_buf), stream_buf.numel(), _ptr(stream_bytes), _ptr(status), _ptr(ws),
                                  ws.numel(), _stream_handle(stream)))


def dckv_decode_paged(plan: Plan, stream_buf, n_bytes: int, token_ids, cache: PagedKV, status, ws, stream=None):
    """Enqueue a decode into the request's rows of a paged cache."""
    T = int(token_ids.shape[0])
    c = cache.c_struct()
    _check(_lib.dckv_decode_paged(plan.handle, _ptr(stream_buf), int(n_bytes), _ptr(token_ids), T, ctypes.byref(c),
                                  _ptr(status), _ptr(ws), ws.numel(), _stream_handle(stream)))


def dckv_decode(plan: Plan, stream_buf, n_bytes: int, token_ids, rows_out, status, ws, stream=None):
    """Enqueue a decode into rows_out [T][D] (bf16 or int16 bits)."""
    T = int(token_ids.shape[0])
    out = _as_bits(rows_out)
    _check(_lib.dckv_decode(plan.handle, _ptr(stream_buf), int(n_bytes), _ptr(token_ids), T, _ptr(out),
                            _ptr(status), _ptr(ws), ws.numel(), _stream_handle(stream)))


class Request:
    """One request of a batch call.  Tensors are device tensors; fields a call
    does not use may be None (rows / stream_bytes for decode, rows_out for
    encode).  For decode, `capacity` is the stream's size in bytes."""

    def __init__(self, plan: Plan, token_ids, rows=None, stream=None, capacity=None, stream_bytes=None,
                 rows_out=None, status=None):
        self.plan, self.token_ids, self.rows, self.stream = plan, token_ids, rows, stream
        self.capacity = int(stream.numel() if capacity is None and stream is not None else (capacity or 0))
        self.stream_bytes, self.rows_out, self.status = stream_bytes, rows_out, status

    def c_req(self) -> _Req:
        T = int(self.token_ids.shape[0])
        rows = _as_bits(self.rows) if self.rows is not None else None
        out = _as_bits(self.rows_out) if self.rows_out is not None else None
        return _Req(self.plan.handle, _ptr(rows), _ptr(self.token_ids), T, _ptr(self.stream), self.capacity,
                    _ptr(self.stream_bytes), _ptr(out), _ptr(self.status))


def _reqs(requests):
    arr = (_Req * max(len(requests), 1))()
    for i, r in enumerate(requests):
        arr[i] = r.c_req()
    return arr


def dckv_bytes_batch(requests) -> int:
    """Workspace bytes for a batch call over these requests."""
    ws = ctypes.c_uint64()
    _check(_lib.dckv_bytes_batch(_reqs(requests), len(requests), ctypes.byref(ws)))
    return ws.value


def dckv_encode_batch(requests, ws, stream=None):
    """Enqueue the encode of every request, in order, on one stream."""
    _check(_lib.dckv_encode_batch(_reqs(requests), len(requests), _ptr(ws), ws.numel(), _stream_handle(stream)))


def dckv_decode_batch(requests, ws, stream=None):
    """Enqueue the decode of every request, in order, on one stream."""
    _check(_lib.dckv_decode_batch(_reqs(requests), len(requests), _ptr(ws), ws.numel(), _stream_handle(stream)))


def dckv_entropy_encode(plan: Plan, T: int, sym, esc, n_esc: int, rows, stream_buf, stream_bytes, status, ws,
                        stream=None):
    rows = _as_bits(rows) if rows is not None else None
    _check(_lib.dckv_entropy_encode(plan.handle, int(T), _ptr(sym), _ptr(esc), int(n_esc), _ptr(rows),
                                    _ptr(stream_buf), stream_buf.numel(), _ptr(stream_bytes), _ptr(status),
                                    _ptr(ws), ws.numel(), _stream_handle(stream)))


def dckv_entropy_decode(plan: Plan, stream_buf, n_bytes: int, T: int, sym_out, n_esc_out, status, ws,
                        stream=None):
    _check(_lib.dckv_entropy_decode(plan.handle, _ptr(stream_buf), int(n_bytes), int(T), _ptr(sym_out),
                                    _ptr(n_esc_out), _ptr(status), _ptr(ws), ws.numel(), _stream_handle(stream)))


def dckv_decode_heads(plan: Plan, stream_buf, n_bytes: int, token_ids, kv_out, status, ws, stream=None):
    """kv_out: 2 * n_layers device tensors [n_kv_heads][T][head_dim] (bf16 bits)."""
    arr = (ctypes.c_void_p * len(kv_out))(*[_ptr(t) for t in kv_out])
    _check(_lib.dckv_decode_heads(plan.handle, _ptr(stream_buf), int(n_bytes), _ptr(token_ids),
                                  int(token_ids.shape[0]), arr, _ptr(status), _ptr(ws), ws.numel(),
                                  _stream_handle(stream)))


def decode_heads(plan: Plan, stream_buf, token_ids, ws=None):
    """Decode into the attention layers' cache layout: returns (list of
    2 * n_layers tensors [n_kv_heads][T][head_dim] (int16 bf16 bits), status)."""
    import torch
    T = int(token_ids.shape[0])
    dev = plan.codec.device
    s = plan.codec.shape
    kv = [torch.empty((s["n_kv_heads"], T, s["head_dim"]), dtype=torch.int16, device=dev)
          for _ in range(2 * s["n_layers"])]
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = workspace(plan, T) if ws is None else ws
    dckv_decode_heads(plan, stream_buf, stream_buf.numel(), token_ids, kv, st, ws)
    return kv, int(st.item())


def dckv_unrope(plan: Plan, rows_in, rows_out, stream=None):
    _check(_lib.dckv_unrope(plan.handle, _ptr(rows_in), int(rows_in.shape[0]), _ptr(rows_out),
                            _stream_handle(stream)))


def dckv_fit_bytes(n: int) -> int:
    v = ctypes.c_uint64()
    _check(_lib.dckv_fit_bytes(int(n), ctypes.byref(v)))
    return v.value


def dckv_fit(codec: "Codec", rows, token_ids, ridge: float, mean_head_out, mean_head_bf16_out, nbr_weight_out,
             laplace_scale_out, status, ws, stream=None):
    n = int(token_ids.shape[0])
    prm = codec.c_params()
    _check(_lib.dckv_fit(ctypes.byref(prm), _ptr(rows), _ptr(token_ids), n, float(ridge), _ptr(mean_head_out),
                         _ptr(mean_head_bf16_out), _ptr(nbr_weight_out), _ptr(laplace_scale_out), _ptr(status),
                         _ptr(ws), ws.numel(), _stream_handle(stream)))


def fit(codec: "Codec", rows, token_ids, ridge: float):
    """Closed-form fit of the conditional models from calibration rows (device
    bf16 bits [n][D]) and token ids (device int32 [n]); returns (mean head fp32
    [n_coef][emb], its bf16 bits, neighbour weights, Laplace scales, status)."""
    import torch
    dev = codec.device
    n = int(token_ids.shape[0])
    H = torch.empty((codec.n_coef, codec.emb_dim), dtype=torch.float32, device=dev)
    Hb = torch.empty((codec.n_coef, codec.emb_dim), dtype=torch.int16, device=dev)
    a = torch.empty(codec.n_coef, dtype=torch.float32, device=dev)
    b = torch.empty(codec.n_coef, dtype=torch.float32, device=dev)
    st = torch.full((1,), 777, dtype=torch.int32, device=dev)
    ws = torch.empty(dckv_fit_bytes(n), dtype=torch.uint8, device=dev)
    dckv_fit(codec, rows, token_ids, ridge, H, Hb, a, b, st, ws)
    torch.cuda.synchronize()
    return H, Hb, a, b, int(st.item())


def dckv_rate_bytes(plan: Plan, T: int) -> int:
    v = ctypes.c_uint64()
    _check(_lib.dckv_rate_bytes(plan.handle, int(T), ctypes.byref(v)))
    return v.value


def dckv_rate_forward(plan: Plan, rows, token_ids, noise, bits_out, yhat_out, grad_y, grad_mean, grad_nbr,
                      grad_scale, status, ws, stream=None):
    _check(_lib.dckv_rate_forward(plan.handle, _ptr(rows), _ptr(token_ids), int(token_ids.shape[0]), _ptr(noise),
                                  _ptr(bits_out), _ptr(yhat_out), _ptr(grad_y), _ptr(grad_mean), _ptr(grad_nbr),
                                  _ptr(grad_scale), _ptr(status), _ptr(ws), ws.numel(), _stream_handle(stream)))


def rate_forward(plan: Plan, rows, token_ids, noise, ws=None):
    """Training rate of one request (device bf16 row bits [T][D], int32 token
    ids [T], fp32 noise [N][n_coef] in steps); returns a dict of device
    tensors: bits [N], yhat, grad_y, grad_mean [N][n_coef], grad_nbr,
    grad_scale [n_coef], and the status."""
    import torch
    dev = rows.device
    T = int(token_ids.shape[0])
    c = plan.codec
    N = max(T - c.shape["keep_head"] - c.shape["keep_tail"], 0)
    out = dict(bits=torch.empty(N, dtype=torch.float32, device=dev),
               yhat=torch.empty((N, c.n_coef), dtype=torch.float32, device=dev),
               grad_y=torch.empty((N, c.n_coef), dtype=torch.float32, device=dev),
               grad_mean=torch.empty((N, c.n_coef), dtype=torch.float32, device=dev),
               grad_nbr=torch.empty(c.n_coef, dtype=torch.float32, device=dev),
               grad_scale=torch.empty(c.n_coef, dtype=torch.float32, device=dev))
    st = torch.full((1,), 777, dtype=torch.int32, device=dev)
    if ws is None:
        ws = torch.empty(dckv_rate_bytes(plan, T), dtype=torch.uint8, device=dev)
    dckv_rate_forward(plan, rows, token_ids, noise, out["bits"], out["yhat"], out["grad_y"], out["grad_mean"],
                      out["grad_nbr"], out["grad_scale"], st, ws)
    torch.cuda.synchronize()
    out["status"] = int(st.item())
    return out


def dckv_rate_backward_bytes(plan: Plan, T: int) -> int:
    v = ctypes.c_uint64()
    _check(_lib.dckv_rate_backward_bytes(plan.handle, int(T), ctypes.byref(v)))
    return v.value


def dckv_rate_backward(plan: Plan, rows, token_ids, grad_y, grad_mean, grad_analysis, grad_mean_head, status, ws,
                       stream=None):
    _check(_lib.dckv_rate_backward(plan.handle, _ptr(rows), _ptr(token_ids), int(token_ids.shape[0]), _ptr(grad_y),
                                   _ptr(grad_mean), _ptr(grad_analysis), _ptr(grad_mean_head), _ptr(status),
                                   _ptr(ws), ws.numel(), _stream_handle(stream)))


def rate_backward(plan: Plan, rows, token_ids, grad_y, grad_mean, ws=None):
    """Weight gradients (dR/dA [n_coef][D], dR/dH [n_coef][emb], fp32 device
    tensors) for upstream gradients grad_y, grad_mean [N][n_coef]; and the status."""
    import torch
    dev = rows.device
    c = plan.codec
    gA = torch.empty((c.n_coef, c.D), dtype=torch.float32, device=dev)
    gH = torch.empty((c.n_coef, c.emb_dim), dtype=torch.float32, device=dev)
    st = torch.full((1,), 777, dtype=torch.int32, device=dev)
    if ws is None:
        ws = torch.empty(dckv_rate_backward_bytes(plan, int(token_ids.shape[0])), dtype=torch.uint8, device=dev)
    dckv_rate_backward(plan, rows, token_ids, grad_y, grad_mean, gA, gH, st, ws)
    torch.cuda.synchronize()
    return gA, gH, int(st.item())


def dckv_workspace_view(plan: Plan, T: int, which: int):
    off = ctypes.c_uint64()
    nb = ctypes.c_uint64()
    rs = ctypes.c_int64()
    _check(_lib.dckv_workspace_view(plan.handle, int(T), int(which), ctypes.byref(off), ctypes.byref(nb),
                                    ctypes.byref(rs)))
    return off.value, nb.value, rs.value


def dckv_profile_enable(on: bool = True):
    _check(_lib.dckv_profile_enable(1 if on else 0))


def dckv_profile_only(kernel=None):
    _check(_lib.dckv_profile_only(kernel.encode() if kernel else None))


def dckv_profile_reset():
    _check(_lib.dckv_profile_reset())


def dckv_profile_read(kernel: str):
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(_lib.dckv_profile_read(kernel.encode(), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


# ---------------------------------------------------------------------------
# convenience (allocating) wrappers
# ---------------------------------------------------------------------------
def encode(plan: Plan, rows, token_ids, ws=None, capacity=None):
    """Encode one request; returns (stream uint8 tensor trimmed to its size, status)."""
    import torch
    T = int(rows.shape[0])
    max_bytes, _ = dckv_bytes(plan, T)
    cap = int(capacity) if capacity is not None else max_bytes
    dev = plan.codec.device
    buf = torch.empty(cap, dtype=torch.uint8, device=dev)
    nb = torch.zeros(1, dtype=torch.int64, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = workspace(plan, T) if ws is None else ws
    dckv_encode(plan, rows, token_ids, buf, nb, st, ws)
    n = int(nb.item())
    code = int(st.item())
    return buf[:n], code


def decode(plan: Plan, stream_buf, token_ids, ws=None, out=None):
    """Decode one request; returns (rows bf16 [T][D], status)."""
    import torch
    T = int(token_ids.shape[0])
    dev = plan.codec.device
    out = torch.empty((T, plan.codec.D), dtype=torch.bfloat16, device=dev) if out is None else out
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = workspace(plan, T) if ws is None else ws
    dckv_decode(plan, stream_buf, stream_buf.numel(), token_ids, out, st, ws)
    return out, int(st.item())
