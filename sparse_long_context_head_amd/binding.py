"""Python binding of the ReTopK C ABI (include/retopk.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of libretopk.so. Functions carry the C entry points' names and take
PyTorch tensors for device buffers (PyTorch supplies device memory and the
stream; it computes nothing here). If the library is missing, importing this
module raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libretopk.so")

RETOPK_OK = 0
STATUS_NAMES = {0: "OK", 1: "INVALID_ARG", 2: "OUT_OF_RANGE", 3: "HIP_ERROR",
                4: "NOT_INITIALIZED", 5: "NO_DEVICE"}


class RetopkError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class RetopkParams(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("max_len", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("cache_cap", ctypes.c_int32), ("window", ctypes.c_int32),
                ("top_r", ctypes.c_int32), ("refresh_every", ctypes.c_int32),
                ("tau", ctypes.c_double), ("retrieval", ctypes.c_int32)]


RETRIEVAL = {"similarity": 0, "recent": 1}


# Exported symbols and their C signatures (restype, argtypes).
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_SIGNATURES = {
    "retopk_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "retopk_last_error": (ctypes.c_char_p, []),
    "retopk_create": (ctypes.c_int, [ctypes.POINTER(RetopkParams), ctypes.POINTER(_P)]),
    "retopk_destroy": (None, [_P]),
    "retopk_init_from_prefill": (ctypes.c_int, [_P, _P, _P, _I32, _P]),
    "retopk_decode_step": (ctypes.c_int, [_P, _P, _P, _P, _I32, _I32, _P, _P]),
    "retopk_exact_topk_attn": (ctypes.c_int, [_P, _P, _P, _P, _I32, _P, _P, _P]),
    "retopk_dense_attn": (ctypes.c_int, [_P, _P, _P, _P, _I32, _P, _P]),
    "retopk_read_state": (ctypes.c_int, [_P, _P, _P, _P, _P]),
    "retopk_write_state": (ctypes.c_int, [_P, _P, _P, _P, _P]),
    "retopk_read_step_info": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "retopk_read_stats": (ctypes.c_int, [_P, _I32, _I32, _P, _P, _P]),
    "retopk_set_stats": (ctypes.c_int, [_P, _I32]),
    "retopk_set_timing": (ctypes.c_int, [_P, _I32]),
    "retopk_read_kernel_times": (ctypes.c_int, [_P, _I32, _P, _P]),
    "retopk_kernel_count": (_I32, []),
    "retopk_kernel_name": (ctypes.c_char_p, [_I32]),
    "retopk_device_bytes": (ctypes.c_size_t, [_P]),
    "retopk_read_device_error": (ctypes.c_int, [_P, _P]),
    "retopk_stream_read": (ctypes.c_int, [_P, ctypes.c_size_t, _P, _P]),
    "retopk_score_probe": (ctypes.c_int, [ctypes.c_int32, _P, ctypes.c_int64, _P, _P, _P]),
    "retopk_dense_attn_noalloc": (ctypes.c_int, [_I32, _I32, _I32, _I32, _P, _P, _P, _I32, _P, _P]),
    "retopk_group_create": (ctypes.c_int, [ctypes.POINTER(RetopkParams), _I32, ctypes.POINTER(_P)]),
    "retopk_group_destroy": (None, [_P]),
    "retopk_group_layer": (_P, [_P, _I32]),
    "retopk_group_device_bytes": (ctypes.c_size_t, [_P]),
    "retopk_group_capture": (ctypes.c_int, [_P, _P, _P, _P, _P, _P]),
    "retopk_group_set_position": (ctypes.c_int, [_P, _I32, _I32]),
    "retopk_group_replay": (ctypes.c_int, [_P, _P]),
}

_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libretopk.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"HIP library {_LIB_PATH} is missing; build it with "
                              "`python -m sparse_long_context_head_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status: int):
    if status != RETOPK_OK:
        raise RetopkError(status, load_library().retopk_last_error().decode())


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        if not t.flags["C_CONTIGUOUS"]:
            raise ValueError("host array must be C-contiguous")
        return t.ctypes.data
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream, device=None) -> int | None:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream(device).cuda_stream


@dataclasses.dataclass
class Handle:
    """An opened library handle and the parameters it was created with."""
    ptr: int
    params: dict

    def __post_init__(self):
        p = self.params
        self.bh = p["batch"] * p["n_q_heads"]
        self.cand_cap = p["top_r"] * p["top_k"] + p["window"]


def _check_tensor(name, t, shape, dtypes):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if str(t.dtype).split(".")[-1] not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_BF16 = ("bfloat16", "int16", "uint16")


def retopk_create(batch, n_q_heads, n_kv_heads, head_dim, max_len, top_k, cache_cap, window,
                  top_r, refresh_every, tau, retrieval="similarity") -> Handle:
    """retrieval: "similarity" (Eq. 7) or "recent" (the ablation's recent-R)."""
    lib = load_library()
    params = dict(batch=batch, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads, head_dim=head_dim,
                  max_len=max_len, top_k=top_k, cache_cap=cache_cap, window=window,
                  top_r=top_r, refresh_every=refresh_every, tau=float(tau))
    p = RetopkParams(**params, retrieval=RETRIEVAL[retrieval])
    params["retrieval"] = retrieval
    out = _P()
    _check(lib.retopk_create(ctypes.byref(p), ctypes.byref(out)))
    return Handle(out.value, params)


def retopk_destroy(h: Handle):
    if h is not None and h.ptr:
        load_library().retopk_destroy(h.ptr)
        h.ptr = 0


def retopk_init_from_prefill(h: Handle, q_tail, k, prompt_len: int, stream=None):
    p = h.params
    n0 = min(p["cache_cap"], prompt_len)
    _check_tensor("q_tail", q_tail, (p["batch"], p["n_q_heads"], n0, p["head_dim"]), _BF16)
    _check_tensor("k", k, (p["batch"], p["n_kv_heads"], p["max_len"], p["head_dim"]), _BF16)
    _check(load_library().retopk_init_from_prefill(h.ptr, _ptr(q_tail), _ptr(k), prompt_len,
                                                   _stream(stream, q_tail.device)))


def retopk_decode_step(h: Handle, q, k, v, length: int, t_dec: int, out, stream=None):
    p = h.params
    _check_tensor("q", q, (p["batch"], p["n_q_heads"], p["head_dim"]), _BF16)
    kv_shape = (p["batch"], p["n_kv_heads"], p["max_len"], p["head_dim"])
    _check_tensor("k", k, kv_shape, _BF16)
    _check_tensor("v", v, kv_shape, _BF16)
    _check_tensor("out", out, (p["batch"], p["n_q_heads"], p["head_dim"]), ("float32",))
    _check(load_library().retopk_decode_step(h.ptr, _ptr(q), _ptr(k), _ptr(v), length, t_dec,
                                             _ptr(out), _stream(stream, q.device)))


def retopk_exact_topk_attn(h: Handle, q, k, v, length: int, out, sel_out=None, stream=None):
    p = h.params
    _check_tensor("q", q, (p["batch"], p["n_q_heads"], p["head_dim"]), _BF16)
    kv_shape = (p["batch"], p["n_kv_heads"], p["max_len"], p["head_dim"])
    _check_tensor("k", k, kv_shape, _BF16)
    _check_tensor("v", v, kv_shape, _BF16)
    _check_tensor("out", out, (p["batch"], p["n_q_heads"], p["head_dim"]), ("float32",))
    if sel_out is not None:
        _check_tensor("sel_out", sel_out, (p["batch"], p["n_q_heads"], p["top_k"]), ("int32",))
    _check(load_library().retopk_exact_topk_attn(h.ptr, _ptr(q), _ptr(k), _ptr(v), length,
                                                 _ptr(out), _ptr(sel_out),
                                                 _stream(stream, q.device)))


def retopk_dense_attn(h: Handle, q, k, v, length: int, out, stream=None):
    p = h.params
    _check_tensor("q", q, (p["batch"], p["n_q_heads"], p["head_dim"]), _BF16)
    kv_shape = (p["batch"], p["n_kv_heads"], p["max_len"], p["head_dim"])
    _check_tensor("k", k, kv_shape, _BF16)
    _check_tensor("v", v, kv_shape, _BF16)
    _check_tensor("out", out, (p["batch"], p["n_q_heads"], p["head_dim"]), ("float32",))
    _check(load_library().retopk_dense_attn(h.ptr, _ptr(q), _ptr(k), _ptr(v), length, _ptr(out),
                                            _stream(stream, q.device)))


def retopk_read_state(h: Handle):
    """Return (qbar [B,Hq,C,D] f32, supp [B,Hq,C,K] i32, supp_len [B,Hq,C] i32, count [B,Hq] i32)."""
    p = h.params
    b, hq, c, k, d = p["batch"], p["n_q_heads"], p["cache_cap"], p["top_k"], p["head_dim"]
    qbar = np.zeros((b, hq, c, d), np.float32)
    supp = np.zeros((b, hq, c, k), np.int32)
    slen = np.zeros((b, hq, c), np.int32)
    count = np.zeros((b, hq), np.int32)
    _check(load_library().retopk_read_state(h.ptr, _ptr(qbar), _ptr(supp), _ptr(slen), _ptr(count)))
    return qbar, supp, slen, count


def retopk_write_state(h: Handle, qbar, supp, supp_len, count):
    p = h.params
    b, hq, c, k, d = p["batch"], p["n_q_heads"], p["cache_cap"], p["top_k"], p["head_dim"]
    arrs = [np.ascontiguousarray(qbar, np.float32).reshape(b, hq, c, d),
            np.ascontiguousarray(supp, np.int32).reshape(b, hq, c, k),
            np.ascontiguousarray(supp_len, np.int32).reshape(b, hq, c),
            np.ascontiguousarray(count, np.int32).reshape(b, hq)]
    _check(load_library().retopk_write_state(h.ptr, *[_ptr(a) for a in arrs]))


def retopk_read_step_info(h: Handle) -> dict:
    p = h.params
    b, hq = p["batch"], p["n_q_heads"]
    info = dict(path=np.zeros((b, hq), np.int32), rho_max=np.zeros((b, hq), np.float64),
                retrieved=np.zeros((b, hq, p["top_r"]), np.int32),
                n_cand=np.zeros((b, hq), np.int32),
                cand=np.zeros((b, hq, h.cand_cap), np.int32),
                sel=np.zeros((b, hq, p["top_k"]), np.int32),
                sel_len=np.zeros((b, hq), np.int32),
                sel_scores=np.zeros((b, hq, p["top_k"]), np.float32))
    order = ["path", "rho_max", "retrieved", "n_cand", "cand", "sel", "sel_len", "sel_scores"]
    _check(load_library().retopk_read_step_info(h.ptr, *[_ptr(info[k]) for k in order]))
    return info


def retopk_read_stats(h: Handle, first_t_dec: int, n_steps: int):
    """Return (path uint8, rho_max float64, n_cand int32), each [n_steps, B, Hq]."""
    p = h.params
    shape = (n_steps, p["batch"], p["n_q_heads"])
    path = np.zeros(shape, np.uint8)
    rho = np.zeros(shape, np.float64)
    m = np.zeros(shape, np.int32)
    _check(load_library().retopk_read_stats(h.ptr, first_t_dec, n_steps, _ptr(path), _ptr(rho),
                                            _ptr(m)))
    return path, rho, m


def retopk_set_stats(h: Handle, enabled: bool):
    _check(load_library().retopk_set_stats(h.ptr, int(bool(enabled))))


def retopk_set_timing(h: Handle, enabled: bool):
    _check(load_library().retopk_set_timing(h.ptr, int(bool(enabled))))


def retopk_kernel_names() -> list[str]:
    lib = load_library()
    return [lib.retopk_kernel_name(i).decode() for i in range(lib.retopk_kernel_count())]


def retopk_read_kernel_times(h: Handle) -> dict:
    """{kernel name: (total milliseconds, launches)} since the last read."""
    lib = load_library()
    n = lib.retopk_kernel_count()
    ms = np.zeros(n, np.float64)
    cnt = np.zeros(n, np.int64)
    _check(lib.retopk_read_kernel_times(h.ptr, n, _ptr(ms), _ptr(cnt)))
    return {lib.retopk_kernel_name(i).decode(): (float(ms[i]), int(cnt[i])) for i in range(n)}


def retopk_device_bytes(h: Handle) -> int:
    return int(load_library().retopk_device_bytes(h.ptr))


def retopk_read_device_error(h: Handle) -> int:
    word = np.zeros(1, np.int32)
    _check(load_library().retopk_read_device_error(h.ptr, _ptr(word)))
    return int(word[0])


def retopk_dense_attn_noalloc(q, k, v, length: int, out, stream=None):
    """Dense attention without a handle or any allocation (shapes from the tensors)."""
    b, hq, d = q.shape
    hkv, max_len = k.shape[1], k.shape[2]
    _check_tensor("q", q, (b, hq, d), _BF16)
    _check_tensor("k", k, (b, hkv, max_len, d), _BF16)
    _check_tensor("v", v, (b, hkv, max_len, d), _BF16)
    _check_tensor("out", out, (b, hq, d), ("float32",))
    _check(load_library().retopk_dense_attn_noalloc(b, hq, hkv, max_len, _ptr(q), _ptr(k), _ptr(v), length,
                                                    _ptr(out), _stream(stream, q.device)))


class ReTopKGroup:
    """n layers sharing one set of per-call workspaces (retopk_group_*), with
    a graph-replayed decode token. layers[l] is a ReTopKLayer view of layer l
    (owned by the group)."""

    def __init__(self, n_layers, retrieval="similarity", **params):
        lib = load_library()
        self.params = dict(params, tau=float(params["tau"]))
        p = RetopkParams(**self.params, retrieval=RETRIEVAL[retrieval])
        self.params["retrieval"] = retrieval
        out = _P()
        _check(lib.retopk_group_create(ctypes.byref(p), n_layers, ctypes.byref(out)))
        self.ptr = out.value
        self.layers = []
        for l in range(n_layers):
            layer = ReTopKLayer.__new__(ReTopKLayer)
            layer.handle = Handle(lib.retopk_group_layer(self.ptr, l), self.params)
            layer.params = self.params
            layer.owned = False
            self.layers.append(layer)
        self._keep = None

    @classmethod
    def from_workload(cls, wl, n_layers, max_len=None, **override):
        p = dict(batch=wl.batch, n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads,
                 head_dim=wl.head_dim, max_len=max_len or wl.max_len, top_k=wl.top_k,
                 cache_cap=wl.cache_cap, window=wl.window, top_r=wl.top_r,
                 refresh_every=wl.refresh_every, tau=wl.tau)
        p.update(override)
        return cls(n_layers, **p)

    def device_bytes(self):
        return int(load_library().retopk_group_device_bytes(self.ptr))

    def capture(self, qs, ks, vs, outs, stream):
        """Capture one token over all layers (lists of device tensors, one per
        layer; the tensors must stay alive while the graph is used)."""
        n = len(self.layers)
        p = self.params
        for name, ts, shape in (("q", qs, (p["batch"], p["n_q_heads"], p["head_dim"])),
                                ("k", ks, (p["batch"], p["n_kv_heads"], p["max_len"], p["head_dim"])),
                                ("v", vs, (p["batch"], p["n_kv_heads"], p["max_len"], p["head_dim"]))):
            if len(ts) != n:
                raise ValueError(f"{name}: one tensor per layer")
            for t in ts:
                _check_tensor(name, t, shape, _BF16)
        for t in outs:
            _check_tensor("out", t, (p["batch"], p["n_q_heads"], p["head_dim"]), ("float32",))
        arr = lambda ts: (ctypes.c_void_p * n)(*[t.data_ptr() for t in ts])
        a = [arr(qs), arr(ks), arr(vs), arr(outs)]
        _check(load_library().retopk_group_capture(self.ptr, *[ctypes.cast(x, ctypes.c_void_p) for x in a],
                                                   _stream(stream)))
        self._keep = (list(qs), list(ks), list(vs), list(outs))

    def set_position(self, length, t_dec):
        _check(load_library().retopk_group_set_position(self.ptr, length, t_dec))

    def replay(self, stream):
        _check(load_library().retopk_group_replay(self.ptr, _stream(stream)))

    def close(self):
        if self.ptr:
            load_library().retopk_group_destroy(self.ptr)
            self.ptr = 0
            for layer in self.layers:
                layer.handle.ptr = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def retopk_stream_read(buf, sink, stream=None):
    """One plain streaming read of the whole device tensor `buf` (measurement aid)."""
    if not buf.is_cuda or not sink.is_cuda:
        raise ValueError("buf and sink must be device tensors")
    _check(load_library().retopk_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                             _stream(stream, buf.device)))


def retopk_score_probe(use_mfma, k, q, sink, stream=None):
    """One score pass of 7 query heads (q [7, 128] bf16) over every row of
    k [n, 128] bf16, on MFMA or on the vector ALUs (measurement aid)."""
    if not (k.is_cuda and q.is_cuda and sink.is_cuda):
        raise ValueError("k, q and sink must be device tensors")
    if k.dim() != 2 or k.shape[1] != 128 or tuple(q.shape) != (7, 128):
        raise ValueError("k must be [n, 128] and q [7, 128]")
    if k.dtype != q.dtype or k.element_size() != 2 or sink.dtype.itemsize != 4:
        raise ValueError("k and q must be 2-byte (bf16) tensors, sink a 4-byte one")
    if not (k.is_contiguous() and q.is_contiguous()):
        raise ValueError("k and q must be contiguous")
    _check(load_library().retopk_score_probe(int(use_mfma), _ptr(k), k.shape[0], _ptr(q), _ptr(sink),
                                             _stream(stream, k.device)))


def bf16_tensor(bits: np.ndarray, device="cuda"):
    """Upload uint16 bf16 bit patterns as a torch.bfloat16 device tensor (same bytes)."""
    import torch
    a = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(a).view(torch.bfloat16).to(device)


class ReTopKLayer:
    """Owns one handle (one attention layer's query-support caches and workspaces)."""

    def __init__(self, **params):
        self.handle = retopk_create(**params)
        self.params = self.handle.params
        self.owned = True

    @classmethod
    def from_workload(cls, wl, max_len=None, **override):
        p = dict(batch=wl.batch, n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads,
                 head_dim=wl.head_dim, max_len=max_len or wl.max_len, top_k=wl.top_k,
                 cache_cap=wl.cache_cap, window=wl.window, top_r=wl.top_r,
                 refresh_every=wl.refresh_every, tau=wl.tau)
        p.update(override)
        return cls(**p)

    def close(self):
        if getattr(self, "owned", True):
            retopk_destroy(self.handle)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def init_from_prefill(self, q_tail, k, prompt_len, stream=None):
        retopk_init_from_prefill(self.handle, q_tail, k, prompt_len, stream)

    def decode_step(self, q, k, v, length, t_dec, out, stream=None):
        retopk_decode_step(self.handle, q, k, v, length, t_dec, out, stream)

    def exact_topk_attn(self, q, k, v, length, out, sel_out=None, stream=None):
        retopk_exact_topk_attn(self.handle, q, k, v, length, out, sel_out, stream)

    def dense_attn(self, q, k, v, length, out, stream=None):
        retopk_dense_attn(self.handle, q, k, v, length, out, stream)

    def read_state(self):
        return retopk_read_state(self.handle)

    def write_state(self, *state):
        retopk_write_state(self.handle, *state)

    def step_info(self):
        return retopk_read_step_info(self.handle)

    def stats(self, first_t_dec, n_steps):
        return retopk_read_stats(self.handle, first_t_dec, n_steps)
