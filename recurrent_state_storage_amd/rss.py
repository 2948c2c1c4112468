"""Thin ctypes binding of librss (include/rss.h), same names as the C ABI.

Only argument marshalling happens here: torch tensors are checked for device,
dtype, shape and contiguity, turned into raw device pointers, and passed with
the current HIP stream. Every step of the decode path runs in the library's
HIP kernels; there is no fallback of any kind. If librss.so has not been built
the first call raises.

PyTorch provides device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librss.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "rss.h")
HEADERS = [HEADER, os.path.join(os.path.dirname(_HERE), "include", "rss_calib.h")]

RSS_OK, RSS_E_INVALID, RSS_E_SHAPE, RSS_E_DTYPE, RSS_E_CAPACITY, RSS_E_ORDER, RSS_E_HIP = range(7)
RSS_DTYPE_F32, RSS_DTYPE_BF16 = 0, 1
RSS_COPY_NONE, RSS_COPY_BF16, RSS_STATE_BF16 = 0, 1, 2
RSS_DEV_ROLLBACK_RANGE, RSS_DEV_RING_OVERFLOW, RSS_DEV_UNCOMMITTED = 1, 2, 4
RSS_KIND_MAMBA2, RSS_KIND_GDN, RSS_KIND_KDA = 0, 1, 2

_I32 = ctypes.c_int32
_VP = ctypes.c_void_p


class rss_config(ctypes.Structure):
    _fields_ = [(n, _I32) for n in ("batch", "nheads", "headdim", "dstate", "ngroups", "window",
                                     "capacity", "max_draft", "in_dtype", "read_copy", "kind")]


class rss_buffers(ctypes.Structure):
    _fields_ = [(n, _VP) for n in ("ckpt", "ckpt_lo", "ring_x", "ring_B", "ring_dl", "ptr", "A",
                                    "dev_err")]


class rss_sizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("ckpt", "ckpt_lo", "ring_x", "ring_B", "ring_dl",
                                                "ptr", "A", "dev_err")]


_SIGS = {
    "rss_version": ([], _I32),
    "rss_status_string": ([_I32], ctypes.c_char_p),
    "rss_buffer_sizes": ([ctypes.POINTER(rss_config), ctypes.POINTER(rss_sizes)], _I32),
    "rss_layer_bind": ([ctypes.POINTER(rss_config), ctypes.POINTER(rss_buffers),
                        ctypes.POINTER(_VP)], _I32),
    "rss_layer_free": ([_VP], _I32),
    "rss_init_state": ([_VP, _VP, _VP], _I32),
    "rss_decode_step": ([_VP, _VP, _VP, _VP, _VP, _VP, _VP], _I32),
    "rss_flush_checkpoint": ([_VP, _I32, _VP], _I32),
    "rss_decode_flush_step": ([_VP, _I32, _VP, _VP, _VP, _VP, _VP, _VP], _I32),
    "rss_decode_flush_step_each": ([_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP], _I32),
    "rss_flush_checkpoint_each": ([_VP, _VP, _VP], _I32),
    "rss_verify_k_tokens": ([_VP, _I32, _VP, _VP, _VP, _VP, _VP, _VP], _I32),
    "rss_verify_k_tokens_fold": ([_VP, _I32, _I32, _VP, _VP, _VP, _VP, _VP, _VP], _I32),
    "rss_rollback": ([_VP, _VP, _VP], _I32),
    "rss_get_device_error": ([_VP, ctypes.POINTER(_I32), _VP], _I32),
    "rss_gdn_decode_step": ([_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP], _I32),
    "rss_gdn_decode_flush_step": ([_VP, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP], _I32),
    "rss_kda_decode_flush_step": ([_VP, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP], _I32),
    "rss_gdn_eager_step": ([ctypes.POINTER(rss_config), _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP],
                           _I32),
    "rss_kda_decode_step": ([_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP], _I32),
    "rss_kda_eager_step": ([ctypes.POINTER(rss_config), _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP],
                           _I32),
    "rss_eager_step": ([ctypes.POINTER(rss_config), _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _VP],
                       _I32),
    "rss_eager_verify": ([ctypes.POINTER(rss_config), _VP, _VP, _I32, _VP, _VP, _VP, _VP, _VP,
                          _VP, _VP], _I32),
    "rss_calib_read": ([_VP, ctypes.c_size_t, _VP, _I32, _VP], _I32),
    "rss_calib_copy": ([_VP, _VP, ctypes.c_size_t, _I32, _VP], _I32),
    "rss_calib_write": ([_VP, ctypes.c_size_t, _I32, _VP], _I32),
    "rss_calib_tiles": ([_VP, ctypes.c_size_t, _I32, _VP, _I32, _I32, _VP], _I32),
}

_lib = None


class RssError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def library() -> ctypes.CDLL:
    """Load librss.so (once). Raises if it is missing: there is no fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
    return _lib


def declared_symbols() -> list:
    """Every function the public headers declare."""
    text = ""
    for h in HEADERS:
        with open(h) as f:
            text += f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z0-9_]+\s*\*?\s*(rss_[a-z0-9_]+)\s*\(",
                                 text, flags=re.M)))


def status_string(status: int) -> str:
    return library().rss_status_string(status).decode()


def _check(status: int, where: str) -> None:
    if status != RSS_OK:
        raise RssError(status, where)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t, dtype, shape, name) -> int:
    """Device pointer of a dense tensor of the given dtype and shape. `shape` may
    be a list of accepted shapes (e.g. with and without a length-1 token axis)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a device tensor (got {t.device})")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    shapes = [tuple(s) for s in shape] if isinstance(shape, list) else [tuple(shape)]
    if tuple(t.shape) not in shapes:
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {shapes[0]}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return t.data_ptr()


def _in_dtype(code: int):
    return torch.bfloat16 if code == RSS_DTYPE_BF16 else torch.float32


def _state_dtype(cfg):
    """Storage of the checkpoint / eager state: bf16 only for RSS_STATE_BF16."""
    return torch.bfloat16 if cfg.read_copy == RSS_STATE_BF16 else torch.float32


def make_config(batch, nheads, headdim, dstate, ngroups, window, capacity, max_draft=0,
                in_dtype=RSS_DTYPE_F32, read_copy=RSS_COPY_NONE, kind=RSS_KIND_MAMBA2) -> rss_config:
    return rss_config(batch, nheads, headdim, dstate, ngroups, window, capacity, max_draft,
                      in_dtype, read_copy, kind)


# ---- the C calls, one wrapper each -------------------------------------------
def rss_version() -> int:
    return library().rss_version()


def rss_buffer_sizes(cfg: rss_config) -> rss_sizes:
    out = rss_sizes()
    _check(library().rss_buffer_sizes(ctypes.byref(cfg), ctypes.byref(out)), "rss_buffer_sizes")
    return out


def rss_layer_bind(cfg: rss_config, bufs: rss_buffers) -> int:
    h = _VP()
    _check(library().rss_layer_bind(ctypes.byref(cfg), ctypes.byref(bufs), ctypes.byref(h)),
           "rss_layer_bind")
    return h.value


def rss_layer_free(handle) -> None:
    _check(library().rss_layer_free(handle), "rss_layer_free")


class ReplayLayer:
    """One SSM layer's decode state on a device: checkpoint (+ bf16 read copy),
    input ring and pointers, allocated with torch, bound to a librss handle."""

    def __init__(self, cfg: rss_config, A, device="cuda"):
        self.cfg = cfg
        c = cfg
        dev = torch.device(device)
        sizes = rss_buffer_sizes(cfg)   # validates cfg
        del sizes
        idt = _in_dtype(c.in_dtype)
        self.ckpt = torch.empty((c.batch, c.nheads, c.headdim, c.dstate), dtype=_state_dtype(c), device=dev)
        self.ckpt_lo = (torch.empty((c.batch, c.nheads, c.headdim, c.dstate), dtype=torch.bfloat16, device=dev)
                        if c.read_copy == RSS_COPY_BF16 else None)
        # slot-major ring: [batch, slot, head (group), row]
        self.ring_x = torch.zeros((c.batch, c.capacity, c.nheads, c.headdim), dtype=idt, device=dev)
        self.ring_B = torch.zeros((c.batch, c.capacity, c.ngroups, c.dstate), dtype=idt, device=dev)
        self.ring_dl = torch.zeros((c.batch, c.capacity, c.nheads, c.dstate if c.kind == RSS_KIND_KDA else 2),
                                   dtype=torch.float32, device=dev)
        self.ptr = torch.zeros((c.batch, c.nheads, 4), dtype=torch.int32, device=dev)
        self.A = A
        if c.kind == RSS_KIND_MAMBA2 or A is not None:
            _ptr(A, torch.float32, (c.nheads,), "A")
        self.dev_err = torch.zeros((4,), dtype=torch.int32, device=dev)
        bufs = rss_buffers(self.ckpt.data_ptr(),
                           self.ckpt_lo.data_ptr() if self.ckpt_lo is not None else None,
                           self.ring_x.data_ptr(), self.ring_B.data_ptr(), self.ring_dl.data_ptr(),
                           self.ptr.data_ptr(), A.data_ptr() if A is not None else None,
                           self.dev_err.data_ptr())
        self.handle = rss_layer_bind(cfg, bufs)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h and _lib is not None:
            _lib.rss_layer_free(h)
            self.handle = None

    # shapes of per-call tensors
    def tok_shapes(self, nt=None):
        c = self.cfg
        lead = (c.batch,) if nt is None else (c.batch, nt)
        return (lead + (c.nheads, c.headdim), lead + (c.ngroups, c.dstate), lead + (c.nheads,))

    def init_state(self, S0=None, stream=None):
        rss_init_state(self, S0, stream)

    def decode_step(self, x, B, C, dt, y, stream=None):
        rss_decode_step(self, x, B, C, dt, y, stream)

    def decode_flush_step(self, min_len, x, B, C, dt, y, stream=None):
        rss_decode_flush_step(self, min_len, x, B, C, dt, y, stream)

    def flush_checkpoint(self, min_len, stream=None):
        rss_flush_checkpoint(self, min_len, stream)

    def decode_flush_step_each(self, min_len, x, B, C, dt, y, stream=None):
        rss_decode_flush_step_each(self, min_len, x, B, C, dt, y, stream)

    def flush_checkpoint_each(self, min_len, stream=None):
        rss_flush_checkpoint_each(self, min_len, stream)

    def verify_k_tokens(self, K, x, B, C, dt, y, stream=None):
        rss_verify_k_tokens(self, K, x, B, C, dt, y, stream)

    def verify_k_tokens_fold(self, min_len, K, x, B, C, dt, y, stream=None):
        rss_verify_k_tokens_fold(self, min_len, K, x, B, C, dt, y, stream)

    def rollback(self, n_drop, stream=None):
        rss_rollback(self, n_drop, stream)

    def gdn_decode_step(self, q, k, v, beta, alpha, o, stream=None):
        rss_gdn_decode_step(self, q, k, v, beta, alpha, o, stream)

    def kda_decode_step(self, q, k, v, beta, alpha, o, stream=None):
        rss_kda_decode_step(self, q, k, v, beta, alpha, o, stream)

    def gdn_decode_flush_step(self, min_len, q, k, v, beta, alpha, o, stream=None):
        rss_gdn_decode_flush_step(self, min_len, q, k, v, beta, alpha, o, stream)

    def kda_decode_flush_step(self, min_len, q, k, v, beta, alpha, o, stream=None):
        rss_kda_decode_flush_step(self, min_len, q, k, v, beta, alpha, o, stream)

    def device_error(self, stream=None) -> int:
        return rss_get_device_error(self, stream)


def rss_init_state(layer: ReplayLayer, S0=None, stream=None) -> None:
    c = layer.cfg
    p = _ptr(S0, torch.float32, (c.batch, c.nheads, c.headdim, c.dstate), "S0")
    _check(library().rss_init_state(layer.handle, p, _stream(stream)), "rss_init_state")


def rss_decode_step(layer: ReplayLayer, x, B, C, dt, y, stream=None) -> None:
    c = layer.cfg
    xs, bs, ds = layer.tok_shapes()
    idt = _in_dtype(c.in_dtype)
    args = (_ptr(x, idt, xs, "x"), _ptr(B, idt, bs, "B"), _ptr(C, idt, bs, "C"),
            _ptr(dt, torch.float32, ds, "dt"), _ptr(y, torch.float32, xs, "y"))
    _check(library().rss_decode_step(layer.handle, *args, _stream(stream)), "rss_decode_step")


def rss_decode_flush_step(layer: ReplayLayer, min_len: int, x, B, C, dt, y, stream=None) -> None:
    c = layer.cfg
    xs, bs, ds = layer.tok_shapes()
    idt = _in_dtype(c.in_dtype)
    args = (_ptr(x, idt, xs, "x"), _ptr(B, idt, bs, "B"), _ptr(C, idt, bs, "C"),
            _ptr(dt, torch.float32, ds, "dt"), _ptr(y, torch.float32, xs, "y"))
    _check(library().rss_decode_flush_step(layer.handle, int(min_len), *args, _stream(stream)),
           "rss_decode_flush_step")


def rss_decode_flush_step_each(layer: ReplayLayer, min_len, x, B, C, dt, y, stream=None) -> None:
    c = layer.cfg
    xs, bs, ds = layer.tok_shapes()
    idt = _in_dtype(c.in_dtype)
    args = (_ptr(x, idt, xs, "x"), _ptr(B, idt, bs, "B"), _ptr(C, idt, bs, "C"),
            _ptr(dt, torch.float32, ds, "dt"), _ptr(y, torch.float32, xs, "y"))
    th = _ptr(min_len, torch.int32, (c.batch,), "min_len")
    _check(library().rss_decode_flush_step_each(layer.handle, th, *args, _stream(stream)),
           "rss_decode_flush_step_each")


def rss_flush_checkpoint_each(layer: ReplayLayer, min_len, stream=None) -> None:
    th = _ptr(min_len, torch.int32, (layer.cfg.batch,), "min_len")
    _check(library().rss_flush_checkpoint_each(layer.handle, th, _stream(stream)),
           "rss_flush_checkpoint_each")


def rss_flush_checkpoint(layer: ReplayLayer, min_len: int, stream=None) -> None:
    _check(library().rss_flush_checkpoint(layer.handle, int(min_len), _stream(stream)),
           "rss_flush_checkpoint")


def rss_verify_k_tokens(layer: ReplayLayer, K: int, x, B, C, dt, y, stream=None) -> None:
    c = layer.cfg
    xs, bs, ds = layer.tok_shapes(K + 1)
    idt = _in_dtype(c.in_dtype)
    args = (_ptr(x, idt, xs, "x"), _ptr(B, idt, bs, "B"), _ptr(C, idt, bs, "C"),
            _ptr(dt, torch.float32, ds, "dt"), _ptr(y, torch.float32, xs, "y"))
    _check(library().rss_verify_k_tokens(layer.handle, int(K), *args, _stream(stream)),
           "rss_verify_k_tokens")


def rss_verify_k_tokens_fold(layer: ReplayLayer, min_len: int, K: int, x, B, C, dt, y,
                             stream=None) -> None:
    c = layer.cfg
    xs, bs, ds = layer.tok_shapes(K + 1)
    idt = _in_dtype(c.in_dtype)
    args = (_ptr(x, idt, xs, "x"), _ptr(B, idt, bs, "B"), _ptr(C, idt, bs, "C"),
            _ptr(dt, torch.float32, ds, "dt"), _ptr(y, torch.float32, xs, "y"))
    _check(library().rss_verify_k_tokens_fold(layer.handle, int(min_len), int(K), *args,
                                              _stream(stream)), "rss_verify_k_tokens_fold")


def rss_rollback(layer: ReplayLayer, n_drop, stream=None) -> None:
    p = _ptr(n_drop, torch.int32, (layer.cfg.batch,), "n_drop")
    _check(library().rss_rollback(layer.handle, p, _stream(stream)), "rss_rollback")


def rss_get_device_error(layer: ReplayLayer, stream=None) -> int:
    v = _I32(0)
    _check(library().rss_get_device_error(layer.handle, ctypes.byref(v), _stream(stream)),
           "rss_get_device_error")
    return v.value


def rss_eager_step(cfg: rss_config, S, x, B, C, dt, A, y, T=1, stream=None) -> None:
    c = cfg
    idt = _in_dtype(c.in_dtype)

    def sh(*tail):  # token axis optional when T == 1
        return [(c.batch, T) + tail] + ([(c.batch,) + tail] if T == 1 else [])
    args = (_ptr(S, _state_dtype(c), (c.batch, c.nheads, c.headdim, c.dstate), "S"),
            _ptr(x, idt, sh(c.nheads, c.headdim), "x"),
            _ptr(B, idt, sh(c.ngroups, c.dstate), "B"),
            _ptr(C, idt, sh(c.ngroups, c.dstate), "C"),
            _ptr(dt, torch.float32, sh(c.nheads), "dt"),
            _ptr(A, torch.float32, (c.nheads,), "A"),
            _ptr(y, torch.float32, sh(c.nheads, c.headdim), "y"))
    _check(library().rss_eager_step(ctypes.byref(cfg), *args, int(T), _stream(stream)),
           "rss_eager_step")


def rss_eager_verify(cfg: rss_config, pool, src_slot, K, x, B, C, dt, A, y, stream=None) -> None:
    c = cfg
    idt = _in_dtype(c.in_dtype)
    lead = (c.batch, K + 1)
    args = (_ptr(pool, torch.float32, (c.batch, K + 1, c.nheads, c.headdim, c.dstate), "pool"),
            _ptr(src_slot, torch.int32, (c.batch,), "src_slot"), int(K),
            _ptr(x, idt, lead + (c.nheads, c.headdim), "x"),
            _ptr(B, idt, lead + (c.ngroups, c.dstate), "B"),
            _ptr(C, idt, lead + (c.ngroups, c.dstate), "C"),
            _ptr(dt, torch.float32, lead + (c.nheads,), "dt"),
            _ptr(A, torch.float32, (c.nheads,), "A"),
            _ptr(y, torch.float32, lead + (c.nheads, c.headdim), "y"))
    _check(library().rss_eager_verify(ctypes.byref(cfg), *args, _stream(stream)),
           "rss_eager_verify")


def rss_gdn_decode_step(layer: ReplayLayer, q, k, v, beta, alpha, o, stream=None) -> None:
    c = layer.cfg
    kn, vp, bh = (c.batch, c.nheads, c.dstate), (c.batch, c.nheads, c.headdim), (c.batch, c.nheads)
    f = torch.float32
    args = (_ptr(q, f, kn, "q"), _ptr(k, f, kn, "k"), _ptr(v, f, vp, "v"), _ptr(beta, f, bh, "beta"),
            _ptr(alpha, f, bh, "alpha"), _ptr(o, f, vp, "o"))
    _check(library().rss_gdn_decode_step(layer.handle, *args, _stream(stream)), "rss_gdn_decode_step")


def rss_gdn_eager_step(cfg: rss_config, S, q, k, v, beta, alpha, o, stream=None) -> None:
    c = cfg
    kn, vp, bh = (c.batch, c.nheads, c.dstate), (c.batch, c.nheads, c.headdim), (c.batch, c.nheads)
    f = torch.float32
    args = (_ptr(S, f, (c.batch, c.nheads, c.headdim, c.dstate), "S"), _ptr(q, f, kn, "q"),
            _ptr(k, f, kn, "k"), _ptr(v, f, vp, "v"), _ptr(beta, f, bh, "beta"),
            _ptr(alpha, f, bh, "alpha"), _ptr(o, f, vp, "o"))
    _check(library().rss_gdn_eager_step(ctypes.byref(cfg), *args, _stream(stream)), "rss_gdn_eager_step")


def rss_kda_decode_step(layer: ReplayLayer, q, k, v, beta, alpha, o, stream=None) -> None:
    c = layer.cfg
    kn, vp, bh = (c.batch, c.nheads, c.dstate), (c.batch, c.nheads, c.headdim), (c.batch, c.nheads)
    f = torch.float32
    args = (_ptr(q, f, kn, "q"), _ptr(k, f, kn, "k"), _ptr(v, f, vp, "v"), _ptr(beta, f, bh, "beta"),
            _ptr(alpha, f, kn, "alpha"), _ptr(o, f, vp, "o"))
    _check(library().rss_kda_decode_step(layer.handle, *args, _stream(stream)), "rss_kda_decode_step")


def rss_kda_eager_step(cfg: rss_config, S, q, k, v, beta, alpha, o, stream=None) -> None:
    c = cfg
    kn, vp, bh = (c.batch, c.nheads, c.dstate), (c.batch, c.nheads, c.headdim), (c.batch, c.nheads)
    f = torch.float32
    args = (_ptr(S, f, (c.batch, c.nheads, c.headdim, c.dstate), "S"), _ptr(q, f, kn, "q"),
            _ptr(k, f, kn, "k"), _ptr(v, f, vp, "v"), _ptr(beta, f, bh, "beta"),
            _ptr(alpha, f, kn, "alpha"), _ptr(o, f, vp, "o"))
    _check(library().rss_kda_eager_step(ctypes.byref(cfg), *args, _stream(stream)), "rss_kda_eager_step")


def _delta_args(layer, q, k, v, beta, alpha, o, kda):
    c = layer.cfg
    kn, vp, bh = (c.batch, c.nheads, c.dstate), (c.batch, c.nheads, c.headdim), (c.batch, c.nheads)
    f = torch.float32
    return (_ptr(q, f, kn, "q"), _ptr(k, f, kn, "k"), _ptr(v, f, vp, "v"), _ptr(beta, f, bh, "beta"),
            _ptr(alpha, f, kn if kda else bh, "alpha"), _ptr(o, f, vp, "o"))


def rss_gdn_decode_flush_step(layer: ReplayLayer, min_len: int, q, k, v, beta, alpha, o, stream=None) -> None:
    args = _delta_args(layer, q, k, v, beta, alpha, o, False)
    _check(library().rss_gdn_decode_flush_step(layer.handle, int(min_len), *args, _stream(stream)),
           "rss_gdn_decode_flush_step")


def rss_kda_decode_flush_step(layer: ReplayLayer, min_len: int, q, k, v, beta, alpha, o, stream=None) -> None:
    args = _delta_args(layer, q, k, v, beta, alpha, o, True)
    _check(library().rss_kda_decode_flush_step(layer.handle, int(min_len), *args, _stream(stream)),
           "rss_kda_decode_flush_step")


# ---- bandwidth calibration kernels (include/rss_calib.h) ----------------------
def rss_calib_read(src, sink, blocks: int = 0, stream=None) -> None:
    """Stream-read the bytes of the contiguous device tensor `src`; `sink` is a
    device float32 tensor of at least one element the kernel may write."""
    if not (isinstance(src, torch.Tensor) and src.is_cuda and src.is_contiguous()):
        raise ValueError("src: expected a contiguous device tensor")
    if not (isinstance(sink, torch.Tensor) and sink.is_cuda and sink.dtype == torch.float32):
        raise ValueError("sink: expected a device float32 tensor")
    nbytes = src.numel() * src.element_size()
    _check(library().rss_calib_read(src.data_ptr(), nbytes, sink.data_ptr(), int(blocks), _stream(stream)),
           "rss_calib_read")


def rss_calib_copy(src, dst, blocks: int = 0, stream=None) -> None:
    """Copy the bytes of the contiguous device tensor `src` into `dst` (same
    byte size, no overlap)."""
    for t, n in ((src, "src"), (dst, "dst")):
        if not (isinstance(t, torch.Tensor) and t.is_cuda and t.is_contiguous()):
            raise ValueError(f"{n}: expected a contiguous device tensor")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("dst: byte size differs from src")
    _check(library().rss_calib_copy(src.data_ptr(), dst.data_ptr(), nbytes, int(blocks), _stream(stream)),
           "rss_calib_copy")


def rss_calib_write(dst, blocks: int = 0, stream=None) -> None:
    """Stream-write the bytes of the contiguous device tensor `dst` (16-byte
    vector i holds the floats (i mod 2^24, 1, 2, 3))."""
    if not (isinstance(dst, torch.Tensor) and dst.is_cuda and dst.is_contiguous()):
        raise ValueError("dst: expected a contiguous device tensor")
    nbytes = dst.numel() * dst.element_size()
    _check(library().rss_calib_write(dst.data_ptr(), nbytes, int(blocks), _stream(stream)), "rss_calib_write")


def rss_calib_tiles(src, tile_bytes: int, n_tiles: int, dst=None, write_bytes: int = 0, order: int = 0,
                    stream=None) -> None:
    """One workgroup per tile: read n_tiles tiles of tile_bytes from the
    contiguous device tensor `src`, then write write_bytes per tile to `dst`;
    tiles in the decode kernels' order (0) or one contiguous range per XCD (1)."""
    if not (isinstance(src, torch.Tensor) and src.is_cuda and src.is_contiguous()):
        raise ValueError("src: expected a contiguous device tensor")
    if src.numel() * src.element_size() < n_tiles * tile_bytes:
        raise ValueError("src: smaller than n_tiles * tile_bytes")
    dptr = 0
    if write_bytes:
        if not (isinstance(dst, torch.Tensor) and dst.is_cuda and dst.is_contiguous()):
            raise ValueError("dst: expected a contiguous device tensor")
        if dst.numel() * dst.element_size() < n_tiles * write_bytes:
            raise ValueError("dst: smaller than n_tiles * write_bytes")
        dptr = dst.data_ptr()
    _check(library().rss_calib_tiles(src.data_ptr(), int(tile_bytes), int(n_tiles), dptr, int(write_bytes),
                                     int(order), _stream(stream)), "rss_calib_tiles")
