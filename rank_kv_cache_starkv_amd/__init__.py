"""Python binding of libstarkv: decode attention over a low-rank, mixed-precision KV cache.

Argument marshalling only.  Every step of the path runs in libstarkv's HIP kernels;
PyTorch provides device memory and the stream.  There is no CPU fallback: if the
library is not built, :func:`lib` raises.

Typical use (one layer)::

    layer = Layer(H_q, H_kv, d_h, d, "bf16", "mix84", s_k, tau_k, s_v, tau_v)
    layer.build_factors(U_k, V_k, U_v, V_v)      # fp32 SVD factors on the device
    layer.calibrate(X_cal)                       # per-channel fp16 scales (mix84)
    cache = layer.new_cache(B, T_max)
    layer.append(cache, X_new, lens)             # project + quantise new tokens
    out = layer.decode(cache, q, lens)           # attention read from the latent
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libstarkv.so")

F32, BF16 = 0, 1
LATENT = {"f32": 0, "bf16": 1, "mix84": 2, "had43": 3, "had43p": 4}
DTYPE = {"f32": F32, "bf16": BF16}
TILE_TOKENS = 32
MAX_BATCH = 128
NOALLOC_SCRATCH_BYTES = 64 << 20  # STARKV_NOALLOC_SCRATCH_BYTES

STATUS = {0: "ok", -1: "EINVAL", -2: "ENOMEM", -3: "ECAPACITY", -4: "EUNSUPPORTED", -5: "EWORKSPACE",
          -6: "EHIP", -7: "ESTATE"}


class StarKVError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {STATUS.get(status, status)} ({status})")
        self.status = status


class _Desc(ctypes.Structure):
    _fields_ = [("H_q", ctypes.c_int), ("H_kv", ctypes.c_int), ("d_h", ctypes.c_int), ("d", ctypes.c_int),
                ("dtype", ctypes.c_int), ("latent", ctypes.c_int), ("shrink", ctypes.c_int), ("n_v", ctypes.c_int),
                ("s_k", ctypes.POINTER(ctypes.c_float)), ("tau_k", ctypes.POINTER(ctypes.c_float)),
                ("s_v", ctypes.POINTER(ctypes.c_float)), ("tau_v", ctypes.c_float)]


class _Info(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("H_q", "H_kv", "d_h", "d", "dtype", "latent", "n_key", "r_v", "n_lat",
                                            "k_row_bytes", "v_tile_rows", "v_tile_bytes", "K8", "K4", "V8", "V4", "K3",
                                            "V3")] + \
               [(n, ctypes.c_size_t) for n in ("a_bytes", "bk_bytes", "bv_bytes", "scale_bytes")]


class _KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int), ("total_ms", ctypes.c_double)]


class _Cache(ctypes.Structure):
    _fields_ = [("k_rows", ctypes.c_void_p), ("v_tiles", ctypes.c_void_p), ("B", ctypes.c_int),
                ("T_max", ctypes.c_int)]


EXPORTS = ["starkv_abi_version", "starkv_status_string", "starkv_layer_create", "starkv_layer_destroy",
           "starkv_layer_get_info", "starkv_layer_ranks", "starkv_build_factors", "starkv_bind_factors",
           "starkv_calibrate", "starkv_bind_scales", "starkv_cache_bytes", "starkv_compress_append",
           "starkv_decode_workspace_bytes", "starkv_decode_attention", "starkv_decode_step", "starkv_reconstruct",
           "starkv_absorb_query", "starkv_decode_attention_hidden", "starkv_profile_enable", "starkv_profile_read",
           "starkv_decode_step_noalloc", "starkv_layer_set_rope", "starkv_prefill_workspace_bytes",
           "starkv_prefill_attention"]

# the ABI these argument lists describe (STARKV_ABI_VERSION of include/starkv.h)
ABI_VERSION = 2

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libstarkv (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libstarkv is not built ({LIB_PATH} missing); run __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    vp, ci, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.starkv_abi_version.restype = ci
    if L.starkv_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{LIB_PATH} has ABI {L.starkv_abi_version()}, the binding expects {ABI_VERSION}: "
                           "rebuild it with __graft_entry__.build()")
    L.starkv_status_string.restype = ctypes.c_char_p
    L.starkv_status_string.argtypes = [ci]
    L.starkv_layer_create.argtypes = [ctypes.POINTER(_Desc), ctypes.POINTER(vp)]
    L.starkv_layer_destroy.argtypes = [vp]
    L.starkv_layer_get_info.argtypes = [vp, ctypes.POINTER(_Info)]
    L.starkv_layer_ranks.argtypes = [vp, ctypes.POINTER(ctypes.c_int32)]
    L.starkv_build_factors.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.starkv_bind_factors.argtypes = [vp, vp, vp, vp]
    L.starkv_calibrate.argtypes = [vp, vp, ci, vp, vp]
    L.starkv_bind_scales.argtypes = [vp, vp]
    L.starkv_cache_bytes.argtypes = [vp, ci, ci, ctypes.POINTER(sz), ctypes.POINTER(sz)]
    L.starkv_compress_append.argtypes = [vp, ctypes.POINTER(_Cache), vp, ci, ci, ctypes.POINTER(ctypes.c_int32), vp,
                                         vp]
    L.starkv_decode_workspace_bytes.argtypes = [vp, ci, ci, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(sz)]
    L.starkv_decode_attention.argtypes = [vp, ctypes.POINTER(_Cache), vp, ci, ci, ctypes.POINTER(ctypes.c_int32),
                                          vp, vp, vp, sz, vp]
    L.starkv_decode_step.argtypes = [vp, ctypes.POINTER(_Cache), vp, vp, ci, ci, ctypes.POINTER(ctypes.c_int32),
                                     vp, vp, vp, sz, vp]
    L.starkv_decode_step_noalloc.argtypes = [vp, ctypes.POINTER(_Cache), vp, vp, ci, ci,
                                             ctypes.POINTER(ctypes.c_int32), vp, vp, vp]
    L.starkv_layer_set_rope.argtypes = [vp, ctypes.c_float, ci]
    L.starkv_prefill_workspace_bytes.argtypes = [vp, ci, ci, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(sz)]
    L.starkv_prefill_attention.argtypes = [vp, ctypes.POINTER(_Cache), vp, ci, ci, ctypes.POINTER(ctypes.c_int32),
                                           vp, vp, sz, vp]
    L.starkv_absorb_query.argtypes = [vp, vp, vp]
    L.starkv_decode_attention_hidden.argtypes = [vp, ctypes.POINTER(_Cache), vp, ci, ci,
                                                 ctypes.POINTER(ctypes.c_int32), vp, vp, vp, sz, vp]
    L.starkv_reconstruct.argtypes = [vp, ctypes.POINTER(_Cache), ci, ci, ci, vp, vp, vp]
    L.starkv_profile_enable.argtypes = [ci]
    L.starkv_profile_read.argtypes = [ctypes.POINTER(_KernelTime), ci, ctypes.POINTER(ci), ci]
    for name in EXPORTS:
        if name not in ("starkv_abi_version", "starkv_status_string"):
            getattr(L, name).restype = ci
    _lib = L
    return L


def profile_enable(on: bool = True) -> None:
    """Bracket every libstarkv kernel launch with HIP events on its stream (measurement only)."""
    _check(lib().starkv_profile_enable(1 if on else 0), "starkv_profile_enable")


def profile_read(reset: bool = True) -> dict:
    """{kernel name: (launches, total ms)} of the launches timed since the last reset."""
    buf = (_KernelTime * 64)()
    n = ctypes.c_int()
    _check(lib().starkv_profile_read(buf, 64, ctypes.byref(n), 1 if reset else 0), "starkv_profile_read")
    return {buf[i].name.decode(): (buf[i].launches, buf[i].total_ms) for i in range(min(n.value, 64))}


def _check(status: int, what: str) -> None:
    if status != 0:
        raise StarKVError(status, what)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(t) -> int:
    return int(t.data_ptr())


def _need(cond: bool, what: str) -> None:
    """Argument check of the binding (shapes, dtypes, devices): a mismatch would make the
    kernels read or write past the caller's buffers, so it is refused before the call."""
    if not cond:
        raise ValueError(what)


def _lens(lens, B: int) -> np.ndarray:
    L = _i32(lens).reshape(-1)
    _need(L.shape[0] == B, f"lens has {L.shape[0]} entries for a batch of {B}")
    return L


def _on_device(t, like) -> bool:
    return t.is_cuda and t.device == like.device


def _lens_dev(lens_dev, B: int, like):
    """Device lengths (int32 [B] on the device of the inputs), or None (0 for the call)."""
    if lens_dev is None:
        return None
    import torch
    _need(isinstance(lens_dev, torch.Tensor) and lens_dev.dtype == torch.int32 and lens_dev.is_contiguous() and
          tuple(lens_dev.shape) == (B,), f"lens_dev: contiguous int32 tensor [{B}] expected")
    _need(_on_device(lens_dev, like), f"lens_dev must be on {like.device}")
    return _ptr(lens_dev)


def _stream(stream=None) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


class Cache:
    """Caller-owned cache buffers of one layer (torch uint8 tensors on the device)."""

    def __init__(self, k_rows, v_tiles, B: int, T_max: int):
        self.k_rows = k_rows
        self.v_tiles = v_tiles
        self.B = B
        self.T_max = T_max

    def struct(self) -> _Cache:
        return _Cache(_ptr(self.k_rows), _ptr(self.v_tiles), self.B, self.T_max)

    def seq(self, b: int) -> "Cache":
        """A one-sequence view of sequence b (same memory)."""
        kb = self.k_rows.numel() // self.B
        vb = self.v_tiles.numel() // self.B
        return Cache(self.k_rows[b * kb:(b + 1) * kb], self.v_tiles[b * vb:(b + 1) * vb], 1, self.T_max)


class Layer:
    """One decoder layer's low-rank, quantised KV cache path (a libstarkv layer handle)."""

    def __init__(self, H_q: int, H_kv: int, d_h: int, d: int, dtype: str, latent: str, s_k, tau_k, s_v, tau_v,
                 shrink: bool = True, device: Optional[str] = None):
        self._lib = lib()
        self.dtype = dtype
        self.latent = latent
        self._s_k = _f32(s_k).reshape(H_kv, d_h)
        self._tau_k = _f32(tau_k).reshape(H_kv)
        self._s_v = _f32(s_v).reshape(-1)
        desc = _Desc(H_q, H_kv, d_h, d, DTYPE[dtype], LATENT[latent], 1 if shrink else 0, len(self._s_v),
                     self._s_k.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                     self._tau_k.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                     self._s_v.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), float(np.float32(tau_v)))
        h = ctypes.c_void_p()
        _check(self._lib.starkv_layer_create(ctypes.byref(desc), ctypes.byref(h)), "starkv_layer_create")
        self._h = h
        info = _Info()
        _check(self._lib.starkv_layer_get_info(h, ctypes.byref(info)), "starkv_layer_get_info")
        self.info = {f: getattr(info, f) for f, _ in _Info._fields_}
        r = np.zeros(H_kv + 1, dtype=np.int32)
        _check(self._lib.starkv_layer_ranks(h, r.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))), "starkv_layer_ranks")
        self.ranks = r[:H_kv].copy()
        self.r_v = int(r[H_kv])
        self.H_q, self.H_kv, self.d_h, self.d = H_q, H_kv, d_h, d
        self.A_t = self.B_k = self.B_vt = self.scales = None
        self._ws = None
        self._ws_memo = None  # (B, n_q, lens bytes) -> workspace bytes of the last query
        self._cb_memo = {}  # (B, T_max) -> cache bytes

    # -- lifecycle
    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            self._lib.starkv_layer_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def torch_dtype(self):
        import torch
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    # -- factors and scales
    def build_factors(self, U_k, V_k, U_v, V_v, stream=None):
        """Truncated factors from fp32 device SVD factors; returns (A_t, B_k, B_vt)."""
        import torch
        dev = U_k.device
        n_lat, n_key = self.info["n_lat"], self.info["n_key"]
        self.A_t = torch.empty((n_lat, self.d), dtype=self.torch_dtype, device=dev)
        self.B_k = torch.empty((n_key, self.d_h), dtype=self.torch_dtype, device=dev)
        self.B_vt = torch.empty((self.H_kv * self.d_h, self.r_v), dtype=self.torch_dtype, device=dev)
        n_v = len(self._s_v)
        for t, shape in ((U_k, (self.H_kv, self.d, self.d_h)), (V_k, (self.H_kv, self.d_h, self.d_h)),
                         (U_v, (self.d, n_v)), (V_v, (self.H_kv * self.d_h, n_v))):
            _need(t.dtype == torch.float32 and t.is_contiguous() and _on_device(t, U_k) and tuple(t.shape) == shape,
                  f"SVD factor: contiguous float32 device tensor {shape} expected, got {tuple(t.shape)}")
        _check(self._lib.starkv_build_factors(self._h, _ptr(U_k), _ptr(V_k), _ptr(U_v), _ptr(V_v), _ptr(self.A_t),
                                              _ptr(self.B_k), _ptr(self.B_vt), _stream(stream)), "starkv_build_factors")
        return self.A_t, self.B_k, self.B_vt

    def bind_factors(self, A_t, B_k, B_vt) -> None:
        for t, shape in ((A_t, (self.info["n_lat"], self.d)), (B_k, (self.info["n_key"], self.d_h)),
                         (B_vt, (self.H_kv * self.d_h, self.r_v))):
            _need(t.dtype == self.torch_dtype and t.is_contiguous() and t.is_cuda and tuple(t.shape) == shape,
                  f"factor: contiguous {self.torch_dtype} device tensor {shape} expected, got {tuple(t.shape)}")
        self.A_t, self.B_k, self.B_vt = A_t, B_k, B_vt
        _check(self._lib.starkv_bind_factors(self._h, _ptr(A_t), _ptr(B_k), _ptr(B_vt)), "starkv_bind_factors")

    def calibrate(self, X_cal, stream=None):
        """Per-channel fp16 scales from calibration hidden states [n_cal, d] (mix84, had43, had43p)."""
        import torch
        _need(X_cal.dtype == self.torch_dtype and X_cal.is_contiguous() and X_cal.is_cuda and X_cal.dim() == 2 and
              int(X_cal.shape[1]) == self.d, f"X_cal: contiguous {self.torch_dtype} device tensor [n_cal, {self.d}] expected")
        self.scales = torch.empty((self.info["n_lat"],), dtype=torch.float16, device=X_cal.device)
        _check(self._lib.starkv_calibrate(self._h, _ptr(X_cal), int(X_cal.shape[0]), _ptr(self.scales),
                                          _stream(stream)), "starkv_calibrate")
        return self.scales

    def bind_scales(self, scales) -> None:
        import torch
        _need(scales.dtype == torch.float16 and scales.is_contiguous() and scales.is_cuda and
              scales.numel() == self.info["n_lat"], f"scales: contiguous float16 device tensor [{self.info['n_lat']}] expected")
        self.scales = scales
        _check(self._lib.starkv_bind_scales(self._h, _ptr(scales)), "starkv_bind_scales")

    # -- cache
    def cache_bytes(self, B: int, T_max: int) -> Tuple[int, int]:
        kb, vb = ctypes.c_size_t(), ctypes.c_size_t()
        _check(self._lib.starkv_cache_bytes(self._h, B, T_max, ctypes.byref(kb), ctypes.byref(vb)), "starkv_cache_bytes")
        return kb.value, vb.value

    def new_cache(self, B: int, T_max: int, device="cuda", zero: bool = False) -> Cache:
        import torch
        T_max = -(-T_max // TILE_TOKENS) * TILE_TOKENS
        kb, vb = self.cache_bytes(B, T_max)
        mk = torch.zeros if zero else torch.empty
        return Cache(mk((kb,), dtype=torch.uint8, device=device), mk((vb,), dtype=torch.uint8, device=device), B, T_max)

    def _check_cache(self, cache: Cache, like) -> None:
        key = (cache.B, cache.T_max)
        if key not in self._cb_memo:
            self._cb_memo[key] = self.cache_bytes(cache.B, cache.T_max)
        kb, vb = self._cb_memo[key]
        _need(cache.k_rows.numel() * cache.k_rows.element_size() >= kb and
              cache.v_tiles.numel() * cache.v_tiles.element_size() >= vb, "cache buffers smaller than its layout")
        _need(_on_device(cache.k_rows, like) and _on_device(cache.v_tiles, like), "cache on another device")

    def _check_q(self, q, what: str = "q"):
        _need(q.dtype == self.torch_dtype and q.is_contiguous() and q.dim() == 4,
              f"{what}: contiguous {self.torch_dtype} tensor [B, n_q, H_q, d_h] expected")
        _need(tuple(q.shape[2:]) == (self.H_q, self.d_h), f"{what} shape {tuple(q.shape)}: heads and head dim "
              f"must be ({self.H_q}, {self.d_h})")
        _need(q.is_cuda, f"{what} must be a device tensor")
        return int(q.shape[0]), int(q.shape[1])

    def _out(self, out, shape, like):
        import torch
        if out is None:
            return torch.empty(shape, dtype=self.torch_dtype, device=like.device)
        _need(out.dtype == self.torch_dtype and out.is_contiguous() and tuple(out.shape) == tuple(shape) and
              _on_device(out, like), f"out: contiguous {self.torch_dtype} tensor {tuple(shape)} on {like.device} expected")
        return out

    def _workspace(self, ws, need: int, like):
        import torch
        if ws is None:
            if self._ws is None or self._ws.numel() < need or self._ws.device != like.device:
                self._ws = torch.empty((max(need, 256),), dtype=torch.uint8, device=like.device)
            return self._ws
        _need(ws.is_contiguous() and _on_device(ws, like), "ws: contiguous tensor on the device of the inputs")
        return ws

    def append(self, cache: Cache, X_new, lens: Sequence[int], stream=None, lens_dev=None) -> None:
        """Project X_new [B, n_new, d] into the latent and store it after position lens[b] (with
        lens_dev, an int32 device tensor [B]: after min(lens_dev[b], lens[b]) as the kernels read it)."""
        _need(X_new.dtype == self.torch_dtype and X_new.is_contiguous() and X_new.dim() == 3,
              f"X_new: contiguous {self.torch_dtype} tensor [B, n_new, d] expected")
        _need(int(X_new.shape[2]) == self.d, f"X_new shape {tuple(X_new.shape)}: hidden size must be {self.d}")
        B, n_new = int(X_new.shape[0]), int(X_new.shape[1])
        L = _lens(lens, B)
        _need(X_new.is_cuda, "X_new must be a device tensor")
        ld = _lens_dev(lens_dev, B, X_new)
        self._check_cache(cache, X_new)
        cs = cache.struct()
        _check(self._lib.starkv_compress_append(self._h, ctypes.byref(cs), _ptr(X_new), B, n_new,
                                                L.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), ld, _stream(stream)),
               "starkv_compress_append")

    # -- decode
    def workspace_bytes(self, B: int, n_q: int, lens: Sequence[int]) -> int:
        L = _lens(lens, B)
        key = (B, n_q, L.tobytes())
        if self._ws_memo is not None and self._ws_memo[0] == key:
            return self._ws_memo[1]
        n = ctypes.c_size_t()
        _check(self._lib.starkv_decode_workspace_bytes(self._h, B, n_q, L.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                                       ctypes.byref(n)), "starkv_decode_workspace_bytes")
        self._ws_memo = (key, n.value)
        return n.value

    def decode(self, cache: Cache, q, lens: Sequence[int], out=None, ws=None, stream=None, lens_dev=None):
        """Attention of q [B, n_q, H_q, d_h] over the cache (lens include the n_q query tokens).
        lens_dev: None, or int32 device lengths [B] read when the kernels run; lens is then their
        upper bound (it sizes the plan and the workspace)."""
        _need(q.dim() == 4, "q: tensor [B, n_q, H_q, d_h] expected")
        L = _lens(lens, int(q.shape[0]))
        B, n_q = self._check_q(q)
        ld = _lens_dev(lens_dev, B, q)
        self._check_cache(cache, q)
        need = self.workspace_bytes(B, n_q, L)
        ws = self._workspace(ws, need, q)
        out = self._out(out, q.shape, q)
        cs = cache.struct()
        _check(self._lib.starkv_decode_attention(self._h, ctypes.byref(cs), _ptr(q), B, n_q,
                                                 L.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), ld, _ptr(out),
                                                 _ptr(ws),
                                                 int(ws.numel() * ws.element_size()), _stream(stream)),
               "starkv_decode_attention")
        return out

    def absorb_query(self, W_q, stream=None) -> None:
        """Absorb the key factors into the query projection W_q [d, H_q * d_h] (device, layer dtype)."""
        _need(W_q.dtype == self.torch_dtype and W_q.is_contiguous() and W_q.is_cuda and
              tuple(W_q.shape) == (self.d, self.H_q * self.d_h),
              f"W_q: contiguous {self.torch_dtype} device tensor {(self.d, self.H_q * self.d_h)} expected")
        _check(self._lib.starkv_absorb_query(self._h, _ptr(W_q), _stream(stream)), "starkv_absorb_query")

    def decode_hidden(self, cache: Cache, x, lens: Sequence[int], out=None, ws=None, stream=None, lens_dev=None):
        """Attention with the query taken from hidden states x [B, n_q, d] through the absorbed
        query factors; returns out [B, n_q, H_q, d_h]."""
        _need(x.dtype == self.torch_dtype and x.is_contiguous() and x.dim() == 3,
              f"x: contiguous {self.torch_dtype} tensor [B, n_q, d] expected")
        _need(int(x.shape[2]) == self.d, f"x shape {tuple(x.shape)}: hidden size must be {self.d}")
        B, n_q = int(x.shape[0]), int(x.shape[1])
        L = _lens(lens, B)
        _need(x.is_cuda, "x must be a device tensor")
        ld = _lens_dev(lens_dev, B, x)
        self._check_cache(cache, x)
        need = self.workspace_bytes(B, n_q, L)
        ws = self._workspace(ws, need, x)
        out = self._out(out, (B, n_q, self.H_q, self.d_h), x)
        cs = cache.struct()
        _check(self._lib.starkv_decode_attention_hidden(self._h, ctypes.byref(cs), _ptr(x), B, n_q,
                                                        L.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), ld,
                                                        _ptr(out),
                                                        _ptr(ws), int(ws.numel() * ws.element_size()),
                                                        _stream(stream)),
               "starkv_decode_attention_hidden")
        return out

    def step(self, cache: Cache, X_new, q, lens: Sequence[int], out=None, ws=None, stream=None, lens_dev=None):
        """One decode step: append X_new [B, n_q, d] at lens - n_q, then attention of q
        [B, n_q, H_q, d_h] over lens (the lengths after the append).  lens_dev: as for decode."""
        _need(q.dim() == 4, "q: tensor [B, n_q, H_q, d_h] expected")
        B, n_q = int(q.shape[0]), int(q.shape[1])
        _need(X_new.dtype == self.torch_dtype and X_new.is_contiguous(),
              f"X_new: contiguous {self.torch_dtype} tensor expected")
        _need(tuple(X_new.shape) == (B, n_q, self.d), f"X_new shape {tuple(X_new.shape)}, expected {(B, n_q, self.d)}")
        L = _lens(lens, B)
        self._check_q(q)
        _need(_on_device(X_new, q), f"X_new must be on {q.device}")
        ld = _lens_dev(lens_dev, B, q)
        self._check_cache(cache, q)
        need = self.workspace_bytes(B, n_q, L)
        ws = self._workspace(ws, need, q)
        out = self._out(out, q.shape, q)
        cs = cache.struct()
        _check(self._lib.starkv_decode_step(self._h, ctypes.byref(cs), _ptr(X_new), _ptr(q), B, n_q,
                                            L.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), ld, _ptr(out),
                                            _ptr(ws),
                                            int(ws.numel() * ws.element_size()), _stream(stream)),
               "starkv_decode_step")
        return out

    def step_noalloc(self, cache: Cache, X_new, q, lens: Sequence[int], out, stream=None, lens_dev=None):
        """starkv_decode_step with the library's static device scratch instead of a workspace: the
        call allocates no device memory (``out`` [B, n_q, H_q, d_h] is the caller's).  Calls that
        overlap on one GPU share the scratch and must be serialised."""
        _need(q.dim() == 4, "q: tensor [B, n_q, H_q, d_h] expected")
        B, n_q = int(q.shape[0]), int(q.shape[1])
        _need(X_new.dtype == self.torch_dtype and X_new.is_contiguous(),
              f"X_new: contiguous {self.torch_dtype} tensor expected")
        _need(tuple(X_new.shape) == (B, n_q, self.d), f"X_new shape {tuple(X_new.shape)}, expected {(B, n_q, self.d)}")
        L = _lens(lens, B)
        self._check_q(q)
        _need(_on_device(X_new, q), f"X_new must be on {q.device}")
        ld = _lens_dev(lens_dev, B, q)
        self._check_cache(cache, q)
        _need(out is not None, "out must be given (the call allocates nothing)")
        out = self._out(out, q.shape, q)
        cs = cache.struct()
        _check(self._lib.starkv_decode_step_noalloc(self._h, ctypes.byref(cs), _ptr(X_new), _ptr(q), B, n_q,
                                                    L.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), ld, _ptr(out),
                                                    _stream(stream)),
               "starkv_decode_step_noalloc")
        return out

    def set_rope(self, theta: float, rotary_dim: Optional[int] = None) -> None:
        """Rotate keys and queries by position (theta: the base; rotary_dim: d_h, or 0 to turn the
        rotation off).  Decode of a rotary layer attends over reconstructed keys."""
        rd = self.d_h if rotary_dim is None else int(rotary_dim)
        _check(self._lib.starkv_layer_set_rope(self._h, float(theta), rd), "starkv_layer_set_rope")
        self._ws_memo = None

    def prefill_workspace_bytes(self, B: int, n_q: int, lens: Sequence[int]) -> int:
        L = _lens(lens, B)
        n = ctypes.c_size_t()
        _check(self._lib.starkv_prefill_workspace_bytes(self._h, B, n_q, L.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                                        ctypes.byref(n)), "starkv_prefill_workspace_bytes")
        return n.value

    def prefill(self, cache: Cache, q, lens: Sequence[int], out=None, ws=None, stream=None):
        """Attention of a query chunk q [B, n_q, H_q, d_h] (positions lens[b] - n_q ..) over keys
        and values reconstructed from the cache; any n_q up to the lengths."""
        _need(q.dim() == 4, "q: tensor [B, n_q, H_q, d_h] expected")
        L = _lens(lens, int(q.shape[0]))
        B, n_q = self._check_q(q)
        self._check_cache(cache, q)
        need = self.prefill_workspace_bytes(B, n_q, L)
        if ws is None:
            import torch
            ws = torch.empty((max(need, 256),), dtype=torch.uint8, device=q.device)
        else:
            _need(ws.is_contiguous() and _on_device(ws, q), "ws: contiguous tensor on the device of the inputs")
        out = self._out(out, q.shape, q)
        cs = cache.struct()
        _check(self._lib.starkv_prefill_attention(self._h, ctypes.byref(cs), _ptr(q), B, n_q,
                                                  L.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), _ptr(out),
                                                  _ptr(ws), int(ws.numel() * ws.element_size()), _stream(stream)),
               "starkv_prefill_attention")
        return out

    def reconstruct(self, cache: Cache, b: int, t0: int, t1: int, stream=None):
        """Dense K, V [t1 - t0, H_kv, d_h] rebuilt from the latent of sequence b."""
        import torch
        self._check_cache(cache, cache.k_rows)
        K = torch.empty((t1 - t0, self.H_kv, self.d_h), dtype=self.torch_dtype, device=cache.k_rows.device)
        V = torch.empty_like(K)
        cs = cache.struct()
        _check(self._lib.starkv_reconstruct(self._h, ctypes.byref(cs), b, t0, t1, _ptr(K), _ptr(V), _stream(stream)),
               "starkv_reconstruct")
        return K, V
