"""Thin Python binding of the C ABI in ``include/h2o.h`` (``libh2o.so``).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, and their ``data_ptr()`` and the current HIP stream are passed
through.  Every step of the H2O path runs in the library's gfx950 kernels;
there is no fallback, and importing this module fails loudly when the built
library is missing (``python -m kv_cache_eviction_amd.build_lib`` builds it).

The functions carry the names of the C entry points.  ``H2OCache`` is a
convenience owner of the state tensors (cache K/V, scores, positions and the
workspace), allocated with torch, which is used for device memory and streams
only.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libh2o.so")

H2O_OK, H2O_ERR_NULL, H2O_ERR_CONFIG, H2O_ERR_SHAPE, H2O_ERR_STATE = 0, 1, 2, 3, 4
H2O_ERR_WORKSPACE, H2O_ERR_HIP, H2O_ERR_UNSUPPORTED, H2O_ERR_ALIGN, H2O_ERR_TOO_LARGE = 5, 6, 7, 8, 9
H2O_BF16, H2O_FP32 = 0, 1
POLICIES = {"h2o": 0, "recent": 1, "sink_recent": 2}
KERNEL_IDS = {"attn_fwd": 0, "score": 1, "select": 2, "reset": 3, "scatter": 4}

EXPORTED = [
    "h2o_validate_config", "h2o_workspace_bytes", "h2o_cache_init", "h2o_prefill",
    "h2o_chunk_step", "h2o_get_scores", "h2o_chunk_backward", "h2o_backward_workspace_bytes",
    "h2o_chunk_backward_static",
    "h2o_recurrence_backward_step", "h2o_recurrence_workspace_bytes",
    "h2o_tokens_seen", "h2o_device_status", "h2o_set_timing", "h2o_get_timing",
    "h2o_cache_destroy", "h2o_status_str", "h2o_last_hip_error",
]


class H2OConfigC(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("cache_slots", ctypes.c_int32),
        ("recent_window", ctypes.c_int32), ("max_chunk", ctypes.c_int32),
        ("max_prefill", ctypes.c_int32), ("dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
        ("policy", ctypes.c_int32), ("n_sink", ctypes.c_int32),
    ]


class H2OError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_str(status)} (status {status})")


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run `python -m kv_cache_eviction_amd.build_lib`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, I64, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    cfgp = ctypes.POINTER(H2OConfigC)
    sig = {
        "h2o_validate_config": (I32, [cfgp]),
        "h2o_workspace_bytes": (SZ, [cfgp]),
        "h2o_cache_init": (I32, [cfgp, P, P, P, P, P, SZ, I32, I64, P, ctypes.POINTER(P)]),
        "h2o_prefill": (I32, [P, P, P, P, I32, P, P, P]),
        "h2o_chunk_step": (I32, [P, P, P, P, I32, P, P, P, P, P, P, P, P]),
        "h2o_get_scores": (I32, [P, P, P, P]),
        "h2o_chunk_backward": (I32, [cfgp, P, P, P, P, P, P, I32, P, P, P, P, P, P, P, P, P, SZ, P]),
        "h2o_backward_workspace_bytes": (SZ, [cfgp, I32]),
        "h2o_chunk_backward_static": (I32, [cfgp, P, P, P, P, P, P, I32, P, P, P, P, P, P, P, P, P]),
        "h2o_recurrence_backward_step": (I32, [cfgp, P, P, P, P, P, P, P, P, P, P, I32, P, P, P, P, P, P, P,
                                               P, P, SZ, P]),
        "h2o_recurrence_workspace_bytes": (SZ, [cfgp, I32]),
        "h2o_tokens_seen": (I64, [P]),
        "h2o_device_status": (I32, [P, P, ctypes.POINTER(I32)]),
        "h2o_set_timing": (I32, [P, I32]),
        "h2o_get_timing": (I32, [P, I32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I64)]),
        "h2o_cache_destroy": (None, [P]),
        "h2o_status_str": (ctypes.c_char_p, [I32]),
        "h2o_last_hip_error": (I32, [P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def library_path() -> str:
    return _LIB_PATH


def status_str(s: int) -> str:
    return _lib.h2o_status_str(s).decode()


@dataclass(frozen=True)
class H2OConfig:
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    cache_slots: int
    recent_window: int
    max_chunk: int
    max_prefill: int
    dtype: str = "bf16"           # "bf16" | "fp32"
    softmax_scale: float = 0.0    # <= 0: 1/sqrt(head_dim)
    policy: str = "h2o"           # "h2o" | "recent" | "sink_recent"
    n_sink: int = 0               # sink_recent: positions below n_sink are kept

    def c(self) -> H2OConfigC:
        return H2OConfigC(self.batch, self.n_q_heads, self.n_kv_heads, self.head_dim,
                          self.cache_slots, self.recent_window, self.max_chunk, self.max_prefill,
                          H2O_BF16 if self.dtype == "bf16" else H2O_FP32, self.softmax_scale,
                          POLICIES.get(self.policy, -1), self.n_sink)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


def _check(status: int, what: str):
    if status != H2O_OK:
        raise H2OError(status, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _expect(t, name, shape, dtype, allow_none=False):
    if t is None:
        if allow_none:
            return
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.data_ptr() % 16:
        raise ValueError(f"{name} must start at a 16-byte aligned address")


def h2o_validate_config(cfg: H2OConfig) -> int:
    c = cfg.c()
    return _lib.h2o_validate_config(ctypes.byref(c))


def h2o_workspace_bytes(cfg: H2OConfig) -> int:
    c = cfg.c()
    return _lib.h2o_workspace_bytes(ctypes.byref(c))


def h2o_backward_workspace_bytes(cfg: H2OConfig, s: int) -> int:
    c = cfg.c()
    return _lib.h2o_backward_workspace_bytes(ctypes.byref(c), s)


def h2o_cache_init(cfg: H2OConfig, k_cache, v_cache, scores, positions, workspace,
                   adopt: bool = False, tokens_seen: int = 0, stream=None):
    B, Hkv, M, d = cfg.batch, cfg.n_kv_heads, cfg.cache_slots, cfg.head_dim
    _expect(k_cache, "k_cache", (B, Hkv, M, d), cfg.torch_dtype)
    _expect(v_cache, "v_cache", (B, Hkv, M, d), cfg.torch_dtype)
    _expect(scores, "scores", (B, Hkv, M), torch.float32)
    _expect(positions, "positions", (B, Hkv, M), torch.int32)
    if (workspace.dtype != torch.uint8 or not workspace.is_cuda or not workspace.is_contiguous()
            or workspace.data_ptr() % 16):
        raise ValueError("workspace must be a contiguous, 16-byte aligned uint8 device tensor")
    c = cfg.c()
    handle = ctypes.c_void_p()
    _check(_lib.h2o_cache_init(ctypes.byref(c), _ptr(k_cache), _ptr(v_cache), _ptr(scores),
                               _ptr(positions), _ptr(workspace), workspace.numel(), int(adopt),
                               int(tokens_seen), _stream(stream), ctypes.byref(handle)),
           "h2o_cache_init")
    return handle


def h2o_prefill(handle, cfg: H2OConfig, q, k, v, out, lse=None, stream=None):
    B, Hq, Hkv, d = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    n = q.shape[2]
    _expect(q, "q", (B, Hq, n, d), cfg.torch_dtype)
    _expect(k, "k", (B, Hkv, n, d), cfg.torch_dtype)
    _expect(v, "v", (B, Hkv, n, d), cfg.torch_dtype)
    _expect(out, "out", (B, Hq, n, d), cfg.torch_dtype)
    _expect(lse, "lse", (B, Hq, n), torch.float32, allow_none=True)
    _check(_lib.h2o_prefill(handle, _ptr(q), _ptr(k), _ptr(v), n, _ptr(out), _ptr(lse), _stream(stream)),
           "h2o_prefill")


def h2o_chunk_step(handle, cfg: H2OConfig, q, k_new, v_new, out, lse=None, slots_out=None,
                   step_mass=None, k_old=None, v_old=None, pos_old=None, stream=None):
    B, Hq, Hkv, d, M = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.cache_slots
    s = q.shape[2]
    _expect(q, "q", (B, Hq, s, d), cfg.torch_dtype)
    _expect(k_new, "k_new", (B, Hkv, s, d), cfg.torch_dtype)
    _expect(v_new, "v_new", (B, Hkv, s, d), cfg.torch_dtype)
    _expect(out, "out", (B, Hq, s, d), cfg.torch_dtype)
    _expect(lse, "lse", (B, Hq, s), torch.float32, allow_none=True)
    _expect(slots_out, "slots_out", (B, Hkv, s), torch.int32, allow_none=True)
    _expect(step_mass, "step_mass", (B, Hkv, M + s), torch.float32, allow_none=True)
    _expect(k_old, "k_old", (B, Hkv, s, d), cfg.torch_dtype, allow_none=True)
    _expect(v_old, "v_old", (B, Hkv, s, d), cfg.torch_dtype, allow_none=True)
    _expect(pos_old, "pos_old", (B, Hkv, s), torch.int32, allow_none=True)
    _check(_lib.h2o_chunk_step(handle, _ptr(q), _ptr(k_new), _ptr(v_new), s, _ptr(out), _ptr(lse),
                               _ptr(slots_out), _ptr(step_mass), _ptr(k_old), _ptr(v_old),
                               _ptr(pos_old), _stream(stream)), "h2o_chunk_step")


def h2o_get_scores(handle, scores_out, positions_out=None, stream=None):
    _check(_lib.h2o_get_scores(handle, _ptr(scores_out), _ptr(positions_out), _stream(stream)),
           "h2o_get_scores")


def _check_backward_args(cfg, q, k_cache, v_cache, positions, k_new, v_new, out, lse, d_out, dq, dk_cache,
                         dv_cache, dk_new, dv_new):
    B, Hq, Hkv, d, M = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.cache_slots
    s = q.shape[2]
    dt = cfg.torch_dtype
    for t, name, shp, ty in [
        (q, "q", (B, Hq, s, d), dt), (k_cache, "k_cache", (B, Hkv, M, d), dt),
        (v_cache, "v_cache", (B, Hkv, M, d), dt), (positions, "positions", (B, Hkv, M), torch.int32),
        (k_new, "k_new", (B, Hkv, s, d), dt), (v_new, "v_new", (B, Hkv, s, d), dt),
        (out, "out", (B, Hq, s, d), dt), (lse, "lse", (B, Hq, s), torch.float32),
        (d_out, "d_out", (B, Hq, s, d), dt), (dq, "dq", (B, Hq, s, d), dt),
        (dk_cache, "dk_cache", (B, Hkv, M, d), dt), (dv_cache, "dv_cache", (B, Hkv, M, d), dt),
        (dk_new, "dk_new", (B, Hkv, s, d), dt), (dv_new, "dv_new", (B, Hkv, s, d), dt)]:
        _expect(t, name, shp, ty)
    return s


def h2o_chunk_backward(cfg: H2OConfig, q, k_cache, v_cache, positions, k_new, v_new, out, lse, d_out,
                       dq, dk_cache, dv_cache, dk_new, dv_new, workspace, stream=None):
    s = _check_backward_args(cfg, q, k_cache, v_cache, positions, k_new, v_new, out, lse, d_out, dq,
                             dk_cache, dv_cache, dk_new, dv_new)
    c = cfg.c()
    ws_bytes = 0 if workspace is None else workspace.numel()
    _check(_lib.h2o_chunk_backward(ctypes.byref(c), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(positions),
                                   _ptr(k_new), _ptr(v_new), s, _ptr(out), _ptr(lse), _ptr(d_out), _ptr(dq),
                                   _ptr(dk_cache), _ptr(dv_cache), _ptr(dk_new), _ptr(dv_new),
                                   _ptr(workspace), ws_bytes, _stream(stream)), "h2o_chunk_backward")


def h2o_chunk_backward_static(cfg: H2OConfig, q, k_cache, v_cache, positions, k_new, v_new, out, lse, d_out,
                              dq, dk_cache, dv_cache, dk_new, dv_new, stream=None):
    """h2o_chunk_backward with the library's static scratch: no workspace, no allocation."""
    s = _check_backward_args(cfg, q, k_cache, v_cache, positions, k_new, v_new, out, lse, d_out, dq,
                             dk_cache, dv_cache, dk_new, dv_new)
    c = cfg.c()
    _check(_lib.h2o_chunk_backward_static(ctypes.byref(c), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                          _ptr(positions), _ptr(k_new), _ptr(v_new), s, _ptr(out), _ptr(lse),
                                          _ptr(d_out), _ptr(dq), _ptr(dk_cache), _ptr(dv_cache), _ptr(dk_new),
                                          _ptr(dv_new), _stream(stream)), "h2o_chunk_backward_static")


def h2o_recurrence_workspace_bytes(cfg: H2OConfig, s: int) -> int:
    c = cfg.c()
    return _lib.h2o_recurrence_workspace_bytes(ctypes.byref(c), s)


def h2o_recurrence_backward_step(cfg: H2OConfig, k_cache, v_cache, positions, slots, k_old, v_old,
                                 pos_old, q, k_new, v_new, out, lse, d_out, acc_k, acc_v, dq, gk, gv,
                                 workspace, stream=None):
    B, Hq, Hkv, d, M = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.cache_slots
    s = q.shape[2]
    dt, f32, i32 = cfg.torch_dtype, torch.float32, torch.int32
    for t, name, shp, ty in [
        (k_cache, "k_cache", (B, Hkv, M, d), dt), (v_cache, "v_cache", (B, Hkv, M, d), dt),
        (positions, "positions", (B, Hkv, M), i32), (slots, "slots", (B, Hkv, s), i32),
        (k_old, "k_old", (B, Hkv, s, d), dt), (v_old, "v_old", (B, Hkv, s, d), dt),
        (pos_old, "pos_old", (B, Hkv, s), i32), (q, "q", (B, Hq, s, d), dt),
        (k_new, "k_new", (B, Hkv, s, d), dt), (v_new, "v_new", (B, Hkv, s, d), dt),
        (out, "out", (B, Hq, s, d), dt), (lse, "lse", (B, Hq, s), f32), (d_out, "d_out", (B, Hq, s, d), dt),
        (acc_k, "acc_k", (B, Hkv, M, d), f32), (acc_v, "acc_v", (B, Hkv, M, d), f32),
        (dq, "dq", (B, Hq, s, d), dt), (gk, "gk", (B, Hkv, s, d), f32), (gv, "gv", (B, Hkv, s, d), f32)]:
        _expect(t, name, shp, ty)
    c = cfg.c()
    ws_bytes = 0 if workspace is None else workspace.numel()
    _check(_lib.h2o_recurrence_backward_step(
        ctypes.byref(c), _ptr(k_cache), _ptr(v_cache), _ptr(positions), _ptr(slots), _ptr(k_old),
        _ptr(v_old), _ptr(pos_old), _ptr(q), _ptr(k_new), _ptr(v_new), s, _ptr(out), _ptr(lse), _ptr(d_out),
        _ptr(acc_k), _ptr(acc_v), _ptr(dq), _ptr(gk), _ptr(gv), _ptr(workspace), ws_bytes,
        _stream(stream)), "h2o_recurrence_backward_step")


def h2o_tokens_seen(handle) -> int:
    return _lib.h2o_tokens_seen(handle)


def h2o_device_status(handle, stream=None) -> int:
    """Device status word (bit 0: an adopted state had too few evictable
    slots; bit 1: the select's bounded wait gave up), cleared by the read."""
    flags = ctypes.c_int32()
    _check(_lib.h2o_device_status(handle, _stream(stream), ctypes.byref(flags)), "h2o_device_status")
    return flags.value


def h2o_set_timing(handle, kernels=True):
    """Brackets the selected kernels' launches with HIP events: True (all),
    False (none), or an iterable of kernel names / ids."""
    if kernels is True:
        mask = -1
    elif kernels is False or kernels is None:
        mask = 0
    else:
        mask = 0
        for k in kernels:
            mask |= 1 << (KERNEL_IDS[k] if isinstance(k, str) else int(k))
    _check(_lib.h2o_set_timing(handle, mask), "h2o_set_timing")


def h2o_get_timing(handle, kernel: str | int):
    kid = KERNEL_IDS[kernel] if isinstance(kernel, str) else kernel
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(_lib.h2o_get_timing(handle, kid, ctypes.byref(ms), ctypes.byref(n)), "h2o_get_timing")
    return ms.value, n.value


def h2o_cache_destroy(handle):
    _lib.h2o_cache_destroy(handle)


def h2o_last_hip_error(handle) -> int:
    return _lib.h2o_last_hip_error(handle)


class H2OCache:
    """Owns the device state of one H2O cache and drives the C ABI on it."""

    def __init__(self, cfg: H2OConfig, device="cuda", adopt_state=None, tokens_seen: int = 0,
                 stream=None):
        _check(h2o_validate_config(cfg), "h2o_validate_config")
        self.cfg = cfg
        B, Hkv, M, d = cfg.batch, cfg.n_kv_heads, cfg.cache_slots, cfg.head_dim
        if adopt_state is None:
            self.k_cache = torch.zeros((B, Hkv, M, d), dtype=cfg.torch_dtype, device=device)
            self.v_cache = torch.zeros_like(self.k_cache)
            self.scores = torch.empty((B, Hkv, M), dtype=torch.float32, device=device)
            self.positions = torch.empty((B, Hkv, M), dtype=torch.int32, device=device)
        else:
            self.k_cache, self.v_cache, self.scores, self.positions = adopt_state
        self.workspace = torch.empty(h2o_workspace_bytes(cfg), dtype=torch.uint8, device=device)
        self.handle = h2o_cache_init(cfg, self.k_cache, self.v_cache, self.scores, self.positions,
                                     self.workspace, adopt=adopt_state is not None,
                                     tokens_seen=tokens_seen, stream=stream)

    def prefill(self, q, k, v, out=None, lse=None, stream=None):
        if out is None:
            out = torch.empty_like(q)
        h2o_prefill(self.handle, self.cfg, q, k, v, out, lse, stream)
        return out

    def chunk_step(self, q, k_new, v_new, out=None, lse=None, slots_out=None, step_mass=None,
                   k_old=None, v_old=None, pos_old=None, stream=None):
        if out is None:
            out = torch.empty_like(q)
        h2o_chunk_step(self.handle, self.cfg, q, k_new, v_new, out, lse, slots_out, step_mass,
                       k_old, v_old, pos_old, stream)
        return out

    def get_scores(self, stream=None):
        s = torch.empty_like(self.scores)
        p = torch.empty_like(self.positions)
        h2o_get_scores(self.handle, s, p, stream)
        return s, p

    @property
    def tokens_seen(self) -> int:
        return h2o_tokens_seen(self.handle)

    def close(self):
        if getattr(self, "handle", None) is not None:
            h2o_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
