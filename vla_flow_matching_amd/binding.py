"""ctypes binding of libae.so (include/ae.h), argument marshalling only.

Every step of the denoise loop runs in the library's HIP kernels; this module
only turns torch tensors into device pointers and the current torch stream
into a hipStream_t.  There is no CPU fallback: without the built library
``load()`` raises.
"""

from __future__ import annotations

import atexit
import ctypes
import os
import sys
import weakref
from typing import Dict, Optional, Sequence

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libae.so")

AE_OK, AE_ERR_INVALID_ARGUMENT, AE_ERR_SHAPE_MISMATCH, AE_ERR_NOT_READY = 0, 1, 2, 3
AE_ERR_OUT_OF_MEMORY, AE_ERR_UNSUPPORTED, AE_ERR_HIP = 4, 5, 6
AE_F32, AE_BF16, AE_FP8_E4M3 = 0, 1, 2
AE_BLOCK_JOINT, AE_BLOCK_DIT = 0, 1
AE_PATH_AUTO, AE_PATH_WHOLE_CALL, AE_PATH_PER_PHASE = 0, 1, 2

# every function include/ae.h declares
EXPORTS = ("ae_create", "ae_load_weights", "ae_set_prefix_kv", "ae_prepare_prefix", "ae_set_prefix_buckets",
           "ae_denoise", "ae_denoise_static", "ae_get_stats", "ae_last_error", "ae_status_string", "ae_destroy")


class Config(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int), ("width", ctypes.c_int), ("n_q_heads", ctypes.c_int),
        ("n_kv_heads", ctypes.c_int), ("head_dim", ctypes.c_int), ("mlp_dim", ctypes.c_int),
        ("action_horizon", ctypes.c_int), ("action_dim", ctypes.c_int),
        ("max_prefix_len", ctypes.c_int), ("max_batch", ctypes.c_int), ("max_steps", ctypes.c_int),
        ("act_dtype", ctypes.c_int), ("proj_weight_dtype", ctypes.c_int),
        ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float), ("use_graphs", ctypes.c_int),
        ("graph_cache_size", ctypes.c_int), ("graph_cache_evict", ctypes.c_int),
        ("context_width", ctypes.c_int), ("state_dim", ctypes.c_int), ("block_type", ctypes.c_int),
        ("fp8_rowwise", ctypes.c_int), ("fp8_oproj", ctypes.c_int), ("exec_path", ctypes.c_int),
    ]


class TensorView(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("data", ctypes.c_void_p), ("ndim", ctypes.c_int),
                ("shape", ctypes.c_longlong * 4), ("dtype", ctypes.c_int)]


class Stats(ctypes.Structure):
    _fields_ = [("denoise_calls", ctypes.c_longlong), ("prefix_sets", ctypes.c_longlong),
                ("graph_captures", ctypes.c_longlong), ("graph_replays", ctypes.c_longlong),
                ("eager_runs", ctypes.c_longlong), ("device_bytes", ctypes.c_longlong),
                ("device_errors", ctypes.c_longlong), ("persistent", ctypes.c_longlong),
                ("persistent_calls", ctypes.c_longlong), ("graph_hits", ctypes.c_longlong),
                ("graph_misses", ctypes.c_longlong), ("graph_evictions", ctypes.c_longlong),
                ("graphs_cached", ctypes.c_longlong), ("prefix_bucket", ctypes.c_longlong),
                ("graph_nodes", ctypes.c_longlong)]


class AeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


_lib: Optional[ctypes.CDLL] = None


def load() -> ctypes.CDLL:
    """Load libae.so and declare its signatures; raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m vla_flow_matching_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, ci = ctypes.c_void_p, ctypes.c_int
    lib.ae_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(vp)]
    lib.ae_load_weights.argtypes = [vp, ctypes.POINTER(TensorView), ci, vp]
    lib.ae_set_prefix_kv.argtypes = [vp, ci, ci, vp, vp, vp, vp]
    lib.ae_set_prefix_buckets.argtypes = [vp, ctypes.POINTER(ci), ci]
    lib.ae_prepare_prefix.argtypes = [vp, ci, ci, vp, vp, vp, vp]
    lib.ae_denoise.argtypes = [vp, vp, ci, ci, vp, vp]
    lib.ae_denoise_static.argtypes = [vp, vp, ci, ci, vp, vp]
    lib.ae_get_stats.argtypes = [vp, ctypes.POINTER(Stats)]
    lib.ae_last_error.argtypes = [vp]
    lib.ae_last_error.restype = ctypes.c_char_p
    lib.ae_status_string.argtypes = [ci]
    lib.ae_status_string.restype = ctypes.c_char_p
    lib.ae_destroy.argtypes = [vp]
    lib.ae_destroy.restype = None
    for f in ("ae_create", "ae_load_weights", "ae_set_prefix_kv", "ae_prepare_prefix", "ae_set_prefix_buckets",
              "ae_denoise", "ae_denoise_static", "ae_get_stats"):
        getattr(lib, f).restype = ci
    _lib = lib
    return lib


def make_config(w, max_batch: Optional[int] = None, max_prefix_len: Optional[int] = None,
                max_steps: Optional[int] = None, use_graphs: bool = True,
                graph_cache_size: int = 16, graph_cache_evict: bool = True,
                context_width: int = 0, state_dim: int = 0, exec_path: int = 0) -> Config:
    """Config from any object with the workload fields (e.g. synth.Workload);
    exec_path: AE_PATH_AUTO (0), AE_PATH_WHOLE_CALL (1) or AE_PATH_PER_PHASE (2)."""
    act = AE_BF16 if w.dtype == "bf16" else AE_F32
    proj = AE_FP8_E4M3 if getattr(w, "proj_dtype", "same") == "fp8" else act
    return Config(w.n_layers, w.width, w.n_q_heads, w.n_kv_heads, w.head_dim, w.mlp_dim,
                  w.action_horizon, w.action_dim,
                  w.prefix_len if max_prefix_len is None else max_prefix_len,
                  w.batch if max_batch is None else max_batch,
                  w.n_steps if max_steps is None else max_steps,
                  act, proj, float(w.rope_theta), float(w.rms_eps), int(bool(use_graphs)),
                  int(graph_cache_size), int(bool(graph_cache_evict)), int(context_width), int(state_dim),
                  AE_BLOCK_DIT if getattr(w, "block", "joint") == "dit" else AE_BLOCK_JOINT,
                  int(proj == AE_FP8_E4M3 and getattr(w, "fp8_scaling", "tensor") == "rowwise"),
                  int(proj == AE_FP8_E4M3 and bool(getattr(w, "fp8_o", False))), int(exec_path))


def _stream_ptr(stream) -> ctypes.c_void_p:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return AE_BF16
    if t.dtype == torch.float32:
        return AE_F32
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def _dev(t, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _expect(t, name: str, shape, dtype):
    """Raise AeError(AE_ERR_SHAPE_MISMATCH) unless t has this shape and dtype.

    The C ABI receives bare pointers, so a short or mistyped buffer would be
    read past its end on the device; the binding checks what the config
    implies before handing the pointer over."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise AeError(AE_ERR_SHAPE_MISMATCH,
                      f"{name}: expected {tuple(shape)} {dtype}, got {tuple(t.shape)} {t.dtype}")


# Handles still open, closed in creation order at interpreter exit while the
# HIP runtime is still up (a finaliser running later, during teardown, would
# call into a runtime that may already be shut down).
_open_handles: "weakref.WeakSet[ActionExpert]" = weakref.WeakSet()


@atexit.register
def _close_all():
    for ex in list(_open_handles):
        ex.close()


class ActionExpert:
    """One library handle: weights, prefix K/V and the denoise loop."""

    def __init__(self, cfg: Config):
        self.lib = load()
        self.cfg = cfg
        self.h = None
        h = ctypes.c_void_p()
        st = self.lib.ae_create(ctypes.byref(cfg), ctypes.byref(h))
        if st != AE_OK:
            raise AeError(st, "ae_create: " + self.lib.ae_status_string(st).decode())
        self.h = h
        self.prefix_batch = None
        _open_handles.add(self)

    def _act_dtype(self):
        import torch
        return torch.bfloat16 if self.cfg.act_dtype == AE_BF16 else torch.float32

    def _check(self, st: int, what: str):
        if st != AE_OK:
            raise AeError(st, f"{what}: {self.lib.ae_last_error(self.h).decode()}")

    def load_weights(self, weights: Dict[str, "object"], stream=None):
        views = (TensorView * len(weights))()
        keep = []
        for i, (name, t) in enumerate(weights.items()):
            b = name.encode()
            keep.append(b)
            views[i].name = b
            views[i].data = _dev(t, name)
            views[i].ndim = t.dim()
            for d in range(min(4, t.dim())):
                views[i].shape[d] = t.shape[d]
            views[i].dtype = _dtype_code(t)
        self._check(self.lib.ae_load_weights(self.h, views, len(weights), _stream_ptr(stream)),
                    "ae_load_weights")

    def set_prefix_kv(self, K, V, mask, stream=None):
        """K, V [L, B, P, Hkv, dh] device tensors in the activation dtype; mask
        [B, P] uint8 device tensor."""
        import torch
        if mask.dim() != 2:
            raise AeError(AE_ERR_SHAPE_MISMATCH, f"mask: expected [batch, prefix_len], got {tuple(mask.shape)}")
        B, P = int(mask.shape[0]), int(mask.shape[1])
        c = self.cfg
        if P == 0:
            nullp = ctypes.c_void_p()
            st = self.lib.ae_set_prefix_kv(self.h, B, 0, nullp, nullp, nullp, _stream_ptr(stream))
        else:
            kv_shape = (c.n_layers, B, P, c.n_kv_heads, c.head_dim)
            _expect(K, "K", kv_shape, self._act_dtype())
            _expect(V, "V", kv_shape, self._act_dtype())
            _expect(mask, "mask", (B, P), torch.uint8)
            st = self.lib.ae_set_prefix_kv(self.h, B, P, _dev(K, "K"), _dev(V, "V"), _dev(mask, "mask"),
                                           _stream_ptr(stream))
        self._check(st, "ae_set_prefix_kv")
        self.prefix_batch = B

    def prepare_prefix(self, hidden, mask, state=None, stream=None):
        """hidden [L, B, P, context_width] bf16, mask [B, P] uint8, state
        [B, state_dim] fp32 or None; device tensors."""
        import torch
        c = self.cfg
        if mask.dim() != 2:
            raise AeError(AE_ERR_SHAPE_MISMATCH, f"mask: expected [batch, prefix_len], got {tuple(mask.shape)}")
        B, P = int(mask.shape[0]), int(mask.shape[1])
        nullp = ctypes.c_void_p()
        hp = mp = nullp
        if P > 0:
            _expect(hidden, "hidden", (c.n_layers, B, P, c.context_width), torch.bfloat16)
            _expect(mask, "mask", (B, P), torch.uint8)
            hp, mp = _dev(hidden, "hidden"), _dev(mask, "mask")
        sp = nullp
        if state is not None:
            _expect(state, "state", (B, c.state_dim), torch.float32)
            sp = _dev(state, "state")
        self._check(self.lib.ae_prepare_prefix(self.h, B, P, hp, mp, sp, _stream_ptr(stream)),
                    "ae_prepare_prefix")
        self.prefix_batch = B

    def set_prefix_buckets(self, lengths: Sequence[int]):
        """Prefix-length buckets (strictly increasing, each <= max_prefix_len)."""
        arr = (ctypes.c_int * max(1, len(lengths)))(*[int(v) for v in lengths])
        self._check(self.lib.ae_set_prefix_buckets(self.h, arr, len(lengths)), "ae_set_prefix_buckets")

    def denoise(self, noise, steps: int, out=None, stream=None, static_scratch: bool = False):
        """noise [B, T, A] fp32 device tensor -> actions (new tensor unless
        ``out``).  static_scratch: the allocation-free entry point
        (ae_denoise_static), for callers that cannot allocate."""
        import torch
        c = self.cfg
        if noise.dim() != 3:
            raise AeError(AE_ERR_SHAPE_MISMATCH, f"noise: expected [batch, T, A], got {tuple(noise.shape)}")
        B = int(noise.shape[0])
        _expect(noise, "noise", (B, c.action_horizon, c.action_dim), torch.float32)
        if out is None:
            out = torch.empty_like(noise)
        _expect(out, "out", (B, c.action_horizon, c.action_dim), torch.float32)
        fn = self.lib.ae_denoise_static if static_scratch else self.lib.ae_denoise
        st = fn(self.h, _dev(noise, "noise"), B, int(steps), _dev(out, "out"), _stream_ptr(stream))
        self._check(st, "ae_denoise_static" if static_scratch else "ae_denoise")
        return out

    def stats(self) -> Dict[str, int]:
        s = Stats()
        self._check(self.lib.ae_get_stats(self.h, ctypes.byref(s)), "ae_get_stats")
        return {f: getattr(s, f) for f, _ in Stats._fields_}

    def close(self):
        """Release the handle (synchronises the device).  Idempotent."""
        if getattr(self, "h", None):
            self.lib.ae_destroy(self.h)
            self.h = None
        _open_handles.discard(self)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        # At interpreter shutdown the HIP runtime (and a profiler attached to
        # it) may already be torn down; the atexit hook has closed every
        # handle by then, so a finaliser that runs late does nothing.
        if sys is None or sys.is_finalizing():
            return
        try:
            self.close()
        except Exception:
            pass


def weights_to_device(weights: Dict[str, "object"], dtype: str, device="cuda"):
    """Host fp32 arrays (already bf16-representable for bf16) -> device tensors."""
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return {k: torch.from_numpy(v).to(device=device, dtype=tdt).contiguous() for k, v in weights.items()}
