"""ctypes binding of libae.so (include/ae.h), argument marshalling only.

Every step of the denoise loop runs in the library's HIP kernels; this module
only turns torch tensors into device pointers and the current torch stream
into a hipStream_t.  There is no CPU fallback: without the built library
``load()`` raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libae.so")

AE_OK, AE_ERR_INVALID_ARGUMENT, AE_ERR_SHAPE_MISMATCH, AE_ERR_NOT_READY = 0, 1, 2, 3
AE_ERR_OUT_OF_MEMORY, AE_ERR_UNSUPPORTED, AE_ERR_HIP = 4, 5, 6
AE_F32, AE_BF16, AE_FP8_E4M3 = 0, 1, 2

# every function include/ae.h declares
EXPORTS = ("ae_create", "ae_load_weights", "ae_set_prefix_kv", "ae_denoise", "ae_get_stats",
           "ae_last_error", "ae_status_string", "ae_destroy")


class Config(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int), ("width", ctypes.c_int), ("n_q_heads", ctypes.c_int),
        ("n_kv_heads", ctypes.c_int), ("head_dim", ctypes.c_int), ("mlp_dim", ctypes.c_int),
        ("action_horizon", ctypes.c_int), ("action_dim", ctypes.c_int),
        ("max_prefix_len", ctypes.c_int), ("max_batch", ctypes.c_int), ("max_steps", ctypes.c_int),
        ("act_dtype", ctypes.c_int), ("proj_weight_dtype", ctypes.c_int),
        ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float), ("use_graphs", ctypes.c_int),
    ]


class TensorView(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("data", ctypes.c_void_p), ("ndim", ctypes.c_int),
                ("shape", ctypes.c_longlong * 4), ("dtype", ctypes.c_int)]


class Stats(ctypes.Structure):
    _fields_ = [("denoise_calls", ctypes.c_longlong), ("prefix_sets", ctypes.c_longlong),
                ("graph_captures", ctypes.c_longlong), ("graph_replays", ctypes.c_longlong),
                ("eager_runs", ctypes.c_longlong), ("device_bytes", ctypes.c_longlong),
                ("device_errors", ctypes.c_longlong), ("persistent", ctypes.c_longlong)]


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
    lib.ae_denoise.argtypes = [vp, vp, ci, ci, vp, vp]
    lib.ae_get_stats.argtypes = [vp, ctypes.POINTER(Stats)]
    lib.ae_last_error.argtypes = [vp]
    lib.ae_last_error.restype = ctypes.c_char_p
    lib.ae_status_string.argtypes = [ci]
    lib.ae_status_string.restype = ctypes.c_char_p
    lib.ae_destroy.argtypes = [vp]
    lib.ae_destroy.restype = None
    for f in ("ae_create", "ae_load_weights", "ae_set_prefix_kv", "ae_denoise", "ae_get_stats"):
        getattr(lib, f).restype = ci
    _lib = lib
    return lib


def make_config(w, max_batch: Optional[int] = None, max_prefix_len: Optional[int] = None,
                max_steps: Optional[int] = None, use_graphs: bool = True) -> Config:
    """Config from any object with the workload fields (e.g. synth.Workload)."""
    act = AE_BF16 if w.dtype == "bf16" else AE_F32
    proj = AE_FP8_E4M3 if getattr(w, "proj_dtype", "same") == "fp8" else act
    return Config(w.n_layers, w.width, w.n_q_heads, w.n_kv_heads, w.head_dim, w.mlp_dim,
                  w.action_horizon, w.action_dim,
                  w.prefix_len if max_prefix_len is None else max_prefix_len,
                  w.batch if max_batch is None else max_batch,
                  w.n_steps if max_steps is None else max_steps,
                  act, proj, float(w.rope_theta), float(w.rms_eps), int(bool(use_graphs)))


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


class ActionExpert:
    """One library handle: weights, prefix K/V and the denoise loop."""

    def __init__(self, cfg: Config):
        self.lib = load()
        self.cfg = cfg
        h = ctypes.c_void_p()
        st = self.lib.ae_create(ctypes.byref(cfg), ctypes.byref(h))
        if st != AE_OK:
            raise AeError(st, "ae_create: " + self.lib.ae_status_string(st).decode())
        self.h = h

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
        """K, V [L, B, P, Hkv, dh] device tensors; mask [B, P] uint8 device tensor."""
        B, P = int(mask.shape[0]), int(mask.shape[1])
        if P == 0:
            nullp = ctypes.c_void_p()
            st = self.lib.ae_set_prefix_kv(self.h, B, 0, nullp, nullp, nullp, _stream_ptr(stream))
        else:
            st = self.lib.ae_set_prefix_kv(self.h, B, P, _dev(K, "K"), _dev(V, "V"), _dev(mask, "mask"),
                                           _stream_ptr(stream))
        self._check(st, "ae_set_prefix_kv")

    def denoise(self, noise, steps: int, out=None, stream=None):
        """noise [B, T, A] fp32 device tensor -> actions (new tensor unless ``out``)."""
        import torch
        if noise.dtype != torch.float32:
            raise TypeError("noise must be float32")
        if out is None:
            out = torch.empty_like(noise)
        st = self.lib.ae_denoise(self.h, _dev(noise, "noise"), int(noise.shape[0]), int(steps),
                                 _dev(out, "out"), _stream_ptr(stream))
        self._check(st, "ae_denoise")
        return out

    def stats(self) -> Dict[str, int]:
        s = Stats()
        self._check(self.lib.ae_get_stats(self.h, ctypes.byref(s)), "ae_get_stats")
        return {f: getattr(s, f) for f, _ in Stats._fields_}

    def close(self):
        if getattr(self, "h", None):
            self.lib.ae_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def weights_to_device(weights: Dict[str, "object"], dtype: str, device="cuda"):
    """Host fp32 arrays (already bf16-representable for bf16) -> device tensors."""
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return {k: torch.from_numpy(v).to(device=device, dtype=tdt).contiguous() for k, v in weights.items()}
