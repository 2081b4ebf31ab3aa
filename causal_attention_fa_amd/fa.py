"""ctypes binding of libfa.so (include/fa.h), plus thin torch conveniences.

The functions named like the C entry points (fa_fwd, fa_bwd, rope_apply,
rope_apply_bwd and their _f32 twins, fa_layer_window, fa_rope_inv_freq,
fa_last_error) only marshal arguments: a tensor argument is passed as its
device pointer, sizes as C ints, the stream as the HIP stream handle (the
current torch stream when omitted).  A negative return code raises FAError
with the library's message.  Every step of the computation runs in the HIP
kernels; there is no fallback: importing this module without the built
library raises.

The convenience wrappers (attention_forward, attention_backward, rope,
FlashAttention) allocate outputs with torch and call the same entry points.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np
import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(
        f"{_LIB_PATH} is missing: build it with `python -m causal_attention_fa_amd.build` "
        "(the HIP library is required; there is no CPU fallback)")
_lib = ctypes.CDLL(_LIB_PATH)

FA_OK = 0
FA_ERR_INVALID_ARG = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_HIP = -3

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float

_ATTN_FWD = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _F, _P]
_ATTN_BWD = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _F, _P]
_ROPE = [_P, _P, _P, _I, _I, _I, _I, _P]

for _name, _args in [("fa_fwd", _ATTN_FWD), ("fa_fwd_f32", _ATTN_FWD),
                     ("fa_bwd", _ATTN_BWD), ("fa_bwd_f32", _ATTN_BWD),
                     ("fa_bwd_noalloc", _ATTN_BWD),
                     ("rope_apply", _ROPE), ("rope_apply_bwd", _ROPE),
                     ("rope_apply_f32", _ROPE), ("rope_apply_bwd_f32", _ROPE)]:
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _I
_lib.fa_fwd_sink.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _F, _P]
_lib.fa_fwd_sink.restype = _I
_lib.fa_bwd_sink.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F,
                             _I, _I, _F, _P]
_lib.fa_bwd_sink.restype = _I
_lib.fa_fwd_rope.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _F, _P]
_lib.fa_fwd_rope.restype = _I
_lib.fa_bwd_rope.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I,
                             _I, _F, _P]
_lib.fa_bwd_rope.restype = _I
_lib.fa_fwd_vdim.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _F, _P]
_lib.fa_fwd_vdim.restype = _I
_lib.fa_bwd_vdim.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I,
                             _I, _F, _P]
_lib.fa_bwd_vdim.restype = _I
_lib.fa_decode.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _F, _P]
_lib.fa_decode.restype = _I
_lib.fa_decode_splits.argtypes = [_I, _I, _I, _I, ctypes.POINTER(_I), ctypes.POINTER(_I)]
_lib.fa_decode_splits.restype = _I
_lib.fa_layer_window.argtypes = [_I, _I, _I]
_lib.fa_layer_window.restype = _I
_lib.fa_rope_inv_freq.argtypes = [ctypes.POINTER(ctypes.c_float), _I, ctypes.c_double]
_lib.fa_rope_inv_freq.restype = _I
_lib.fa_rope_inv_freq_llama3.argtypes = [ctypes.POINTER(ctypes.c_float), _I, ctypes.c_double,
                                         ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                         ctypes.c_double]
_lib.fa_rope_inv_freq_llama3.restype = _I
_lib.fa_layer_rope_theta.argtypes = [_I, ctypes.c_double, ctypes.c_double, _I,
                                     ctypes.POINTER(ctypes.c_double)]
_lib.fa_layer_rope_theta.restype = _I
_lib.fa_set_stage_events.argtypes = [ctypes.POINTER(ctypes.c_void_p), _I]
_lib.fa_set_stage_events.restype = _I
_lib.fa_bwd_kernels.argtypes = [_I, _I]
_lib.fa_bwd_kernels.restype = ctypes.c_char_p
_lib.fa_bwd_workspace.argtypes = [_I, _I, _I, _I, _I, _I, ctypes.POINTER(ctypes.c_size_t),
                                  ctypes.POINTER(_I), ctypes.POINTER(_I)]
_lib.fa_bwd_workspace.restype = _I
_lib.fa_set_dq_mode.argtypes = [_I]
_lib.fa_set_dq_mode.restype = _I
_lib.fa_measure_dq_atomics.argtypes = [_I, _I, _I, _I, _I, _I, ctypes.POINTER(ctypes.c_float)]
_lib.fa_measure_dq_atomics.restype = _I
_lib.fa_last_error.argtypes = []
_lib.fa_last_error.restype = ctypes.c_char_p

EXPORTS = ("fa_fwd", "fa_bwd", "fa_bwd_noalloc", "fa_fwd_sink", "fa_bwd_sink", "fa_fwd_vdim", "fa_bwd_vdim",
           "fa_fwd_rope", "fa_bwd_rope",
           "fa_decode", "fa_decode_splits", "rope_apply", "rope_apply_bwd", "fa_fwd_f32",
           "fa_bwd_f32", "rope_apply_f32", "rope_apply_bwd_f32", "fa_layer_window", "fa_rope_inv_freq",
           "fa_rope_inv_freq_llama3", "fa_layer_rope_theta", "fa_set_stage_events",
           "fa_bwd_kernels", "fa_bwd_workspace", "fa_set_dq_mode", "fa_measure_dq_atomics", "fa_last_error")


class FAError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


def library_path() -> str:
    return _LIB_PATH


def fa_last_error() -> str:
    return _lib.fa_last_error().decode()


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.data_ptr()
    return int(x)


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(rc: int):
    if rc != FA_OK:
        raise FAError(rc, fa_last_error())
    return rc


def _call_fwd(fn, q, k, v, o, lse, B, H, Hkv, T, d, scale, window, global_every, softcap,
              stream):
    return _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, T, d,
                     float(scale), window, global_every, float(softcap), _stream(stream)))


def _call_bwd(fn, q, k, v, o, lse, dO, dq, dk, dv, B, H, Hkv, T, d, scale, window,
              global_every, softcap, stream):
    return _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq),
                     _ptr(dk), _ptr(dv), B, H, Hkv, T, d, float(scale), window, global_every,
                     float(softcap), _stream(stream)))


def fa_fwd(q, k, v, o, lse, B, H, Hkv, T, d, scale, window=0, global_every=0, softcap=0.0,
           stream=None):
    return _call_fwd(_lib.fa_fwd, q, k, v, o, lse, B, H, Hkv, T, d, scale, window,
                     global_every, softcap, stream)


def fa_fwd_f32(q, k, v, o, lse, B, H, Hkv, T, d, scale, window=0, global_every=0,
               softcap=0.0, stream=None):
    return _call_fwd(_lib.fa_fwd_f32, q, k, v, o, lse, B, H, Hkv, T, d, scale, window,
                     global_every, softcap, stream)


def fa_bwd(q, k, v, o, lse, dO, dq, dk, dv, B, H, Hkv, T, d, scale, window=0, global_every=0,
           softcap=0.0, stream=None):
    return _call_bwd(_lib.fa_bwd, q, k, v, o, lse, dO, dq, dk, dv, B, H, Hkv, T, d, scale,
                     window, global_every, softcap, stream)


def fa_bwd_f32(q, k, v, o, lse, dO, dq, dk, dv, B, H, Hkv, T, d, scale, window=0,
               global_every=0, softcap=0.0, stream=None):
    return _call_bwd(_lib.fa_bwd_f32, q, k, v, o, lse, dO, dq, dk, dv, B, H, Hkv, T, d, scale,
                     window, global_every, softcap, stream)


def fa_bwd_noalloc(q, k, v, o, lse, dO, dq, dk, dv, B, H, Hkv, T, d, scale, window=0,
                   global_every=0, softcap=0.0, stream=None):
    return _call_bwd(_lib.fa_bwd_noalloc, q, k, v, o, lse, dO, dq, dk, dv, B, H, Hkv, T, d,
                     scale, window, global_every, softcap, stream)


def fa_fwd_sink(q, k, v, o, lse, sinks, max_logit, B, H, Hkv, T, d, scale, window=0,
                global_every=0, softcap=0.0, stream=None):
    return _check(_lib.fa_fwd_sink(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(sinks),
                                   _ptr(max_logit), B, H, Hkv, T, d, float(scale), window,
                                   global_every, float(softcap), _stream(stream)))


def fa_bwd_sink(q, k, v, o, lse, dO, sinks, dq, dk, dv, dsinks, B, H, Hkv, T, d, scale,
                window=0, global_every=0, softcap=0.0, stream=None):
    return _check(_lib.fa_bwd_sink(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO),
                                   _ptr(sinks), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dsinks), B, H,
                                   Hkv, T, d, float(scale), window, global_every, float(softcap),
                                   _stream(stream)))


def fa_fwd_rope(q, k, v, o, lse, inv_freq, q_rot, B, H, Hkv, T, d, scale, window=0,
                global_every=0, softcap=0.0, stream=None):
    return _check(_lib.fa_fwd_rope(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(inv_freq),
                                   _ptr(q_rot), B, H, Hkv, T, d, float(scale), window,
                                   global_every, float(softcap), _stream(stream)))


def fa_bwd_rope(q_rot, k, v, o, lse, dO, inv_freq, dq, dk, dv, B, H, Hkv, T, d, scale,
                window=0, global_every=0, softcap=0.0, stream=None):
    return _check(_lib.fa_bwd_rope(_ptr(q_rot), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO),
                                   _ptr(inv_freq), _ptr(dq), _ptr(dk), _ptr(dv), B, H, Hkv, T, d,
                                   float(scale), window, global_every, float(softcap),
                                   _stream(stream)))


def fa_fwd_vdim(q, k, v, o, lse, B, H, Hkv, T, d, d_v, scale, window=0, global_every=0,
                softcap=0.0, stream=None):
    return _check(_lib.fa_fwd_vdim(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, T,
                                   d, d_v, float(scale), window, global_every, float(softcap),
                                   _stream(stream)))


def fa_bwd_vdim(q, k, v, o, lse, dO, dq, dk, dv, B, H, Hkv, T, d, d_v, scale, window=0,
                global_every=0, softcap=0.0, stream=None):
    return _check(_lib.fa_bwd_vdim(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO),
                                   _ptr(dq), _ptr(dk), _ptr(dv), B, H, Hkv, T, d, d_v,
                                   float(scale), window, global_every, float(softcap),
                                   _stream(stream)))


def fa_decode(q, k_cache, v_cache, lens, o, lse, sinks, B, H, Hkv, S, d, scale, window=0,
              softcap=0.0, stream=None):
    return _check(_lib.fa_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(lens), _ptr(o),
                                 _ptr(lse), _ptr(sinks), B, H, Hkv, S, d, float(scale), window,
                                 float(softcap), _stream(stream)))


def fa_bwd_kernels(d, d_v=None):
    """Names of the kernels the bf16 backward launches for (d, d_v), in order."""
    r = _lib.fa_bwd_kernels(d, d if d_v is None else d_v)
    if r is None:
        raise FAError(FA_ERR_UNSUPPORTED, f"fa_bwd_kernels: unsupported head sizes ({d}, {d_v})")
    return r.decode().split(",")


def fa_bwd_workspace(B, H, T, d, d_v=None, window=0):
    """(bytes, query tiles per head, band slots per query tile) of the dS
    workspace the bf16 backward takes for these sizes under the current dQ
    mode (bytes 0: the recomputing dQ pass runs)."""
    nb, nq, nk = ctypes.c_size_t(), _I(), _I()
    _check(_lib.fa_bwd_workspace(B, H, T, d, d if d_v is None else d_v, window,
                                 ctypes.byref(nb), ctypes.byref(nq), ctypes.byref(nk)))
    return nb.value, nq.value, nk.value


def fa_set_dq_mode(mode):
    """Process-wide dQ strategy of the bf16 backward (0: dQ from stored dS
    where it applies, 1: the recomputing dQ pass); returns the previous one."""
    r = _lib.fa_set_dq_mode(int(mode))
    if r < 0:
        _check(r)
    return r


def fa_measure_dq_atomics(B, H, Hkv, T, d, window=0):
    """ms of only the float atomics that accumulating dQ inside the dK/dV
    pass would issue for this shape (best of three; synchronous)."""
    ms = ctypes.c_float(0.0)
    _check(_lib.fa_measure_dq_atomics(B, H, Hkv, T, d, window, ctypes.byref(ms)))
    return ms.value


def fa_decode_splits(B, Hkv, S, window=0):
    """(nsplit, chunk) fa_decode uses for these sizes."""
    ns, ch = _I(), _I()
    _check(_lib.fa_decode_splits(B, Hkv, S, window, ctypes.byref(ns), ctypes.byref(ch)))
    return ns.value, ch.value


def _rope_call(fn, x, y, inv_freq, B, H, T, d, stream):
    return _check(fn(_ptr(x), _ptr(y), _ptr(inv_freq), B, H, T, d, _stream(stream)))


def rope_apply(x, y, inv_freq, B, H, T, d, stream=None):
    return _rope_call(_lib.rope_apply, x, y, inv_freq, B, H, T, d, stream)


def rope_apply_bwd(dy, dx, inv_freq, B, H, T, d, stream=None):
    return _rope_call(_lib.rope_apply_bwd, dy, dx, inv_freq, B, H, T, d, stream)


def rope_apply_f32(x, y, inv_freq, B, H, T, d, stream=None):
    return _rope_call(_lib.rope_apply_f32, x, y, inv_freq, B, H, T, d, stream)


def rope_apply_bwd_f32(dy, dx, inv_freq, B, H, T, d, stream=None):
    return _rope_call(_lib.rope_apply_bwd_f32, dy, dx, inv_freq, B, H, T, d, stream)


def fa_layer_window(layer: int, window: int, global_every: int) -> int:
    r = _lib.fa_layer_window(layer, window, global_every)
    if r < 0:
        raise FAError(r, fa_last_error())
    return r


def fa_rope_inv_freq(d: int, theta: float) -> np.ndarray:
    out = np.zeros(max(d // 2, 1), dtype=np.float32)
    _check(_lib.fa_rope_inv_freq(out.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), d,
                                 float(theta)))
    return out[: d // 2]


def fa_rope_inv_freq_llama3(d: int, theta: float, factor: float, low_freq_factor: float = 1.0,
                            high_freq_factor: float = 4.0, orig_ctx: float = 8192.0) -> np.ndarray:
    out = np.zeros(max(d // 2, 1), dtype=np.float32)
    _check(_lib.fa_rope_inv_freq_llama3(out.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), d,
                                        float(theta), float(factor), float(low_freq_factor),
                                        float(high_freq_factor), float(orig_ctx)))
    return out[: d // 2]


def fa_layer_rope_theta(layer: int, theta: float, theta_global: float, global_every: int) -> float:
    out = ctypes.c_double(0.0)
    _check(_lib.fa_layer_rope_theta(layer, float(theta), float(theta_global), global_every,
                                    ctypes.byref(out)))
    return out.value


def fa_set_stage_events(events):
    """Arm per-kernel stage events (a list of hipEvent_t handles as ints);
    an empty list disarms."""
    arr = (ctypes.c_void_p * max(len(events), 1))(*[int(e) for e in events])
    return _check(_lib.fa_set_stage_events(arr, len(events)))


# ------------------------------------------------------------ conveniences

def _dims(q, k):
    B, H, T, d = q.shape
    Hkv = k.shape[1]
    return B, H, Hkv, T, d


def _need(t, dtype):
    if not (t.is_cuda and t.is_contiguous() and t.dtype == dtype):
        raise ValueError("expected contiguous device tensors of dtype " + str(dtype))


def attention_forward(q, k, v, scale=None, window=0, global_every=0, softcap=0.0,
                      stream=None):
    """o, lse = attention(q [B,H,T,d], k/v [B,Hkv,T,d]) on the device."""
    B, H, Hkv, T, d = _dims(q, k)
    dt = q.dtype
    for t in (q, k, v):
        _need(t, dt)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    o = torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    fn = fa_fwd_f32 if dt == torch.float32 else fa_fwd
    fn(q, k, v, o, lse, B, H, Hkv, T, d, scale, window, global_every, softcap, stream)
    return o, lse


def attention_backward(q, k, v, o, lse, do, scale=None, window=0, global_every=0,
                       softcap=0.0, stream=None):
    B, H, Hkv, T, d = _dims(q, k)
    dt = q.dtype
    for t in (q, k, v, o, do):
        _need(t, dt)
    _need(lse, torch.float32)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    fn = fa_bwd_f32 if dt == torch.float32 else fa_bwd
    fn(q, k, v, o, lse, do, dq, dk, dv, B, H, Hkv, T, d, scale, window, global_every, softcap,
       stream)
    return dq, dk, dv


def rope(x, inv_freq, out=None, backward=False, stream=None):
    """RoPE of x [B,H,T,d] with a device fp32 table [d/2]; out may be x."""
    B, H, T, d = x.shape
    y = torch.empty_like(x) if out is None else out
    if x.dtype == torch.float32:
        fn = rope_apply_bwd_f32 if backward else rope_apply_f32
    else:
        fn = rope_apply_bwd if backward else rope_apply
    fn(x, y, inv_freq, B, H, T, d, stream)
    return y


class FlashAttention(torch.autograd.Function):
    """torch.autograd wrapper: forward = fa_fwd, backward = fa_bwd."""

    @staticmethod
    def forward(ctx, q, k, v, scale, window, softcap):
        o, lse = attention_forward(q, k, v, scale, window, 0, softcap)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.cfg = (scale, window, softcap)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        scale, window, softcap = ctx.cfg
        dq, dk, dv = attention_backward(q, k, v, o, lse, do.contiguous(), scale, window, 0,
                                        softcap)
        return dq, dk, dv, None, None, None
