"""MI355X (gfx950) library for causal grouped-query attention with rotary
position embedding over a key/value cache: prefill and cached decode.

The compute runs in hand-written HIP kernels inside ``librgc.so`` (C ABI in
``include/rgc.h``).  This module is a thin ctypes binding with the same
names: it checks that tensors live on the GPU, passes their pointers,
strides and torch's current stream, and turns a negative status into an
exception.  It never computes anything itself and there is no fallback: if
the library is missing or no GPU is present, every call raises.

    import rope_gqa_causal_amd as rgc
    rgc.rope_apply(q, pos0)                   # in place, q [B,S,Hq,D]
    rgc.kv_cache_append(kc, vc, k, v, lens)   # caches [B,Hkv,S_max,D]
    o = rgc.gqa_attn_prefill(q, kc, vc, q_start)
    o = rgc.gqa_attn_decode(q1, kc, vc, lens, max_len, ws)
    o = rgc.diff_attn_prefill(q1, q2, k1c, k2c, vc, 0.8, q_start)
"""
import contextlib
import ctypes
import os

import torch

__all__ = [
    "RgcError", "library", "rope_apply", "kv_cache_append", "rope_append", "norm_rope_append",
    "gqa_attn_prefill",
    "gqa_attn_decode", "gqa_attn_decode_workspace_size", "decode_workspace", "diff_attn_prefill",
    "gqa_attn_decode_rope_append", "gqa_attn_decode_rope_append_static", "diff_attn_decode",
    "diff_decode_workspace",
    "gqa_attn_prefill_varlen", "rope_backward", "gqa_attn_backward", "backward_workspace",
    "ROPE_HALF", "ROPE_INTERLEAVED", "timed_library", "kernel_timing", "timing_report",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librgc.so")
TIMED_LIB_PATH = os.path.join(_HERE, "librgc_timed.so")
ROPE_HALF, ROPE_INTERLEAVED = 0, 1
_F32, _BF16 = 0, 1

_p = ctypes.c_void_p
_i = ctypes.c_int
_i64 = ctypes.c_int64
_f = ctypes.c_float
_d = ctypes.c_double
_sz = ctypes.c_size_t

_SIGNATURES = {
    "rgc_abi_version": (_i, []),
    "rgc_status_string": (ctypes.c_char_p, [_i]),
    "rgc_rope_apply": (_i, [_p, _i, _i, _i, _i, _i, _i64, _i64, _i64, _p, _d, _i, _p]),
    "rgc_rope_backward": (_i, [_p, _i, _i, _i, _i, _i, _i64, _i64, _i64, _p, _d, _i, _p]),
    "rgc_gqa_attn_backward_workspace_size": (_sz, [_i, _i, _i]),
    "rgc_gqa_attn_backward": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i,
                                   _i64, _i64, _i64, _i64, _i64, _i64, _f, _p, _sz, _p]),
    "rgc_kv_cache_append": (_i, [_p, _p, _i, _i, _i, _i, _i, _i64, _i64, _i64, _p, _p, _i,
                                 _i64, _i64, _i64, _p, _p, _p]),
    "rgc_rope_append": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i64, _i64, _i64,
                             _i64, _i64, _i64, _i64, _i64, _i64, _p, _d, _i, _p, _p]),
    "rgc_norm_rope_append": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i64, _i64, _i64,
                                  _i64, _i64, _i64, _i64, _i64, _i64, _p, _d, _i, _f, _p, _p]),
    "rgc_gqa_attn_prefill": (_i, [_p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i,
                                  _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                  _p, _f, _p, _p, _p]),
    "rgc_gqa_attn_prefill_varlen": (_i, [_p, _p, _p, _p, _i, _i, _p, _i, _i, _i, _i, _i,
                                         _i64, _i64, _i64, _i64, _i64, _i64, _f, _p, _p, _p]),
    "rgc_diff_attn_prefill": (_i, [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i,
                                   _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                   _p, _f, _f, _p, _p]),
    "rgc_gqa_attn_decode_workspace_size": (_sz, [_i, _i, _i, _i, _i]),
    "rgc_diff_attn_decode_workspace_size": (_sz, [_i, _i, _i, _i, _i]),
    "rgc_diff_attn_decode": (_i, [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i,
                                  _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                  _p, _i, _f, _f, _p, _sz, _p, _p]),
    "rgc_gqa_attn_decode": (_i, [_p, _p, _p, _p, _i, _i, _i, _i, _i, _i,
                                 _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                 _p, _i, _f, _p, _sz, _p, _p, _p]),
    "rgc_gqa_attn_decode_rope_append": (_i, [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i,
                                             _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                             _p, _i, _d, _i, _f, _p, _sz, _p, _p, _p]),
    "rgc_gqa_attn_decode_rope_append_static": (_i, [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i,
                                                    _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                                    _p, _i, _d, _i, _f, _p, _p, _p]),
}

_TIMING_SIGNATURES = {
    "rgc_timing_enable": (_i, [_i]),
    "rgc_timing_report": (ctypes.c_long, [ctypes.c_char_p, _sz]),
}

_lib = None
_timed_lib = None
_active = None  # the library calls go to: the product one, or the timed one inside kernel_timing()


class RgcError(RuntimeError):
    """A negative status from the C ABI (nothing was launched)."""

    def __init__(self, fn, status, text):
        super().__init__(f"{fn}: status {status} ({text})")
        self.status = status


def _load(path, signatures):
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m rope_gqa_causal_amd.build` "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in signatures.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def library():
    """Load ``librgc.so`` (built by ``rope_gqa_causal_amd.build``); raise if absent."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH, _SIGNATURES)
    return _lib


def timed_library():
    """Load the instrumented build ``librgc_timed.so`` (same kernels, plus
    per-kernel timing); raise if absent.  For measurement only."""
    global _timed_lib
    if _timed_lib is None:
        _timed_lib = _load(TIMED_LIB_PATH, {**_SIGNATURES, **_TIMING_SIGNATURES})
    return _timed_lib


def _call(name, *args):
    lib = _active if _active is not None else library()
    st = getattr(lib, name)(*args)
    if st != 0:
        raise RgcError(name, st, lib.rgc_status_string(st).decode())


def _dtype(t):
    if t.dtype == torch.bfloat16:
        return _BF16
    if t.dtype == torch.float32:
        return _F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("rope_gqa_causal_amd works on GPU tensors only")


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _lens(t, B, name):
    if t is None:
        return None
    if t.dtype != torch.int32 or not t.is_contiguous() or t.numel() != B:
        raise ValueError(f"{name} must be a contiguous int32 tensor of {B} elements")
    return t


@contextlib.contextmanager
def kernel_timing():
    """Route the calls made inside the block through the instrumented build
    with per-kernel timing on: each kernel it launches is bracketed by HIP
    events on its own stream.  Read the result with ``timing_report()``."""
    global _active
    lib = timed_library()
    prev = _active
    _active = lib
    lib.rgc_timing_enable(1)
    try:
        yield
    finally:
        lib.rgc_timing_enable(0)
        _active = prev


def timing_report():
    """Per-kernel {name: (launches, total microseconds)} recorded by the
    instrumented build since the last report (waits for the events; clears
    the record)."""
    lib = timed_library()
    buf = ctypes.create_string_buffer(1 << 16)
    n = lib.rgc_timing_report(buf, len(buf))
    if n < 0:
        raise RgcError("rgc_timing_report", n, lib.rgc_status_string(n).decode())
    out = {}
    for line in buf.value.decode().splitlines():
        name, calls, us = line.split()
        out[name] = (int(calls), float(us))
    return out


def rope_apply(x, pos0=None, base=10000.0, style=ROPE_HALF):
    """Rotate x [B,S,H,D] in place; token (b,s) sits at position pos0[b] + s."""
    _gpu(x, pos0)
    B, S, H, D = x.shape
    pos0 = _lens(pos0, B, "pos0")
    _call("rgc_rope_apply", _ptr(x), _dtype(x), B, S, H, D, x.stride(0), x.stride(1),
          x.stride(2), _ptr(pos0), float(base), int(style), _stream(x))
    return x


def rope_backward(g, pos0=None, base=10000.0, style=ROPE_HALF):
    """Gradient through RoPE: turn g [B,S,H,D] back by its angles, in place."""
    _gpu(g, pos0)
    B, S, H, D = g.shape
    pos0 = _lens(pos0, B, "pos0")
    _call("rgc_rope_backward", _ptr(g), _dtype(g), B, S, H, D, g.stride(0), g.stride(1), g.stride(2),
          _ptr(pos0), float(base), int(style), _stream(g))
    return g


def kv_cache_append(k_cache, v_cache, k_new, v_new, pos0, err_flag=None):
    """Copy k_new, v_new [B,S_new,Hkv,D] to slots pos0[b].. of caches [B,Hkv,S_max,D]."""
    _gpu(k_cache, v_cache, k_new, v_new, pos0, err_flag)
    B, Hkv, S_max, D = k_cache.shape
    S_new = k_new.shape[1]
    if v_cache.stride() != k_cache.stride() or v_new.stride() != k_new.stride():
        raise ValueError("k and v tensors must share strides")
    if tuple(k_new.shape) != (B, S_new, Hkv, D) or v_new.shape != k_new.shape:
        raise ValueError("new rows must be [B,S_new,Hkv,D]")
    pos0 = _lens(pos0, B, "pos0")
    _call("rgc_kv_cache_append", _ptr(k_cache), _ptr(v_cache), _dtype(k_cache), B, Hkv, D, S_max,
          k_cache.stride(0), k_cache.stride(1), k_cache.stride(2), _ptr(k_new), _ptr(v_new),
          S_new, k_new.stride(0), k_new.stride(1), k_new.stride(2), _ptr(pos0),
          _ptr(err_flag), _stream(k_cache))


def _rope_append_args(q, k_new, v_new, k_cache, v_cache, pos0, err_flag):
    _gpu(q, k_new, v_new, k_cache, v_cache, pos0, err_flag)
    B, S, Hq, D = q.shape
    _, Hkv, S_max, _ = k_cache.shape
    if v_cache.stride() != k_cache.stride() or v_new.stride() != k_new.stride():
        raise ValueError("k and v tensors must share strides")
    if tuple(k_new.shape) != (B, S, Hkv, D) or v_new.shape != k_new.shape:
        raise ValueError("new rows must be [B,S,Hkv,D]")
    pos0 = _lens(pos0, B, "pos0")
    return (_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _dtype(q),
            B, S, Hq, Hkv, D, S_max, q.stride(0), q.stride(1), q.stride(2),
            k_new.stride(0), k_new.stride(1), k_new.stride(2),
            k_cache.stride(0), k_cache.stride(1), k_cache.stride(2), _ptr(pos0))


def rope_append(q, k_new, v_new, k_cache, v_cache, pos0, base=10000.0, style=ROPE_HALF, err_flag=None):
    """Fused step prologue: rotate q in place and k_new into the caches, copy v_new.

    q [B,S,Hq,D]; k_new, v_new [B,S,Hkv,D]; caches [B,Hkv,S_max,D]; token (b,s)
    has position and cache slot pos0[b] + s."""
    args = _rope_append_args(q, k_new, v_new, k_cache, v_cache, pos0, err_flag)
    _call("rgc_rope_append", *args, float(base), int(style), _ptr(err_flag), _stream(q))
    return q


def norm_rope_append(q, k_new, v_new, k_cache, v_cache, pos0, base=10000.0, style=ROPE_HALF, eps=1e-6,
                     err_flag=None):
    """rope_append with each q and k head vector first divided by sqrt(mean square + eps)."""
    args = _rope_append_args(q, k_new, v_new, k_cache, v_cache, pos0, err_flag)
    _call("rgc_norm_rope_append", *args, float(base), int(style), float(eps), _ptr(err_flag), _stream(q))
    return q


def gqa_attn_prefill(q, k_cache, v_cache, q_start=None, scale=None, out=None, lse=None,
                     err_flag=None):
    """Causal GQA of q [B,Sq,Hq,D] over caches [B,Hkv,S_max,D] (row s at slot q_start[b]+s)."""
    _gpu(q, k_cache, v_cache, q_start, out, lse, err_flag)
    B, Sq, Hq, D = q.shape
    _, Hkv, S_max, _ = k_cache.shape
    if v_cache.stride() != k_cache.stride():
        raise ValueError("k_cache and v_cache must share strides")
    if scale is None:
        scale = D ** -0.5
    o = torch.empty_like(q) if out is None else out
    q_start = _lens(q_start, B, "q_start")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != (B, Hq, Sq)):
        raise ValueError("lse must be a contiguous float32 [B,Hq,Sq] tensor")
    _call("rgc_gqa_attn_prefill", _ptr(o), _ptr(q), _ptr(k_cache), _ptr(v_cache), _dtype(q),
          B, Sq, Hq, Hkv, D, S_max, q.stride(0), q.stride(1), q.stride(2),
          o.stride(0), o.stride(1), o.stride(2),
          k_cache.stride(0), k_cache.stride(1), k_cache.stride(2),
          _ptr(q_start), float(scale), _ptr(lse), _ptr(err_flag), _stream(q))
    return o


def gqa_attn_prefill_varlen(q, k, v, cu_seqlens, max_seqlen, scale=None, out=None, lse=None, err_flag=None):
    """Causal GQA over packed documents: q [T,Hq,D], k, v [T,Hkv,D] (bf16);
    document i is tokens cu_seqlens[i]..cu_seqlens[i+1]-1 and attends only to
    itself.  max_seqlen (host int) bounds every document's length."""
    _gpu(q, k, v, cu_seqlens, out, lse, err_flag)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (T, Hkv, D) or v.shape != k.shape or v.stride() != k.stride():
        raise ValueError("k and v must be [T,Hkv,D] with the same strides")
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_contiguous() or cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be a contiguous int32 vector")
    if scale is None:
        scale = D ** -0.5
    o = torch.empty_like(q) if out is None else out
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (Hq, T)):
        raise ValueError("lse must be a contiguous float32 [Hq,T] tensor")
    _call("rgc_gqa_attn_prefill_varlen", _ptr(o), _ptr(q), _ptr(k), _ptr(v), _dtype(q),
          cu_seqlens.numel() - 1, _ptr(cu_seqlens), int(max_seqlen), T, Hq, Hkv, D,
          q.stride(0), q.stride(1), o.stride(0), o.stride(1), k.stride(0), k.stride(1),
          float(scale), _ptr(lse), _ptr(err_flag), _stream(q))
    return o


def backward_workspace(B, S, Hq, device="cuda"):
    n = max(int(library().rgc_gqa_attn_backward_workspace_size(B, S, Hq)), 256)
    return torch.empty(n, dtype=torch.uint8, device=device)


def gqa_attn_backward(q, k, v, o, d_o, lse, scale=None, workspace=None, dq=None, dk=None, dv=None):
    """Gradients of causal GQA self-attention (bf16).  q, o, d_o [B,S,Hq,D]
    (same strides); k, v [B,S,Hkv,D] (same strides); lse [B,Hq,S] fp32 from
    gqa_attn_prefill.  Returns (dq, dk, dv)."""
    _gpu(q, k, v, o, d_o, lse, workspace, dq, dk, dv)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if o.stride() != q.stride() or d_o.stride() != q.stride() or v.stride() != k.stride():
        raise ValueError("q, o, d_o must share strides, and k, v")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (B, Hq, S):
        raise ValueError("lse must be a contiguous float32 [B,Hq,S] tensor")
    if scale is None:
        scale = D ** -0.5
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if dq.stride() != q.stride() or dk.stride() != k.stride() or dv.stride() != k.stride():
        raise ValueError("gradients must have the strides of their inputs")
    if workspace is None:
        workspace = backward_workspace(B, S, Hq, q.device)
    _call("rgc_gqa_attn_backward", _ptr(dq), _ptr(dk), _ptr(dv), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
          _ptr(d_o), _ptr(lse), _dtype(q), B, S, Hq, Hkv, D, q.stride(0), q.stride(1), q.stride(2),
          k.stride(0), k.stride(1), k.stride(2), float(scale), _ptr(workspace),
          workspace.numel() * workspace.element_size(), _stream(q))
    return dq, dk, dv


def diff_attn_prefill(q1, q2, k1_cache, k2_cache, v_cache, lam, q_start=None, scale=None, out=None,
                      err_flag=None):
    """Causal differential GQA: (softmax(q1 K1^T) - lam softmax(q2 K2^T)) V.

    q1, q2 [B,Sq,Hq,D] (same strides); caches [B,Hkv,S_max,D] (same strides);
    bf16, D in {32, 64, 128}."""
    _gpu(q1, q2, k1_cache, k2_cache, v_cache, q_start, out, err_flag)
    B, Sq, Hq, D = q1.shape
    _, Hkv, S_max, _ = k1_cache.shape
    if q2.shape != q1.shape or q2.stride() != q1.stride():
        raise ValueError("q1 and q2 must share shape and strides")
    if (k2_cache.shape != k1_cache.shape or v_cache.shape != k1_cache.shape
            or k2_cache.stride() != k1_cache.stride() or v_cache.stride() != k1_cache.stride()):
        raise ValueError("k1, k2 and v caches must share shape and strides")
    if scale is None:
        scale = D ** -0.5
    o = torch.empty_like(q1) if out is None else out
    q_start = _lens(q_start, B, "q_start")
    _call("rgc_diff_attn_prefill", _ptr(o), _ptr(q1), _ptr(q2), _ptr(k1_cache), _ptr(k2_cache),
          _ptr(v_cache), _dtype(q1), B, Sq, Hq, Hkv, D, S_max, q1.stride(0), q1.stride(1), q1.stride(2),
          o.stride(0), o.stride(1), o.stride(2),
          k1_cache.stride(0), k1_cache.stride(1), k1_cache.stride(2),
          _ptr(q_start), float(lam), float(scale), _ptr(err_flag), _stream(q1))
    return o


def diff_decode_workspace(B, Hq, Hkv, D, max_len, device="cuda"):
    """A workspace tensor large enough for diff_attn_decode."""
    n = max(int(library().rgc_diff_attn_decode_workspace_size(B, Hq, Hkv, D, max_len)), 256)
    return torch.empty(n, dtype=torch.uint8, device=device)


def diff_attn_decode(q1, q2, k1_cache, k2_cache, v_cache, seq_lens, lam, max_len=None, workspace=None,
                     scale=None, out=None, err_flag=None):
    """Cached differential decode: q1, q2 [B,Hq,D] (same strides) over caches
    [B,Hkv,S_max,D] (same strides) of lengths seq_lens[b]; bf16."""
    _gpu(q1, q2, k1_cache, k2_cache, v_cache, seq_lens, workspace, out, err_flag)
    B, Hq, D = q1.shape
    _, Hkv, S_max, _ = k1_cache.shape
    if q2.shape != q1.shape or q2.stride() != q1.stride():
        raise ValueError("q1 and q2 must share shape and strides")
    if (k2_cache.shape != k1_cache.shape or v_cache.shape != k1_cache.shape
            or k2_cache.stride() != k1_cache.stride() or v_cache.stride() != k1_cache.stride()):
        raise ValueError("k1, k2 and v caches must share shape and strides")
    if scale is None:
        scale = D ** -0.5
    if max_len is None:
        max_len = S_max
    if workspace is None:
        workspace = diff_decode_workspace(B, Hq, Hkv, D, max_len, q1.device)
    o = torch.empty_like(q1) if out is None else out
    seq_lens = _lens(seq_lens, B, "seq_lens")
    _call("rgc_diff_attn_decode", _ptr(o), _ptr(q1), _ptr(q2), _ptr(k1_cache), _ptr(k2_cache), _ptr(v_cache),
          _dtype(q1), B, Hq, Hkv, D, S_max, q1.stride(0), q1.stride(1), o.stride(0), o.stride(1),
          k1_cache.stride(0), k1_cache.stride(1), k1_cache.stride(2), _ptr(seq_lens), int(max_len), float(lam),
          float(scale), _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(err_flag), _stream(q1))
    return o


def gqa_attn_decode_workspace_size(B, Hq, Hkv, D, max_len):
    return int(library().rgc_gqa_attn_decode_workspace_size(B, Hq, Hkv, D, max_len))


def decode_workspace(B, Hq, Hkv, D, max_len, device="cuda"):
    """A zero-filled workspace tensor large enough for gqa_attn_decode."""
    n = max(gqa_attn_decode_workspace_size(B, Hq, Hkv, D, max_len), 256)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def _decode_rope_append_args(q, k_new, v_new, k_cache, v_cache, seq_lens, max_len, out, lse, err_flag):
    _gpu(q, k_new, v_new, k_cache, v_cache, seq_lens, out, lse, err_flag)
    B, Hq, D = q.shape
    _, Hkv, S_max, _ = k_cache.shape
    if v_cache.stride() != k_cache.stride():
        raise ValueError("k_cache and v_cache must share strides")
    if tuple(k_new.shape) != (B, Hkv, D) or tuple(v_new.shape) != (B, Hkv, D) or k_new.stride() != v_new.stride():
        raise ValueError("k_new and v_new must be [B,Hkv,D] with one set of strides")
    if k_new.stride(2) != 1 or q.stride(2) != 1:
        raise ValueError("q, k_new and v_new need unit stride along D")
    if max_len is None:
        max_len = S_max
    o = torch.empty_like(q) if out is None else out
    seq_lens = _lens(seq_lens, B, "seq_lens")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != (B, Hq)):
        raise ValueError("lse must be a contiguous float32 [B,Hq] tensor")
    args = (_ptr(o), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _dtype(q), B, Hq, Hkv, D,
            S_max, q.stride(0), q.stride(1), k_new.stride(0), k_new.stride(1), o.stride(0), o.stride(1),
            k_cache.stride(0), k_cache.stride(1), k_cache.stride(2), _ptr(seq_lens), int(max_len))
    return o, args, max_len


def gqa_attn_decode_rope_append(q, k_new, v_new, k_cache, v_cache, seq_lens, max_len=None, workspace=None,
                                base=10000.0, style=ROPE_HALF, scale=None, out=None, lse=None, err_flag=None):
    """One generation step in one decode launch: q [B,Hq,D] and k_new [B,Hkv,D] turned at
    position seq_lens[b]-1, k_new (rotated) and v_new [B,Hkv,D] written to that cache slot,
    and the attention of q over slots 0..seq_lens[b]-1.  q is left unrotated; bf16 only."""
    _gpu(workspace)
    o, args, max_len = _decode_rope_append_args(q, k_new, v_new, k_cache, v_cache, seq_lens, max_len, out, lse,
                                                err_flag)
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    if scale is None:
        scale = D ** -0.5
    if workspace is None:
        workspace = decode_workspace(B, Hq, Hkv, D, max_len, q.device)
    _call("rgc_gqa_attn_decode_rope_append", *args, float(base), int(style), float(scale), _ptr(workspace),
          workspace.numel() * workspace.element_size(), _ptr(lse), _ptr(err_flag), _stream(q))
    return o


def gqa_attn_decode_rope_append_static(q, k_new, v_new, k_cache, v_cache, seq_lens, max_len=None,
                                       base=10000.0, style=ROPE_HALF, scale=None, out=None, lse=None,
                                       err_flag=None):
    """gqa_attn_decode_rope_append with the partials in the library's own
    per-GPU array (16 MiB) instead of a workspace: the library allocates
    nothing.  Calls that overlap in time on one GPU race."""
    o, args, _ = _decode_rope_append_args(q, k_new, v_new, k_cache, v_cache, seq_lens, max_len, out, lse,
                                          err_flag)
    if scale is None:
        scale = q.shape[2] ** -0.5
    _call("rgc_gqa_attn_decode_rope_append_static", *args, float(base), int(style), float(scale), _ptr(lse),
          _ptr(err_flag), _stream(q))
    return o


def gqa_attn_decode(q, k_cache, v_cache, seq_lens, max_len=None, workspace=None, scale=None,
                    out=None, lse=None, err_flag=None):
    """One query row per sequence (q [B,Hq,D]) at slot seq_lens[b]-1 over its cache."""
    _gpu(q, k_cache, v_cache, seq_lens, workspace, out, lse, err_flag)
    B, Hq, D = q.shape
    _, Hkv, S_max, _ = k_cache.shape
    if v_cache.stride() != k_cache.stride():
        raise ValueError("k_cache and v_cache must share strides")
    if scale is None:
        scale = D ** -0.5
    if max_len is None:
        max_len = S_max
    if workspace is None:
        workspace = decode_workspace(B, Hq, Hkv, D, max_len, q.device)
    o = torch.empty_like(q) if out is None else out
    seq_lens = _lens(seq_lens, B, "seq_lens")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != (B, Hq)):
        raise ValueError("lse must be a contiguous float32 [B,Hq] tensor")
    _call("rgc_gqa_attn_decode", _ptr(o), _ptr(q), _ptr(k_cache), _ptr(v_cache), _dtype(q),
          B, Hq, Hkv, D, S_max, q.stride(0), q.stride(1), o.stride(0), o.stride(1),
          k_cache.stride(0), k_cache.stride(1), k_cache.stride(2), _ptr(seq_lens), int(max_len),
          float(scale), _ptr(workspace), workspace.numel() * workspace.element_size(),
          _ptr(lse), _ptr(err_flag), _stream(q))
    return o
