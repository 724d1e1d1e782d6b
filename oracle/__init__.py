"""ctypes front end of the fp64 CPU oracle (test infrastructure).

Only the test-suite, ``__graft_entry__.smoke()`` and the benchmark's CPU
baseline use this package.  It marshals CPU torch tensors into the C oracle
(``oracle/orc.c``) and returns float64 tensors; all arithmetic happens in C.
It imports nothing from the HIP library and the HIP library imports nothing
from it.
"""
import ctypes
import os

import torch

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

F32, BF16 = 0, 1
ROPE_HALF, ROPE_INTERLEAVED = 0, 1
_c_i64 = ctypes.c_int64
_c_int = ctypes.c_int
_c_p = ctypes.c_void_p
_c_d = ctypes.c_double


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        lib.orc_bf16_bits.restype = ctypes.c_uint16
        lib.orc_bf16_bits.argtypes = [_c_d]
        lib.orc_rope_f64.argtypes = [_c_p, _c_p, _c_int, _c_int, _c_int, _c_int, _c_int,
                                     _c_i64, _c_i64, _c_i64, _c_p, _c_d, _c_int]
        lib.orc_norm_rope_f64.argtypes = [_c_p, _c_p, _c_int, _c_int, _c_int, _c_int, _c_int,
                                          _c_i64, _c_i64, _c_i64, _c_p, _c_d, _c_int, _c_d]
        lib.orc_rope_grad_f64.argtypes = [_c_p, _c_p, _c_int, _c_int, _c_int, _c_int, _c_int,
                                          _c_i64, _c_i64, _c_i64, _c_p, _c_d, _c_int]
        lib.orc_attn_backward.argtypes = [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_int, _c_int,
                                          _c_int, _c_int, _c_int, _c_int, _c_i64, _c_i64, _c_i64,
                                          _c_i64, _c_i64, _c_i64, _c_d, _c_int]
        lib.orc_rope_apply.argtypes = [_c_p, _c_int, _c_int, _c_int, _c_int, _c_int,
                                       _c_i64, _c_i64, _c_i64, _c_p, _c_d, _c_int]
        lib.orc_kv_cache_append.argtypes = [_c_p, _c_p, _c_int, _c_int, _c_int, _c_int, _c_int,
                                            _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_int,
                                            _c_i64, _c_i64, _c_i64, _c_p]
        lib.orc_attn.argtypes = [_c_p, _c_p, _c_p, _c_p, _c_p, _c_int, _c_int, _c_int, _c_int,
                                 _c_int, _c_int, _c_int, _c_i64, _c_i64, _c_i64,
                                 _c_i64, _c_i64, _c_i64, _c_p, _c_d, _c_int]
        lib.orc_attn_decode.argtypes = [_c_p, _c_p, _c_p, _c_p, _c_p, _c_int, _c_int, _c_int,
                                        _c_int, _c_int, _c_int, _c_i64, _c_i64,
                                        _c_i64, _c_i64, _c_i64, _c_p, _c_d, _c_int]
        lib.orc_diff_attn.argtypes = [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_int, _c_int, _c_int,
                                      _c_int, _c_int, _c_int, _c_int, _c_int,
                                      _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                      _c_i64, _c_i64, _c_i64, _c_p, _c_d, _c_d, _c_int]
        _lib = lib
    return _lib


class OracleError(RuntimeError):
    pass


def _check(status):
    if status != 0:
        raise OracleError(f"oracle status {status}")


def _dt(t):
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"oracle takes float32 or bfloat16, got {t.dtype}")


def _cpu(t):
    if t.device.type != "cpu":
        raise ValueError("oracle inputs must be CPU tensors")
    if t.stride(-1) != 1:
        raise ValueError("last dimension must be contiguous")
    return t


def _i32(t, n):
    if t is None:
        return None, None
    t = torch.as_tensor(t, dtype=torch.int32).contiguous()
    assert t.numel() == n
    return t, t.data_ptr()


def _threads(nthreads):
    return int(nthreads) if nthreads else (os.cpu_count() or 1)


def bf16_bits(x: float) -> int:
    """Nearest bfloat16 (ties to even) of a double, as 16 raw bits."""
    return int(_load().orc_bf16_bits(float(x)))


def round_to_bf16(t: torch.Tensor) -> torch.Tensor:
    """Element-wise single rounding of a float64 tensor to bfloat16."""
    flat = t.detach().to(torch.float64).reshape(-1).tolist()
    bits = torch.tensor([bf16_bits(v) for v in flat], dtype=torch.int32)
    return bits.to(torch.int16).view(torch.bfloat16).reshape(t.shape)


def rope_f64(x, pos0=None, base=10000.0, style=ROPE_HALF):
    """Exact (double) RoPE of x [B,S,H,D]; returns a float64 tensor."""
    x = _cpu(x)
    B, S, H, D = x.shape
    out = torch.empty((B, S, H, D), dtype=torch.float64)
    p, pp = _i32(pos0, B)
    _check(_load().orc_rope_f64(out.data_ptr(), x.data_ptr(), _dt(x), B, S, H, D,
                                x.stride(0), x.stride(1), x.stride(2), pp, base, style))
    return out


def norm_rope_f64(x, pos0=None, base=10000.0, style=ROPE_HALF, eps=1e-6):
    """Exact (double) QK normalisation then RoPE of x [B,S,H,D]: each head
    vector divided by sqrt(mean of squares + eps), then rotated."""
    x = _cpu(x)
    B, S, H, D = x.shape
    out = torch.empty((B, S, H, D), dtype=torch.float64)
    p, pp = _i32(pos0, B)
    _check(_load().orc_norm_rope_f64(out.data_ptr(), x.data_ptr(), _dt(x), B, S, H, D,
                                     x.stride(0), x.stride(1), x.stride(2), pp, base, style, eps))
    return out


def rope_apply_(x, pos0=None, base=10000.0, style=ROPE_HALF):
    """In-place RoPE of x [B,S,H,D], rounded once to x's dtype."""
    x = _cpu(x)
    B, S, H, D = x.shape
    p, pp = _i32(pos0, B)
    _check(_load().orc_rope_apply(x.data_ptr(), _dt(x), B, S, H, D,
                                  x.stride(0), x.stride(1), x.stride(2), pp, base, style))
    return x


def kv_cache_append_(k_cache, v_cache, k_new, v_new, pos0):
    """Copy k_new/v_new [B,S,Hkv,D] into caches [B,Hkv,S_max,D] at pos0[b]+s."""
    k_cache, v_cache, k_new, v_new = map(_cpu, (k_cache, v_cache, k_new, v_new))
    B, Hkv, S_max, D = k_cache.shape
    S_new = k_new.shape[1]
    assert tuple(v_cache.stride()) == tuple(k_cache.stride())
    assert tuple(v_new.stride()) == tuple(k_new.stride())
    p, pp = _i32(pos0, B)
    return _load().orc_kv_cache_append(
        k_cache.data_ptr(), v_cache.data_ptr(), _dt(k_cache), B, Hkv, D, S_max,
        k_cache.stride(0), k_cache.stride(1), k_cache.stride(2),
        k_new.data_ptr(), v_new.data_ptr(), S_new,
        k_new.stride(0), k_new.stride(1), k_new.stride(2), pp)


def attn(q, k_cache, v_cache, q_start=None, scale=None, want_lse=False, nthreads=None):
    """Causal GQA attention of q [B,Sq,Hq,D] over caches [B,Hkv,S_max,D].

    Returns float64 o [B,Sq,Hq,D] (and lse [B,Hq,Sq] when asked)."""
    q, k_cache, v_cache = map(_cpu, (q, k_cache, v_cache))
    B, Sq, Hq, D = q.shape
    _, Hkv, S_max, _ = k_cache.shape
    assert tuple(v_cache.stride()) == tuple(k_cache.stride())
    if scale is None:
        scale = D ** -0.5
    o = torch.empty((B, Sq, Hq, D), dtype=torch.float64)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float64) if want_lse else None
    p, pp = _i32(q_start, B)
    _check(_load().orc_attn(o.data_ptr(), lse.data_ptr() if lse is not None else None,
                            q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), _dt(q),
                            B, Sq, Hq, Hkv, D, S_max,
                            q.stride(0), q.stride(1), q.stride(2),
                            k_cache.stride(0), k_cache.stride(1), k_cache.stride(2),
                            pp, float(scale), _threads(nthreads)))
    return (o, lse) if want_lse else o


def attn_varlen(q, k, v, cu_seqlens, scale=None, want_lse=False, nthreads=None):
    """Causal GQA over packed documents (document masking, page "训练3.8B LLM至
    0.384 CORE，成本998美元 – Hugo Vergnes", section 无效的方法): q [T,Hq,D],
    k, v [T,Hkv,D]; document i is tokens cu_seqlens[i]..cu_seqlens[i+1]-1 and
    each of its tokens attends to its own document's tokens at or before it.
    Each document is one orc_attn call on its slice.  Returns float64 o
    [T,Hq,D] (and lse [Hq,T])."""
    q, k, v = map(_cpu, (q, k, v))
    T, Hq, D = q.shape
    cu = [int(c) for c in _cpu(cu_seqlens).tolist()]
    o = torch.empty((T, Hq, D), dtype=torch.float64)
    lse = torch.empty((Hq, T), dtype=torch.float64) if want_lse else None
    for c0, c1 in zip(cu[:-1], cu[1:]):
        if c1 == c0:
            continue
        # document slice as a batch of one: q [1,n,Hq,D], k/v as a [1,Hkv,n,D] cache view
        r = attn(q[c0:c1][None], k[c0:c1].transpose(0, 1)[None], v[c0:c1].transpose(0, 1)[None],
                 None, scale, want_lse, nthreads)
        if want_lse:
            o[c0:c1] = r[0][0]
            lse[:, c0:c1] = r[1][0]
        else:
            o[c0:c1] = r[0]
    return (o, lse) if want_lse else o


def attn_backward(q, k, v, dO, scale=None, nthreads=None):
    """Gradients of causal GQA self-attention: q, dO [B,S,Hq,D] (same
    strides), k, v [B,S,Hkv,D] (same strides).  Returns float64 dq, dk, dv."""
    q, k, v, dO = map(_cpu, (q, k, v, dO))
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    assert tuple(dO.stride()) == tuple(q.stride()) and tuple(v.stride()) == tuple(k.stride())
    if scale is None:
        scale = D ** -0.5
    dq = torch.empty((B, S, Hq, D), dtype=torch.float64)
    dk = torch.empty((B, S, Hkv, D), dtype=torch.float64)
    dv = torch.empty((B, S, Hkv, D), dtype=torch.float64)
    _check(_load().orc_attn_backward(dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), q.data_ptr(), k.data_ptr(),
                                     v.data_ptr(), dO.data_ptr(), _dt(q), B, S, Hq, Hkv, D,
                                     q.stride(0), q.stride(1), q.stride(2), k.stride(0), k.stride(1),
                                     k.stride(2), float(scale), _threads(nthreads)))
    return dq, dk, dv


def rope_grad_f64(g, pos0=None, base=10000.0, style=ROPE_HALF):
    """Gradient through RoPE (g [B,S,H,D] turned back by its angle); float64."""
    g = _cpu(g)
    B, S, H, D = g.shape
    out = torch.empty((B, S, H, D), dtype=torch.float64)
    p, pp = _i32(pos0, B)
    _check(_load().orc_rope_grad_f64(out.data_ptr(), g.data_ptr(), _dt(g), B, S, H, D,
                                     g.stride(0), g.stride(1), g.stride(2), pp, base, style))
    return out


def attn_decode(q, k_cache, v_cache, seq_lens, scale=None, want_lse=False, nthreads=None):
    """Cached decode of q [B,Hq,D] at slot seq_lens[b]-1; float64 o [B,Hq,D]."""
    q, k_cache, v_cache = map(_cpu, (q, k_cache, v_cache))
    B, Hq, D = q.shape
    _, Hkv, S_max, _ = k_cache.shape
    if scale is None:
        scale = D ** -0.5
    o = torch.empty((B, Hq, D), dtype=torch.float64)
    lse = torch.empty((B, Hq), dtype=torch.float64) if want_lse else None
    L, pl = _i32(seq_lens, B)
    _check(_load().orc_attn_decode(o.data_ptr(), lse.data_ptr() if lse is not None else None,
                                   q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), _dt(q),
                                   B, Hq, Hkv, D, S_max, q.stride(0), q.stride(1),
                                   k_cache.stride(0), k_cache.stride(1), k_cache.stride(2),
                                   pl, float(scale), _threads(nthreads)))
    return (o, lse) if want_lse else o


def diff_attn(q1, q2, k1, k2, v, lam, q_start=None, scale=None, nthreads=None):
    """Differential causal GQA attention; float64 o [B,S,Hq,Dv]."""
    q1, q2, k1, k2, v = map(_cpu, (q1, q2, k1, k2, v))
    B, S, Hq, D = q1.shape
    _, Hkv, S_max, _ = k1.shape
    Dv = v.shape[3]
    assert tuple(q1.stride()) == tuple(q2.stride())
    assert tuple(k1.stride()) == tuple(k2.stride())
    if scale is None:
        scale = D ** -0.5
    o = torch.empty((B, S, Hq, Dv), dtype=torch.float64)
    p, pp = _i32(q_start, B)
    _check(_load().orc_diff_attn(o.data_ptr(), q1.data_ptr(), q2.data_ptr(), k1.data_ptr(),
                                 k2.data_ptr(), v.data_ptr(), _dt(q1), B, S, Hq, Hkv, D, Dv,
                                 S_max, q1.stride(0), q1.stride(1), q1.stride(2),
                                 k1.stride(0), k1.stride(1), k1.stride(2),
                                 v.stride(0), v.stride(1), v.stride(2),
                                 pp, float(lam), float(scale), _threads(nthreads)))
    return o
