"""The oracle: TEST INFRASTRUCTURE ONLY.

A plain double-precision CPU definition of one pre-LayerNorm GPT layer with a KV cache and of the
group-wise int8 weight quantizer, written in C (oracle.c) and called here through ctypes. Only the
tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import this package;
the GPU library shares no code with it and never calls it.

Sources and readings are listed in oracle.h. Inputs are the exact values the GPU receives
(float32, float16 or int8 arrays) widened to float64 by the caller.
"""
import ctypes as C
import os
from dataclasses import dataclass

import numpy as np

from . import build as _build

_LIB = None
_D = C.POINTER(C.c_double)


def lib():
    """Load oracle/liboracle.so, compiling it first if it is not there."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = C.CDLL(_build.LIB)
        L.ora_layernorm.argtypes = [_D, C.c_int, _D, _D, C.c_double, _D]
        L.ora_linear.argtypes = [_D, _D, _D, C.c_int, C.c_int, _D]
        L.ora_gelu.argtypes = [C.c_double, C.c_int]
        L.ora_gelu.restype = C.c_double
        L.ora_softmax.argtypes = [_D, C.c_int, _D]
        L.ora_attend.argtypes = [_D, _D, _D, C.c_int, C.c_int, _D]
        L.ora_layer_forward.argtypes = [C.c_void_p, C.c_void_p, _D, _D, C.c_int,
                                        C.POINTER(C.c_int), _D, _D, C.c_int, C.c_int, C.c_void_p]
        L.ora_lm_head.argtypes = [_D, C.c_int, _D, _D, C.c_double, _D, C.c_int, _D]
        L.ora_argmax.argtypes = [_D, C.c_int]
        L.ora_argmax.restype = C.c_int
        L.ora_fp16_from_double.argtypes = [C.c_double]
        L.ora_fp16_from_double.restype = C.c_uint16
        L.ora_fp16_to_double.argtypes = [C.c_uint16]
        L.ora_fp16_to_double.restype = C.c_double
        L.ora_quantize_i8.argtypes = [C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_void_p]
        L.ora_dequantize_i8.argtypes = [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int, _D]
        L.ora_moe_forward.argtypes = [C.c_void_p, C.c_void_p, _D, C.c_int, C.c_void_p, _D, C.c_void_p, _D]
        L.ora_moe_forward.restype = C.c_int
        L.ora_quantize_row_i8.argtypes = [_D, C.c_int, C.c_void_p, C.c_void_p]
        _LIB = L
    return _LIB


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a):
    return a.ctypes.data_as(_D)


# ---------------------------------------------------------------- single steps
def layernorm(x, g, b, eps=1e-5):
    x, g, b = _f64(x), _f64(g), _f64(b)
    out = np.empty_like(x)
    n = x.shape[-1]
    for r in range(x.size // n):
        xr, orow = x.reshape(-1, n)[r], out.reshape(-1, n)[r]
        lib().ora_layernorm(_p(xr), n, _p(g), _p(b), eps, _p(orow))
    return out


def linear(w, bias, x):
    w, x = _f64(w), _f64(x)
    n_out, k = w.shape
    out = np.empty(n_out)
    b = _f64(bias) if bias is not None else None
    lib().ora_linear(_p(w), _p(b) if b is not None else None, _p(x), n_out, k, _p(out))
    return out


def gelu(u, tanh_form=False):
    u = _f64(u)
    f = lib().ora_gelu
    return np.array([f(float(v), int(tanh_form)) for v in u.ravel()]).reshape(u.shape)


def softmax(s):
    s = _f64(s)
    p = np.empty_like(s)
    lib().ora_softmax(_p(s), s.size, _p(p))
    return p


def attend(q, keys, vals):
    q, keys, vals = _f64(q), _f64(keys), _f64(vals)
    n, d = keys.shape
    out = np.empty(d)
    lib().ora_attend(_p(q), _p(keys), _p(vals), n, d, _p(out))
    return out


# ---------------------------------------------------------------- the ends of a generation step
def lm_head(y, g, b, w_vocab, eps=1e-5):
    """logits [V] = W_vocab LN(y; g, b) for one row y [H]."""
    y, g, b, w = _f64(y), _f64(g), _f64(b), _f64(w_vocab)
    V, H = w.shape
    out = np.empty(V)
    lib().ora_lm_head(_p(y), H, _p(g), _p(b), eps, _p(w), V, _p(out))
    return out


def argmax(v):
    """Greedy choice over a 1-D array: first index of the largest value."""
    v = _f64(v)
    if v.ndim != 1 or v.size < 1:
        raise ValueError("argmax needs a non-empty 1-D array")
    return int(lib().ora_argmax(_p(v), v.size))


def quantize_rows_i8(x):
    """The int8 KV-cache reading: each row of x [..., n] (float64) as int8 codes [..., n] and one fp16
    scale (uint16 bits) [...] per row, scale = fp16(amax/127), code = clamp(RNE(x/scale), -127, 127)."""
    x = _f64(x)
    n = x.shape[-1]
    rows = x.reshape(-1, n)
    q = np.empty(rows.shape, dtype=np.int8)
    s = np.empty(rows.shape[0], dtype=np.uint16)
    for i in range(rows.shape[0]):
        r = np.ascontiguousarray(rows[i])
        lib().ora_quantize_row_i8(_p(r), n, q[i:].ctypes.data, s[i:].ctypes.data)
    return q.reshape(x.shape), s.reshape(x.shape[:-1])


# ---------------------------------------------------------------- the MoE expert FF
class _MoeDesc(C.Structure):
    _fields_ = [("hidden", C.c_int), ("ffn", C.c_int), ("experts", C.c_int), ("top_k", C.c_int),
                ("ln_eps", C.c_double), ("gelu_tanh", C.c_int), ("residual", C.c_int), ("combine", C.c_int)]


class _MoeWeights(C.Structure):
    _fields_ = [(n, _D) for n in ("ln_g", "ln_b", "w_gate", "w1", "b1", "w2", "b2", "r_w1", "r_b1", "r_w2", "r_b2")]


def moe_forward(w, x2, top_k=1, eps=1e-5, gelu_tanh=False, combine=0, force_sel=None):
    """The MoE expert FF ("DeepSpeed MoE 大规模稀疏模型推理实战指南", the MoE sections; the gate and
    combine readings are in oracle.h). w: dict with ln_g, ln_b [H], w_gate [E,H], w1 [E,F,H],
    b1 [E,F], w2 [E,H,F], b2 [E,H], and r_w1, r_b1, r_w2, r_b2 for the 'residual' type (else
    absent). x2: [T,H]. force_sel: [T,top_k] experts to use instead of the top-k. Returns
    (y [T,H], sel [T,top_k] int32, wgt [T,top_k])."""
    arr = {k: _f64(v) for k, v in w.items() if v is not None}
    E, F, H = arr["w1"].shape
    x2 = _f64(x2)
    T = x2.shape[0]
    residual = "r_w1" in arr
    d = _MoeDesc(H, F, E, top_k, eps, int(gelu_tanh), int(residual), int(combine))
    cw = _MoeWeights(*[(_p(arr[n]) if n in arr else None) for n, _ in _MoeWeights._fields_])
    y = np.empty((T, H))
    sel = np.empty((T, top_k), dtype=np.int32)
    wgt = np.empty((T, top_k))
    fs = None
    if force_sel is not None:
        fs = np.ascontiguousarray(force_sel, dtype=np.int32)
        if fs.shape != (T, top_k):
            raise ValueError("force_sel must be [tokens, top_k]")
    rc = lib().ora_moe_forward(C.byref(d), C.byref(cw), _p(x2), T, fs.ctypes.data if fs is not None else None,
                               _p(y), sel.ctypes.data, _p(wgt))
    if rc != 0:
        raise ValueError("moe_forward: inconsistent shapes or a forced expert out of range")
    return y, sel, wgt


# ---------------------------------------------------------------- fp16 and int8
def fp16_from_double(a):
    a = _f64(a)
    f = lib().ora_fp16_from_double
    return np.array([f(float(v)) for v in a.ravel()], dtype=np.uint16).reshape(a.shape)


def fp16_to_double(h):
    h = np.ascontiguousarray(h, dtype=np.uint16)
    f = lib().ora_fp16_to_double
    return np.array([f(int(v)) for v in h.ravel()], dtype=np.float64).reshape(h.shape)


def quantize_i8(w, group=64):
    """w: float32 [N,K] -> (q int8 [N,K], s uint16 fp16-bits [N,K/group])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    q = np.empty((n, k), dtype=np.int8)
    s = np.empty((n, k // group), dtype=np.uint16)
    rc = lib().ora_quantize_i8(w.ctypes.data, n, k, group, q.ctypes.data, s.ctypes.data)
    if rc != 0:
        raise ValueError("quantize_i8: K must be a multiple of the group size")
    return q, s


def dequantize_i8(q, s, group=64):
    q = np.ascontiguousarray(q, dtype=np.int8)
    s = np.ascontiguousarray(s, dtype=np.uint16)
    n, k = q.shape
    w = np.empty((n, k))
    rc = lib().ora_dequantize_i8(q.ctypes.data, s.ctypes.data, n, k, group, _p(w))
    if rc != 0:
        raise ValueError("dequantize_i8: K must be a multiple of the group size")
    return w


# ---------------------------------------------------------------- the layer
class _Desc(C.Structure):
    _fields_ = [("hidden", C.c_int), ("heads", C.c_int), ("head_dim", C.c_int), ("ffn", C.c_int),
                ("ln_eps", C.c_double), ("gelu_tanh", C.c_int), ("triangular_masking", C.c_int),
                ("kv_int8", C.c_int)]


_WNAMES = ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_o", "b_o",
           "ln2_g", "ln2_b", "w_ff1", "b_ff1", "w_ff2", "b_ff2")


class _Weights(C.Structure):
    _fields_ = [(n, _D) for n in _WNAMES]


_SNAMES = ("ln1", "qkv", "ctx", "x2", "ln2", "ff1", "act")


class _Stages(C.Structure):
    _fields_ = [(n, _D) for n in _SNAMES]


@dataclass
class Desc:
    hidden: int
    heads: int
    head_dim: int
    ffn: int
    ln_eps: float = 1e-5
    gelu_tanh: bool = False
    triangular_masking: bool = True
    kv_int8: bool = False  # the int8 KV cache reading (ora_quantize_row_i8 per appended head row)


def layer_forward(desc: Desc, weights: dict, k_cache, v_cache, lens, x, stages=False):
    """One layer on T new rows of B sequences.

    weights: the twelve arrays named in _WNAMES (any float dtype; widened to float64 here).
    k_cache, v_cache: float64 [B, heads, cap, head_dim], updated in place.
    lens: int32 [B], advanced by T in place. x: [B, T, H]. Returns y [B, T, H] (and the stage
    outputs as a dict when stages=True).
    """
    B, T, H = x.shape
    assert k_cache.dtype == np.float64 and v_cache.dtype == np.float64
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    assert lens.dtype == np.int32 and lens.flags.c_contiguous
    cap = k_cache.shape[2]
    ws = {n: _f64(weights[n]) for n in _WNAMES}
    cw = _Weights(*[_p(ws[n]) for n in _WNAMES])
    cd = _Desc(desc.hidden, desc.heads, desc.head_dim, desc.ffn, desc.ln_eps,
               int(desc.gelu_tanh), int(desc.triangular_masking), int(desc.kv_int8))
    xx = _f64(x)
    y = np.empty((B, T, H))
    st_arrays = None
    st_ptr = None
    if stages:
        F = desc.ffn
        widths = {"ln1": H, "qkv": 3 * H, "ctx": H, "x2": H, "ln2": H, "ff1": F, "act": F}
        st_arrays = {n: np.empty((B, T, widths[n])) for n in _SNAMES}
        st_ptr = C.byref(_Stages(*[_p(st_arrays[n]) for n in _SNAMES]))
    rc = lib().ora_layer_forward(C.byref(cd), C.byref(cw), _p(k_cache), _p(v_cache), cap,
                                 lens.ctypes.data_as(C.POINTER(C.c_int)), _p(xx), _p(y), B, T, st_ptr)
    if rc != 0:
        raise ValueError("oracle layer_forward: inconsistent shapes or KV cache overflow")
    return (y, st_arrays) if stages else y
