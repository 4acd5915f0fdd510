"""ctypes binding of libdslayer.so (include/ds_layer.h).

Argument marshalling only: torch tensors give device pointers and streams, every step of the layer
runs in the library's HIP kernels. There is no fallback: if the library is missing, loading fails
with an error that says so.
"""
import ctypes as C
import os

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdslayer.so")

DS_F32, DS_F16, DS_I8, DS_BF16 = 0, 1, 2, 3
DS_OK, DS_ERR_NULL, DS_ERR_SHAPE, DS_ERR_DTYPE, DS_ERR_ALIGN = 0, -1, -2, -3, -4
DS_ERR_KV_FULL, DS_ERR_UNSUPPORTED, DS_ERR_HIP, DS_ERR_WORKSPACE = -5, -6, -7, -8
PARTS = ("ln1", "qkv", "attn", "o", "ln2", "ff1", "ff2", "len")  # ds_part names, in enum order

# every symbol the header declares
EXPORTS = ("ds_layer_create", "ds_layer_destroy", "ds_layer_workspace_bytes", "ds_kv_append",
           "ds_layer_forward_decode", "ds_layer_forward_prefill", "ds_quantize_i8",
           "ds_dequantize_i8", "ds_last_error", "ds_stack_create", "ds_stack_destroy",
           "ds_stack_workspace_bytes", "ds_stack_groups", "ds_stack_forward_decode",
           "ds_stack_check", "ds_stack_set_timeout_us", "ds_read_probe", "ds_stack_state_bytes",
           "ds_stack_forward_decode_static", "ds_stack_forward_generate", "ds_layer_time_kernels",
           "ds_moe_create", "ds_moe_destroy", "ds_moe_workspace_bytes", "ds_moe_forward",
           "ds_moe_time_kernels")
MOE_PARTS = ("gate", "route", "ff1", "ff2", "combine")  # ds_moe_time_kernels launch order


class LayerDescC(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("heads", C.c_int32), ("head_dim", C.c_int32),
                ("ffn", C.c_int32), ("weight_dtype", C.c_int32), ("act_dtype", C.c_int32),
                ("quant_group", C.c_int32), ("quant_group_mlp", C.c_int32), ("ln_eps", C.c_float), ("gelu_tanh", C.c_int32),
                ("triangular_masking", C.c_int32), ("kv_dtype", C.c_int32)]


WEIGHT_FIELDS = ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "s_qkv", "w_o", "b_o", "s_o",
                 "ln2_g", "ln2_b", "w_ff1", "b_ff1", "s_ff1", "w_ff2", "b_ff2", "s_ff2")


class LayerWeightsC(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in WEIGHT_FIELDS]


class LmHeadC(C.Structure):
    _fields_ = [("ln_g", C.c_void_p), ("ln_b", C.c_void_p), ("w", C.c_void_p), ("s", C.c_void_p),
                ("vocab", C.c_int32)]


class MoeDescC(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("ffn", C.c_int32), ("experts", C.c_int32), ("top_k", C.c_int32),
                ("weight_dtype", C.c_int32), ("act_dtype", C.c_int32), ("quant_group", C.c_int32),
                ("ln_eps", C.c_float), ("gelu_tanh", C.c_int32), ("residual", C.c_int32), ("combine", C.c_int32)]


MOE_WEIGHT_FIELDS = ("ln_g", "ln_b", "w_gate", "w1", "b1", "s1", "w2", "b2", "s2",
                     "r_w1", "r_b1", "r_s1", "r_w2", "r_b2", "r_s2")


class MoeWeightsC(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in MOE_WEIGHT_FIELDS]


class KVCacheC(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("d_len", C.c_void_p),
                ("h_len", C.POINTER(C.c_int32)), ("batch", C.c_int32), ("capacity", C.c_int32),
                ("k_scale", C.c_void_p), ("v_scale", C.c_void_p)]


_LIB = None


def lib():
    """Load libdslayer.so. Raises if it has not been built: nothing runs without it."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = C.CDLL(LIB_PATH)
        vp, i32 = C.c_void_p, C.c_int32
        L.ds_layer_create.argtypes = [C.POINTER(LayerDescC), C.POINTER(LayerWeightsC), C.POINTER(vp)]
        L.ds_layer_destroy.argtypes = [vp]
        L.ds_layer_workspace_bytes.argtypes = [vp, i32, i32, i32]
        L.ds_layer_workspace_bytes.restype = C.c_size_t
        L.ds_kv_append.argtypes = [vp, C.POINTER(KVCacheC), vp, vp, i32, i32, vp]
        L.ds_layer_forward_decode.argtypes = [vp, C.POINTER(KVCacheC), vp, vp, i32, vp, C.c_size_t, vp]
        L.ds_layer_forward_prefill.argtypes = [vp, C.POINTER(KVCacheC), vp, vp, i32, i32, vp, C.c_size_t, vp]
        L.ds_quantize_i8.argtypes = [vp, vp, vp, i32, i32, i32, vp]
        L.ds_dequantize_i8.argtypes = [vp, vp, vp, i32, i32, i32, vp]
        L.ds_last_error.restype = C.c_char_p
        L.ds_stack_state_bytes.argtypes = [i32]
        L.ds_stack_state_bytes.restype = C.c_size_t
        L.ds_stack_create.argtypes = [C.POINTER(vp), C.POINTER(KVCacheC), i32, i32, C.POINTER(LmHeadC), vp,
                                      C.c_size_t, C.POINTER(vp)]
        L.ds_stack_forward_generate.argtypes = [vp, vp, vp, vp, vp, i32, vp, C.c_size_t, vp]
        L.ds_stack_forward_generate.restype = C.c_int
        L.ds_layer_time_kernels.argtypes = [vp, C.POINTER(KVCacheC), vp, vp, i32, i32, vp, C.c_size_t, vp,
                                            C.POINTER(C.c_float), C.POINTER(C.c_int32), i32]
        L.ds_layer_time_kernels.restype = C.c_int
        L.ds_stack_destroy.argtypes = [vp]
        L.ds_stack_workspace_bytes.argtypes = [vp, i32]
        L.ds_stack_workspace_bytes.restype = C.c_size_t
        L.ds_stack_groups.argtypes = [vp]
        L.ds_stack_groups.restype = i32
        L.ds_stack_forward_decode.argtypes = [vp, vp, vp, i32, vp, C.c_size_t, vp]
        L.ds_stack_forward_decode_static.argtypes = [vp, vp, vp, i32, vp]
        L.ds_stack_forward_decode_static.restype = C.c_int
        L.ds_stack_check.argtypes = [vp]
        L.ds_stack_set_timeout_us.argtypes = [vp, C.c_int64]
        L.ds_read_probe.argtypes = [vp, C.c_size_t, vp, vp]
        L.ds_moe_create.argtypes = [C.POINTER(MoeDescC), C.POINTER(MoeWeightsC), C.POINTER(vp)]
        L.ds_moe_destroy.argtypes = [vp]
        L.ds_moe_workspace_bytes.argtypes = [vp, i32]
        L.ds_moe_workspace_bytes.restype = C.c_size_t
        L.ds_moe_forward.argtypes = [vp, vp, vp, i32, vp, vp, vp, C.c_size_t, vp]
        L.ds_moe_time_kernels.argtypes = [vp, vp, vp, i32, vp, C.c_size_t, vp, C.POINTER(C.c_float), i32]
        for name in ("ds_moe_create", "ds_moe_destroy", "ds_moe_forward", "ds_moe_time_kernels"):
            getattr(L, name).restype = C.c_int
        for name in ("ds_layer_create", "ds_layer_destroy", "ds_kv_append", "ds_layer_forward_decode",
                     "ds_layer_forward_prefill", "ds_quantize_i8", "ds_dequantize_i8", "ds_stack_create",
                     "ds_stack_destroy", "ds_stack_forward_decode", "ds_stack_check",
                     "ds_stack_set_timeout_us", "ds_read_probe"):
            getattr(L, name).restype = C.c_int
        _LIB = L
    return _LIB


def check(rc: int, what: str):
    """Map a ds_status to a Python exception: ValueError for argument/shape/dtype errors,
    OverflowError for a full KV cache, RuntimeError for HIP errors."""
    if rc == DS_OK:
        return
    msg = f"{what}: {lib().ds_last_error().decode(errors='replace')} (status {rc})"
    if rc == DS_ERR_KV_FULL:
        raise OverflowError(msg)
    if rc in (DS_ERR_HIP,):
        raise RuntimeError(msg)
    if rc == DS_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise ValueError(msg)


def ptr(t):
    """Device (or host) address of a tensor, or None."""
    if t is None:
        return None
    return C.c_void_p(t.data_ptr())


def stream_handle(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def host_lengths(values) -> np.ndarray:
    return np.ascontiguousarray(values, dtype=np.int32)
