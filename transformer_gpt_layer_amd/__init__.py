"""transformer_gpt_layer_amd: a fused pre-LN GPT layer with a KV cache for MI355X (gfx950).

Python face of libdslayer.so (include/ds_layer.h). The classes here marshal torch tensors into the
C ABI; every step of the layer runs in the library's HIP kernels.

The configuration mirrors the inference config of the page "DeepSpeed Inference 内核优化深度解析"
(blog.gitcode.com), section 四 4.2 (dtype fp32 / fp16 / int8 with fp16 as default, max_out_tokens
1024) and section 五 5.2 (int8 with quantize_groups), plus triangular_masking (default True) from
the config table of "DeepSpeed MoE 大规模稀疏模型推理实战指南". As in init_inference on that page, a
config dict (or JSON text / file) and keyword arguments merge, and a key given both ways with
different values raises.
"""
import ctypes as C
import json
import os
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import DS_BF16, DS_F16, DS_F32, DS_I8, check, lib, ptr, stream_handle

__all__ = ["LayerConfig", "make_config", "Layer", "KVCache", "Stack", "MoE", "quantize_i8", "dequantize_i8"]

_DTYPE_NAMES = {"fp32": DS_F32, "float32": DS_F32, "float": DS_F32, "f32": DS_F32,
                "fp16": DS_F16, "float16": DS_F16, "half": DS_F16, "f16": DS_F16,
                "int8": DS_I8, "i8": DS_I8, "bf16": DS_BF16, "bfloat16": DS_BF16}
_TORCH_DT = {DS_F32: torch.float32, DS_F16: torch.float16, DS_I8: torch.int8, DS_BF16: torch.bfloat16}


def _dtype_code(v) -> int:
    if isinstance(v, torch.dtype):
        v = {torch.float32: "fp32", torch.float16: "fp16", torch.int8: "int8", torch.bfloat16: "bf16"}.get(v, str(v))
    if isinstance(v, int) and v in (DS_F32, DS_F16, DS_I8, DS_BF16):
        return v
    key = str(v).lower().replace("torch.", "")
    if key not in _DTYPE_NAMES:
        raise ValueError(f"unsupported dtype {v!r}: fp32, fp16, bf16 or int8")
    return _DTYPE_NAMES[key]


@dataclass(frozen=True)
class LayerConfig:
    hidden: int
    heads: int
    ffn: int
    dtype: int = DS_F16            # weight dtype; activations: fp32 for fp32, bf16 for bf16, else fp16
    quant_group: int = 0           # int8 only: elements per scale along the reduction dimension
    quant_group_mlp: int = 0       # int8 only: elements per scale of the MLP matrices (0: quant_group)
    ln_eps: float = 1e-5
    gelu_tanh: bool = False
    triangular_masking: bool = True
    max_out_tokens: int = 1024
    kv_dtype: int = 0              # 0: the cache in the activation dtype; DS_I8: int8 rows, fp16 scales

    @property
    def head_dim(self) -> int:
        return self.hidden // self.heads

    @property
    def act_dtype(self) -> int:
        return self.dtype if self.dtype in (DS_F32, DS_BF16) else DS_F16

    @property
    def torch_act_dtype(self) -> torch.dtype:
        return _TORCH_DT[self.act_dtype]

    def c_desc(self) -> _lib.LayerDescC:
        return _lib.LayerDescC(self.hidden, self.heads, self.head_dim, self.ffn, self.dtype,
                               self.act_dtype, self.quant_group, self.quant_group_mlp, self.ln_eps,
                               int(self.gelu_tanh), int(self.triangular_masking), int(self.kv_dtype))

    @property
    def torch_cache_dtype(self) -> torch.dtype:
        return torch.int8 if self.kv_dtype == DS_I8 else self.torch_act_dtype


_CONFIG_KEYS = {"hidden", "heads", "ffn", "dtype", "quant_group", "quant_group_mlp", "ln_eps", "gelu_tanh",
                "triangular_masking", "max_out_tokens", "quantization_setting", "kv_dtype"}


def make_config(config=None, **kwargs) -> LayerConfig:
    """Merge a config (dict, JSON text or JSON file path) with keyword arguments.

    Keyword arguments add to the config; a key present in both with different values raises
    ValueError.

    int8 grouping. `quant_group` gives the group size directly (elements per fp16 scale along the
    reduction dimension; 64 when int8 is chosen without a setting). `quantization_setting` follows
    the page "DeepSpeed Inference 内核优化深度解析", section 五 5.2: (quantize_groups,
    mlp_extra_grouping), where quantize_groups is a number of groups. Read here as the number of
    groups each weight row of the hidden-width reduction (K = hidden) is cut into, so the group size
    is hidden / quantize_groups, which must divide evenly; mlp_extra_grouping=True asks for twice as
    many groups (half the group size) in the MLP matrices. A bare int is taken the same way as
    quantize_groups. Group sizes must be multiples of 16 dividing the matrices' reduction widths.
    """
    base = {}
    if config is not None:
        if isinstance(config, str):
            config = json.load(open(config)) if os.path.exists(config) else json.loads(config)
        base = dict(config)
    for k, v in kwargs.items():
        if k in base and base[k] != v:
            raise ValueError(f"Conflicting argument '{k}' in 'config':{base[k]!r} and kwargs:{v!r}")
        base[k] = v
    unknown = set(base) - _CONFIG_KEYS
    if unknown:
        raise ValueError(f"unknown config keys: {sorted(unknown)}")
    dt = _dtype_code(base.pop("dtype", "fp16"))
    kvd = base.pop("kv_dtype", None)
    if kvd in (None, 0, "auto"):
        kvd = 0
    else:
        kvd = _dtype_code(kvd)
        if kvd != DS_I8 and kvd != (dt if dt in (DS_F32, DS_BF16) else DS_F16):
            raise ValueError("kv_dtype is the activation dtype (the default) or int8")
        kvd = DS_I8 if kvd == DS_I8 else 0
    base["kv_dtype"] = kvd
    qs = base.pop("quantization_setting", None)
    group = base.pop("quant_group", None)
    group_mlp = base.pop("quant_group_mlp", None)
    if qs is not None:
        count, extra = (qs[0], bool(qs[1]) if len(qs) > 1 else False) if isinstance(qs, (tuple, list)) else (qs, False)
        count = int(count)
        hidden = int(base.get("hidden", 0))
        if count < 1 or hidden < 1 or hidden % count:
            raise ValueError(f"quantize_groups {count} must be a positive number of groups dividing hidden {hidden}")
        g = hidden // count
        if group is not None and int(group) != g:
            raise ValueError(f"quant_group {group} and quantization_setting ({count} groups -> {g}) disagree")
        group = g
        if extra:
            if g % 2:
                raise ValueError(f"mlp_extra_grouping needs an even group size, got {g}")
            if group_mlp is not None and int(group_mlp) != g // 2:
                raise ValueError("quant_group_mlp and mlp_extra_grouping disagree")
            group_mlp = g // 2
    if dt == DS_I8:
        group = 64 if group is None else int(group)
        group_mlp = 0 if group_mlp is None or int(group_mlp) == group else int(group_mlp)
    elif group not in (None, 0) or group_mlp not in (None, 0):
        raise ValueError("quant_group and quantization_setting apply to int8 weights only")
    else:
        group, group_mlp = 0, 0
    return LayerConfig(dtype=dt, quant_group=group, quant_group_mlp=group_mlp, **base)


class KVCache:
    """Caller-owned K/V cache of one layer: k, v [batch][heads][capacity][head_dim] in the
    activation dtype (or int8 codes with fp16 row scales k_scale, v_scale [batch][heads][capacity]
    for a layer whose kv_dtype is int8), device lengths d_len int32[batch] and an optional host
    mirror."""

    def __init__(self, batch, heads, capacity, head_dim, dtype, device="cuda", track_host=True):
        self.batch, self.heads, self.capacity, self.head_dim = batch, heads, capacity, head_dim
        self.k = torch.zeros((batch, heads, capacity, head_dim), dtype=dtype, device=device)
        self.v = torch.zeros_like(self.k)
        self.k_scale = self.v_scale = None
        if dtype == torch.int8:
            self.k_scale = torch.zeros((batch, heads, capacity), dtype=torch.float16, device=device)
            self.v_scale = torch.zeros_like(self.k_scale)
        self.d_len = torch.zeros(batch, dtype=torch.int32, device=device)
        self.h_len = _lib.host_lengths([0] * batch) if track_host else None
        self._c = None

    def c_struct(self) -> _lib.KVCacheC:
        hl = self.h_len.ctypes.data_as(C.POINTER(C.c_int32)) if self.h_len is not None else None
        self._c = _lib.KVCacheC(self.k.data_ptr(), self.v.data_ptr(), self.d_len.data_ptr(), hl,
                                self.batch, self.capacity, ptr(self.k_scale), ptr(self.v_scale))
        return self._c

    def dequantized(self):
        """(k, v) as float32: the stored values, q * s for an int8 cache."""
        if self.k_scale is None:
            return self.k.float(), self.v.float()
        return self.k.float() * self.k_scale.float()[..., None], self.v.float() * self.v_scale.float()[..., None]

    def set_lengths(self, lengths):
        vals = [int(v) for v in lengths]
        self.d_len.copy_(torch.tensor(vals, dtype=torch.int32))
        if self.h_len is not None:
            self.h_len[:] = vals

    def lengths(self):
        return self.d_len.cpu().tolist()


class Layer:
    """One layer bound to device weight tensors (borrowed: keep them alive with the layer)."""

    _SHAPES = {"ln1_g": "H", "ln1_b": "H", "w_qkv": ("3H", "H"), "b_qkv": "3H", "w_o": ("H", "H"),
               "b_o": "H", "ln2_g": "H", "ln2_b": "H", "w_ff1": ("F", "H"), "b_ff1": "F",
               "w_ff2": ("H", "F"), "b_ff2": "H"}

    def __init__(self, cfg: LayerConfig, weights: dict):
        self.cfg = cfg
        H, F = cfg.hidden, cfg.ffn
        dims = {"H": H, "3H": 3 * H, "F": F}
        wdt, adt = _TORCH_DT[cfg.dtype], cfg.torch_act_dtype
        for name, shp in self._SHAPES.items():
            t = weights.get(name)
            if t is None:
                raise ValueError(f"missing weight {name}")
            want = tuple(dims[s] for s in shp) if isinstance(shp, tuple) else (dims[shp],)
            if tuple(t.shape) != want:
                raise ValueError(f"{name}: shape {tuple(t.shape)} != {want}")
            exp = wdt if name.startswith("w_") else adt
            if t.dtype != exp:
                raise ValueError(f"{name}: dtype {t.dtype} != {exp}")
            if not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")
        if cfg.dtype == DS_I8:
            for name in ("s_qkv", "s_o", "s_ff1", "s_ff2"):
                t = weights.get(name)
                if t is None or t.dtype != torch.float16 or not t.is_contiguous():
                    raise ValueError(f"{name}: int8 weights need contiguous fp16 scales")
        self._weights = dict(weights)
        cw = _lib.LayerWeightsC(*[self._weights[n].data_ptr() if self._weights.get(n) is not None else None
                                  for n in _lib.WEIGHT_FIELDS])
        h = C.c_void_p()
        check(lib().ds_layer_create(C.byref(cfg.c_desc()), C.byref(cw), C.byref(h)), "ds_layer_create")
        self._h = h

    def close(self):
        """Release the library handle (the weight tensors stay the caller's). Idempotent."""
        h, self._h = getattr(self, "_h", None), None
        if h is not None and h.value:
            lib().ds_layer_destroy(h)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        # at interpreter shutdown the modules this needs may already be gone: then the process
        # ends anyway and the small host handle goes with it
        try:
            self.close()
        except Exception:
            pass

    @property
    def handle(self):
        if self._h is None:
            raise ValueError("layer is closed")
        return self._h

    def workspace_bytes(self, batch, tokens, capacity) -> int:
        return int(lib().ds_layer_workspace_bytes(self.handle, batch, tokens, capacity))

    def workspace(self, batch, tokens, capacity, device="cuda") -> torch.Tensor:
        return torch.empty(self.workspace_bytes(batch, tokens, capacity), dtype=torch.uint8, device=device)

    def _io(self, x, y, shape):
        if tuple(x.shape) != shape or x.dtype != self.cfg.torch_act_dtype or not x.is_contiguous():
            raise ValueError(f"x must be contiguous {shape} {self.cfg.torch_act_dtype}")
        if y is None:
            y = torch.empty_like(x)
        elif tuple(y.shape) != shape or y.dtype != x.dtype or not y.is_contiguous():
            raise ValueError("y must match x")
        return y

    def decode(self, kv: KVCache, x, y=None, workspace=None, stream=None):
        """One decode step: x, y [batch, hidden]."""
        B = x.shape[0]
        y = self._io(x, y, (B, self.cfg.hidden))
        if workspace is None:
            workspace = self.workspace(B, 1, kv.capacity, x.device)
        check(lib().ds_layer_forward_decode(self.handle, C.byref(kv.c_struct()), ptr(x), ptr(y), B,
                                            ptr(workspace), workspace.numel(), stream_handle(stream)),
              "ds_layer_forward_decode")
        return y

    def prefill(self, kv: KVCache, x, y=None, workspace=None, stream=None):
        """Prefill: x, y [batch, seq, hidden]."""
        B, S = x.shape[0], x.shape[1]
        y = self._io(x, y, (B, S, self.cfg.hidden))
        if workspace is None:
            workspace = self.workspace(B, S, kv.capacity, x.device)
        check(lib().ds_layer_forward_prefill(self.handle, C.byref(kv.c_struct()), ptr(x), ptr(y), B, S,
                                             ptr(workspace), workspace.numel(), stream_handle(stream)),
              "ds_layer_forward_prefill")
        return y

    def time_kernels(self, kv: KVCache, x, y=None, workspace=None, stream=None):
        """One decode ([batch, hidden]) or prefill ([batch, seq, hidden]) step with an event between
        kernel launches: returns [(part name, milliseconds)] in launch order. Synchronizes."""
        B = x.shape[0]
        T = 1 if x.dim() == 2 else x.shape[1]
        y = self._io(x, y, tuple(x.shape))
        if workspace is None:
            workspace = self.workspace(B, T, kv.capacity, x.device)
        ms = (C.c_float * 16)()
        kinds = (C.c_int32 * 16)()
        n = lib().ds_layer_time_kernels(self.handle, C.byref(kv.c_struct()), ptr(x), ptr(y), B, T, ptr(workspace),
                                        workspace.numel(), stream_handle(stream), ms, kinds, 16)
        check(min(n, 0), "ds_layer_time_kernels")
        return [(_lib.PARTS[kinds[i]], float(ms[i])) for i in range(n)]

    def kv_append(self, kv: KVCache, k_new, v_new, stream=None):
        """Copy k_new, v_new [batch, ntok, hidden] into the cache after the filled rows."""
        B, T = k_new.shape[0], k_new.shape[1]
        for t in (k_new, v_new):
            if tuple(t.shape) != (B, T, self.cfg.hidden) or t.dtype != self.cfg.torch_act_dtype or not t.is_contiguous():
                raise ValueError("k_new, v_new must be contiguous [batch, ntok, hidden] in the activation dtype")
        check(lib().ds_kv_append(self.handle, C.byref(kv.c_struct()), ptr(k_new), ptr(v_new), B, T,
                                 stream_handle(stream)), "ds_kv_append")


class Stack:
    """Persistent decode of a whole stack: layers[l] bound to caches[l]; one launch per step.

    The layers (and their weight tensors) and the caches must outlive the stack. The stack's device
    state (layer table, launch counter, error flag) is a tensor this object owns. Call close() (or
    use the stack as a context manager) when done: it releases the library handle at a point the
    program chooses rather than during interpreter shutdown.
    """

    def __init__(self, layers, caches, max_batch: int = 1, device="cuda", head=None):
        """head: optional LM head, a dict with ln_g, ln_b [hidden] (activation dtype), w [vocab,
        hidden] (weight dtype) and, for int8 weights, s [vocab, hidden / group] fp16 scales; the
        tensors are borrowed and must outlive the stack."""
        if len(layers) != len(caches) or not layers:
            raise ValueError("need one cache per layer")
        self.layers, self.caches, self.max_batch = list(layers), list(caches), max_batch
        cfg = layers[0].cfg
        self._head = None
        chead = None
        if head is not None:
            w = head["w"]
            if w.dim() != 2 or w.shape[1] != cfg.hidden or not w.is_contiguous() or w.dtype != _TORCH_DT[cfg.dtype]:
                raise ValueError(f"head w must be a contiguous [vocab, {cfg.hidden}] {_TORCH_DT[cfg.dtype]} tensor")
            for n in ("ln_g", "ln_b"):
                t = head[n]
                if tuple(t.shape) != (cfg.hidden,) or t.dtype != cfg.torch_act_dtype or not t.is_contiguous():
                    raise ValueError(f"head {n} must be a contiguous [{cfg.hidden}] {cfg.torch_act_dtype} tensor")
            s = head.get("s")
            self._head = dict(head)
            self.vocab = int(w.shape[0])
            chead = C.byref(_lib.LmHeadC(head["ln_g"].data_ptr(), head["ln_b"].data_ptr(), w.data_ptr(),
                                         s.data_ptr() if s is not None else None, self.vocab))
        handles = (C.c_void_p * len(layers))(*[l.handle.value for l in layers])
        self._cstructs = (_lib.KVCacheC * len(caches))(*[c.c_struct() for c in caches])
        nbytes = int(lib().ds_stack_state_bytes(len(layers)))
        self._state = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=device)
        h = C.c_void_p()
        check(lib().ds_stack_create(handles, self._cstructs, len(layers), max_batch, chead, ptr(self._state),
                                    self._state.numel(), C.byref(h)), "ds_stack_create")
        self._h = h
        self.cfg = layers[0].cfg

    def close(self):
        """Release the library handle; the state tensor is freed with this object. Idempotent."""
        h, self._h = getattr(self, "_h", None), None
        if h is not None and h.value:
            lib().ds_stack_destroy(h)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _handle(self):
        if self._h is None:
            raise ValueError("stack is closed")
        return self._h

    @property
    def groups(self) -> int:
        return int(lib().ds_stack_groups(self._handle()))

    def workspace_bytes(self, batch) -> int:
        return int(lib().ds_stack_workspace_bytes(self._handle(), batch))

    def workspace(self, batch, device="cuda") -> torch.Tensor:
        n = self.workspace_bytes(batch)
        if n == 0:
            raise ValueError(f"batch {batch} outside 1..{self.max_batch}")
        return torch.empty(n, dtype=torch.uint8, device=device)

    def decode(self, x, y=None, workspace=None, stream=None):
        """One decode step through every layer: x, y [batch, hidden]."""
        B = x.shape[0]
        if tuple(x.shape) != (B, self.cfg.hidden) or x.dtype != self.cfg.torch_act_dtype or not x.is_contiguous():
            raise ValueError("x must be contiguous [batch, hidden] in the activation dtype")
        y = torch.empty_like(x) if y is None else y
        if workspace is None:
            workspace = self.workspace(B, x.device)
        check(lib().ds_stack_forward_decode(self._handle(), ptr(x), ptr(y), B, ptr(workspace), workspace.numel(),
                                            stream_handle(stream)), "ds_stack_forward_decode")
        return y

    def generate(self, x, y=None, logits=None, tokens=None, workspace=None, stream=None):
        """One generation step: every layer, then the LM head and the greedy choice, in one launch.
        Returns (y, logits, tokens); pass logits=False to skip storing the logits."""
        B = x.shape[0]
        if tuple(x.shape) != (B, self.cfg.hidden) or x.dtype != self.cfg.torch_act_dtype or not x.is_contiguous():
            raise ValueError("x must be contiguous [batch, hidden] in the activation dtype")
        if self._head is None:
            raise ValueError("this stack has no LM head")
        y = torch.empty_like(x) if y is None else y
        if logits is None:
            logits = torch.empty((B, self.vocab), dtype=torch.float32, device=x.device)
        tokens = torch.empty(max(B, 4), dtype=torch.int32, device=x.device) if tokens is None else tokens
        if workspace is None:
            workspace = self.workspace(B, x.device)
        check(lib().ds_stack_forward_generate(self._handle(), ptr(x), ptr(y), ptr(logits) if logits is not False else None,
                                              ptr(tokens), B, ptr(workspace), workspace.numel(), stream_handle(stream)),
              "ds_stack_forward_generate")
        return y, (logits if logits is not False else None), tokens[:B]

    def decode_static(self, x, y=None, stream=None):
        """The same step with the library's static device scratch as workspace: allocates nothing
        (for callers that cannot allocate). Calls that overlap on one GPU race."""
        B = x.shape[0]
        if tuple(x.shape) != (B, self.cfg.hidden) or x.dtype != self.cfg.torch_act_dtype or not x.is_contiguous():
            raise ValueError("x must be contiguous [batch, hidden] in the activation dtype")
        if y is None:
            raise ValueError("decode_static writes into a caller-provided y (it allocates nothing)")
        check(lib().ds_stack_forward_decode_static(self._handle(), ptr(x), ptr(y), B, stream_handle(stream)),
              "ds_stack_forward_decode_static")
        return y

    def check(self):
        """Synchronize; raise if a step hit the wait timeout (the state is then reset)."""
        check(lib().ds_stack_check(self._handle()), "ds_stack_check")

    def set_timeout_us(self, us: int):
        check(lib().ds_stack_set_timeout_us(self._handle(), int(us)), "ds_stack_set_timeout_us")


def read_probe(buf: torch.Tensor, out: torch.Tensor, stream=None):
    """Stream-read every byte of the device tensor buf once; out (int32, 1 element) receives a
    digest. The launch time gives the HBM read bandwidth the device reaches."""
    if not buf.is_cuda or not buf.is_contiguous() or (buf.numel() * buf.element_size()) % 16:
        raise ValueError("buf must be a contiguous device tensor of a multiple of 16 bytes")
    if out.dtype != torch.int32 or out.numel() < 1 or not out.is_cuda:
        raise ValueError("out must be a device int32 tensor")
    check(lib().ds_read_probe(ptr(buf), buf.numel() * buf.element_size(), ptr(out), stream_handle(stream)),
          "ds_read_probe")


class MoE:
    """The MoE expert FF of one layer (ds_moe_* in include/ds_layer.h): y = x2 + the gated top-k
    experts' FF of LN(x2), plus a dense MLP for the residual (PR-MoE) type; the gate reading is the
    one stated with ds_moe_desc. Weights (device tensors, contiguous): ln_g, ln_b [H] and w_gate
    [E,H] in the activation dtype; w1 [E,F,H], b1 [E,F], w2 [E,H,F], b2 [E,H] (weights in the weight
    dtype, biases in the activation dtype; int8 also s1 [E,F,H/g], s2 [E,H,F/g] fp16); for the
    residual type r_w1 [F,H], r_b1 [F], r_w2 [H,F], r_b2 [H] (and r_s1, r_s2 for int8)."""

    def __init__(self, hidden: int, ffn: int, experts: int, top_k: int, weights: dict, dtype="fp16",
                 quant_group=None, ln_eps: float = 1e-5, gelu_tanh: bool = False, combine: int = 0):
        dt = _dtype_code(dtype)
        adt = dt if dt in (DS_F32, DS_BF16) else DS_F16
        self.dtype, self.act_dtype = dt, adt
        self.hidden, self.ffn, self.experts, self.top_k = hidden, ffn, experts, top_k
        self.residual = weights.get("r_w1") is not None
        group = (64 if quant_group is None else int(quant_group)) if dt == DS_I8 else 0
        if dt != DS_I8 and quant_group not in (None, 0):
            raise ValueError("quant_group applies to int8 weights only")
        H, F, E = hidden, ffn, experts
        wdt, atd = _TORCH_DT[dt], _TORCH_DT[adt]
        shapes = {"ln_g": ((H,), atd), "ln_b": ((H,), atd), "w_gate": ((E, H), atd),
                  "w1": ((E, F, H), wdt), "b1": ((E, F), atd), "w2": ((E, H, F), wdt), "b2": ((E, H), atd)}
        if dt == DS_I8:
            shapes.update({"s1": ((E, F, H // group), torch.float16), "s2": ((E, H, F // group), torch.float16)})
        if self.residual:
            shapes.update({"r_w1": ((F, H), wdt), "r_b1": ((F,), atd), "r_w2": ((H, F), wdt), "r_b2": ((H,), atd)})
            if dt == DS_I8:
                shapes.update({"r_s1": ((F, H // group), torch.float16), "r_s2": ((H, F // group), torch.float16)})
        for name, (shp, dty) in shapes.items():
            t = weights.get(name)
            if t is None:
                raise ValueError(f"missing MoE weight {name}")
            if tuple(t.shape) != shp or t.dtype != dty or not t.is_contiguous():
                raise ValueError(f"{name}: need a contiguous {shp} {dty} tensor, got {tuple(t.shape)} {t.dtype}")
        extra = set(k for k, v in weights.items() if v is not None) - set(shapes)
        if extra:
            raise ValueError(f"unexpected MoE weights {sorted(extra)}")
        self._weights = dict(weights)
        self._desc = _lib.MoeDescC(H, F, E, top_k, dt, adt, group, ln_eps, int(gelu_tanh), int(self.residual), int(combine))
        cw = _lib.MoeWeightsC(*[ptr(self._weights.get(n)) for n in _lib.MOE_WEIGHT_FIELDS])
        h = C.c_void_p()
        check(lib().ds_moe_create(C.byref(self._desc), C.byref(cw), C.byref(h)), "ds_moe_create")
        self._h = h
        self.device = weights["w1"].device

    def close(self):
        h, self._h = getattr(self, "_h", None), None
        if h is not None and h.value:
            lib().ds_moe_destroy(h)

    def __del__(self):
        self.close()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def _handle(self):
        if self._h is None:
            raise ValueError("MoE is closed")
        return self._h

    def workspace(self, tokens: int) -> torch.Tensor:
        n = lib().ds_moe_workspace_bytes(self._handle(), tokens)
        if n == 0:
            raise ValueError(f"tokens {tokens} out of range")
        return torch.empty(n, dtype=torch.uint8, device=self.device)

    def _check_x(self, x2):
        if x2.dim() != 2 or x2.shape[1] != self.hidden or x2.dtype != _TORCH_DT[self.act_dtype] or not x2.is_contiguous():
            raise ValueError(f"x2 must be a contiguous [tokens, {self.hidden}] {_TORCH_DT[self.act_dtype]} tensor")

    def forward(self, x2: torch.Tensor, y=None, workspace=None, stream=None, routing: bool = False):
        """y [T,H] for x2 [T,H]; with routing=True also the chosen experts (int32 [T,k]) and their
        combine weights (fp32 [T,k])."""
        self._check_x(x2)
        T = x2.shape[0]
        y = torch.empty_like(x2) if y is None else y
        ws = self.workspace(T) if workspace is None else workspace
        sel = torch.empty((T, self.top_k), dtype=torch.int32, device=x2.device) if routing else None
        wgt = torch.empty((T, self.top_k), dtype=torch.float32, device=x2.device) if routing else None
        check(lib().ds_moe_forward(self._handle(), ptr(x2), ptr(y), T, ptr(sel), ptr(wgt), ptr(ws), ws.numel(),
                                   stream_handle(stream)), "ds_moe_forward")
        return (y, sel, wgt) if routing else y

    def time_kernels(self, x2: torch.Tensor, y=None, workspace=None, stream=None):
        """Per-launch milliseconds of one step: a dict over MOE_PARTS (synchronizes)."""
        self._check_x(x2)
        T = x2.shape[0]
        y = torch.empty_like(x2) if y is None else y
        ws = self.workspace(T) if workspace is None else workspace
        ms = (C.c_float * 8)()
        n = lib().ds_moe_time_kernels(self._handle(), ptr(x2), ptr(y), T, ptr(ws), ws.numel(), stream_handle(stream), ms, 8)
        if n < 0:
            check(n, "ds_moe_time_kernels")
        return {_lib.MOE_PARTS[i]: ms[i] for i in range(n)}


def quantize_i8(w: torch.Tensor, group: int = 64, stream=None):
    """Group-wise symmetric int8 quantization on the GPU: w float32 [n, k] ->
    (q int8 [n, k], s float16 [n, k/group])."""
    if w.dtype != torch.float32 or w.dim() != 2 or not w.is_contiguous():
        raise ValueError("w must be a contiguous 2-D float32 tensor")
    n, k = w.shape
    q = torch.empty((n, k), dtype=torch.int8, device=w.device)
    s = torch.empty((n, k // group if group else 0), dtype=torch.float16, device=w.device)
    check(lib().ds_quantize_i8(ptr(w), ptr(q), ptr(s), n, k, group, stream_handle(stream)), "ds_quantize_i8")
    return q, s


def dequantize_i8(q: torch.Tensor, s: torch.Tensor, group: int = 64, stream=None):
    """w = q * s as float32, through the GEMV kernels' int8 -> fp16 conversion."""
    n, k = q.shape
    w = torch.empty((n, k), dtype=torch.float32, device=q.device)
    check(lib().ds_dequantize_i8(ptr(q), ptr(s), ptr(w), n, k, group, stream_handle(stream)), "ds_dequantize_i8")
    return w
