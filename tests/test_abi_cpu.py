"""The C ABI on the host: the library loads, exports every declared symbol, and rejects bad
arguments before anything is enqueued (no GPU needed: these paths make no HIP call)."""
import ctypes as C
import os
import re

import numpy as np
import pytest
import torch

import transformer_gpt_layer_amd as tg
from transformer_gpt_layer_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # a 16-byte aligned address that is never dereferenced on these paths


def _declared():
    names = set()
    for h in os.listdir(os.path.join(ROOT, "include")):
        if h.endswith(".h"):
            txt = open(os.path.join(ROOT, "include", h)).read()
            names |= set(re.findall(r"^\s*(?:int32_t|int|size_t|const char\*)\s+(ds_\w+)\s*\(", txt, re.M))
    return names


def test_exports_every_declared_symbol():
    L = _lib.lib()
    declared = _declared()
    assert declared == set(_lib.EXPORTS), declared ^ set(_lib.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def _desc(**kw):
    d = dict(hidden=256, heads=2, head_dim=128, ffn=512, weight_dtype=1, act_dtype=1, quant_group=0,
             quant_group_mlp=0, ln_eps=1e-5, gelu_tanh=0, triangular_masking=1)
    d.update(kw)
    return _lib.LayerDescC(**d)


def _weights(int8=False, **kw):
    vals = {n: FAKE for n in _lib.WEIGHT_FIELDS}
    if not int8:
        for n in ("s_qkv", "s_o", "s_ff1", "s_ff2"):
            vals[n] = None
    vals.update(kw)
    return _lib.LayerWeightsC(**vals)


def _create(desc, w):
    h = C.c_void_p()
    rc = _lib.lib().ds_layer_create(C.byref(desc), C.byref(w), C.byref(h))
    return rc, h


@pytest.mark.parametrize("kw,code", [
    (dict(hidden=250), _lib.DS_ERR_SHAPE),
    (dict(head_dim=96, hidden=192, heads=2), _lib.DS_ERR_SHAPE),
    (dict(heads=3), _lib.DS_ERR_SHAPE),
    (dict(ffn=100), _lib.DS_ERR_SHAPE),
    (dict(weight_dtype=2, act_dtype=2), _lib.DS_ERR_DTYPE),
    (dict(weight_dtype=0, act_dtype=1), _lib.DS_ERR_DTYPE),
    (dict(weight_dtype=3, act_dtype=1), _lib.DS_ERR_DTYPE),      # bf16 weights need bf16 activations
    (dict(weight_dtype=1, act_dtype=3), _lib.DS_ERR_DTYPE),
    (dict(weight_dtype=2, act_dtype=3, quant_group=64), _lib.DS_ERR_DTYPE),
    (dict(weight_dtype=4, act_dtype=4), _lib.DS_ERR_DTYPE),
    (dict(weight_dtype=3, act_dtype=3, quant_group=64), _lib.DS_ERR_DTYPE),
    (dict(quant_group=64), _lib.DS_ERR_DTYPE),
    (dict(quant_group_mlp=32), _lib.DS_ERR_DTYPE),
    # int8 groups: multiples of 16 that divide the reduction width of their matrices
    (dict(weight_dtype=2, act_dtype=1, quant_group=24), _lib.DS_ERR_SHAPE),
    (dict(weight_dtype=2, act_dtype=1, quant_group=0), _lib.DS_ERR_SHAPE),
    (dict(weight_dtype=2, act_dtype=1, quant_group=48), _lib.DS_ERR_SHAPE),      # 48 does not divide 256
    (dict(weight_dtype=2, act_dtype=1, quant_group=512), _lib.DS_ERR_SHAPE),
    (dict(weight_dtype=2, act_dtype=1, quant_group=64, quant_group_mlp=24), _lib.DS_ERR_SHAPE),
    (dict(weight_dtype=2, act_dtype=1, quant_group=64, quant_group_mlp=-32), _lib.DS_ERR_SHAPE),
    (dict(weight_dtype=2, act_dtype=1, quant_group=64, quant_group_mlp=96), _lib.DS_ERR_SHAPE),
    (dict(ln_eps=0.0), _lib.DS_ERR_SHAPE),
    (dict(triangular_masking=2), _lib.DS_ERR_SHAPE),
])
def test_create_rejects_bad_descriptions(kw, code):
    rc, h = _create(_desc(**kw), _weights(int8=kw.get("weight_dtype") == 2))
    assert rc == code, (rc, _lib.lib().ds_last_error())
    assert not h.value
    assert _lib.lib().ds_last_error()


def test_create_rejects_null_and_misaligned_pointers():
    assert _create(_desc(), _weights(w_o=None))[0] == _lib.DS_ERR_NULL
    assert _create(_desc(), _weights(w_ff1=FAKE + 8))[0] == _lib.DS_ERR_ALIGN
    assert _create(_desc(), _weights(s_o=FAKE))[0] == _lib.DS_ERR_DTYPE       # scales on fp16 weights
    assert _create(_desc(weight_dtype=2, quant_group=64), _weights(int8=True, s_ff2=None))[0] == _lib.DS_ERR_NULL
    for ga, gm in ((64, 64), (64, 32), (32, 0), (128, 64), (16, 256)):
        rc, h = _create(_desc(weight_dtype=2, quant_group=ga, quant_group_mlp=gm), _weights(int8=True))
        assert rc == 0, (ga, gm, _lib.lib().ds_last_error())
        _lib.lib().ds_layer_destroy(h)
    h = C.c_void_p()
    assert _lib.lib().ds_layer_create(None, C.byref(_weights()), C.byref(h)) == _lib.DS_ERR_NULL


def _layer():
    rc, h = _create(_desc(), _weights())
    assert rc == 0, _lib.lib().ds_last_error()
    return h


def test_workspace_bytes():
    L, h = _lib.lib(), _layer()
    a = L.ds_layer_workspace_bytes(h, 1, 1, 64)
    b = L.ds_layer_workspace_bytes(h, 8, 1, 64)
    c = L.ds_layer_workspace_bytes(h, 8, 1, 1024)
    assert 0 < a < b < c
    assert L.ds_layer_workspace_bytes(h, 0, 1, 64) == 0
    assert L.ds_layer_workspace_bytes(None, 1, 1, 64) == 0
    L.ds_layer_destroy(h)


def test_int8_workspace_holds_one_fp16_matrix_above_sixteen_rows():
    """int8 layers above the skinny kernel's 16 rows expand each matrix into fp16 in the workspace
    before its MFMA product: the size grows by the largest matrix in fp16 (here Wqkv, 3H x H, which
    is larger than W1 and W2 at F = 2H) plus the row buffers of one more row."""
    L = _lib.lib()
    rc, h = _create(_desc(weight_dtype=2, quant_group=64), _weights(int8=True))
    assert rc == 0, L.ds_last_error()
    H, F = 256, 512
    wmax = max(3 * H * H, F * H) * 2
    at16 = L.ds_layer_workspace_bytes(h, 16, 1, 64)
    at17 = L.ds_layer_workspace_bytes(h, 17, 1, 64)
    assert wmax <= at17 - at16 < wmax + 64 * 1024
    L.ds_layer_destroy(h)
    # fp16 layers carry no such copy
    h16 = _layer()
    assert L.ds_layer_workspace_bytes(h16, 17, 1, 64) - L.ds_layer_workspace_bytes(h16, 16, 1, 64) < 64 * 1024
    L.ds_layer_destroy(h16)


def test_forward_rejects_before_enqueue():
    L, h = _lib.lib(), _layer()
    hl = np.array([63, 10], dtype=np.int32)
    kv = _lib.KVCacheC(FAKE, FAKE, FAKE, hl.ctypes.data_as(C.POINTER(C.c_int32)), 2, 64)
    need = L.ds_layer_workspace_bytes(h, 2, 1, 64)
    # every call below fails a host-side check, so no kernel is ever launched on the fake pointers
    run = lambda batch=2, x=FAKE, ws=need: L.ds_layer_forward_decode(h, C.byref(kv), C.c_void_p(x), C.c_void_p(FAKE), batch, C.c_void_p(FAKE), ws, None)
    hl[:] = [64, 10]
    assert run() == _lib.DS_ERR_KV_FULL
    assert list(hl) == [64, 10]                      # nothing advanced on failure
    hl[:] = [3, 3]
    assert run(batch=3) == _lib.DS_ERR_SHAPE         # more sequences than the cache holds
    assert run(ws=need - 1) == _lib.DS_ERR_WORKSPACE
    assert run(x=FAKE + 4) == _lib.DS_ERR_ALIGN
    assert run(x=0) == _lib.DS_ERR_NULL
    assert L.ds_layer_forward_prefill(h, C.byref(kv), C.c_void_p(FAKE), C.c_void_p(FAKE), 2, 62,
                                      C.c_void_p(FAKE), 1 << 40, None) == _lib.DS_ERR_KV_FULL
    assert L.ds_kv_append(h, C.byref(kv), C.c_void_p(FAKE), C.c_void_p(FAKE), 2, 70, None) == _lib.DS_ERR_KV_FULL
    assert L.ds_quantize_i8(C.c_void_p(FAKE), C.c_void_p(FAKE), C.c_void_p(FAKE), 4, 100, 64, None) == _lib.DS_ERR_SHAPE
    assert L.ds_dequantize_i8(C.c_void_p(FAKE), None, C.c_void_p(FAKE), 4, 128, 64, None) == _lib.DS_ERR_NULL
    L.ds_layer_destroy(h)


def test_python_errors_map_to_exceptions():
    with pytest.raises(OverflowError):
        _lib.check(_lib.DS_ERR_KV_FULL, "x")
    with pytest.raises(ValueError):
        _lib.check(_lib.DS_ERR_SHAPE, "x")
    with pytest.raises(RuntimeError):
        _lib.check(_lib.DS_ERR_HIP, "x")


def test_config_merge_rules():
    cfg = tg.make_config({"hidden": 256, "heads": 2, "ffn": 512}, dtype="int8")
    assert cfg.dtype == _lib.DS_I8 and cfg.quant_group == 64 and cfg.triangular_masking and cfg.max_out_tokens == 1024
    assert tg.make_config('{"hidden": 256, "heads": 4, "ffn": 512}').dtype == _lib.DS_F16   # fp16 default
    assert tg.make_config(hidden=256, heads=2, ffn=512, dtype="int8", quant_group=64).quant_group == 64
    with pytest.raises(ValueError, match="Conflicting"):
        tg.make_config({"hidden": 256, "heads": 2, "ffn": 512, "dtype": "fp16"}, dtype="fp32")
    with pytest.raises(ValueError):
        tg.make_config(hidden=256, heads=2, ffn=512, quant_group=64)          # group on fp16 weights
    with pytest.raises(ValueError):
        tg.make_config(hidden=256, heads=2, ffn=512, bogus=1)


def test_bf16_is_a_weight_and_activation_dtype():
    """dtype bf16 (torch.bfloat16): bf16 weights with bf16 activations, caches and parameters."""
    for v in ("bf16", "bfloat16", torch.bfloat16, "torch.bfloat16"):
        cfg = tg.make_config(hidden=256, heads=2, ffn=512, dtype=v)
        assert cfg.dtype == _lib.DS_BF16 and cfg.act_dtype == _lib.DS_BF16 and cfg.torch_act_dtype == torch.bfloat16
    rc, h = _create(_desc(weight_dtype=3, act_dtype=3), _weights())
    assert rc == 0, _lib.lib().ds_last_error()
    _lib.lib().ds_layer_destroy(h)
    with pytest.raises(ValueError, match="int8"):
        tg.make_config(hidden=256, heads=2, ffn=512, dtype="bf16", quant_group=64)


def test_quantization_setting_is_a_group_count():
    """quantization_setting=(quantize_groups, mlp_extra_grouping): quantize_groups is a number of
    groups per hidden-width weight row, so the group size is hidden / quantize_groups."""
    cfg = tg.make_config(hidden=5120, heads=40, ffn=20480, dtype="int8", quantization_setting=(80, False))
    assert cfg.quant_group == 64 and cfg.quant_group_mlp == 0
    assert tg.make_config(hidden=2560, heads=20, ffn=10240, dtype="int8", quantization_setting=40).quant_group == 64
    with pytest.raises(ValueError, match="dividing hidden"):
        tg.make_config(hidden=2560, heads=20, ffn=10240, dtype="int8", quantization_setting=(48, False))
    with pytest.raises(ValueError, match="disagree"):
        tg.make_config(hidden=2560, heads=20, ffn=10240, dtype="int8", quantization_setting=(40, False), quant_group=32)
    # extra MLP grouping halves the MLP group size
    cfg = tg.make_config(hidden=5120, heads=40, ffn=20480, dtype="int8", quantization_setting=(80, True))
    assert cfg.quant_group == 64 and cfg.quant_group_mlp == 32
    with pytest.raises(ValueError, match="disagree"):
        tg.make_config(hidden=5120, heads=40, ffn=20480, dtype="int8", quantization_setting=(80, True),
                       quant_group_mlp=64)
    with pytest.raises(ValueError, match="int8"):
        tg.make_config(hidden=256, heads=2, ffn=512, dtype="fp16", quantization_setting=(4, False))


def test_stack_create_rejects_before_device_work():
    """ds_stack_create refuses bad layer counts and state buffers before any HIP call."""
    L, h = _lib.lib(), _layer()
    hl = np.zeros(1, dtype=np.int32)
    n = 600
    handles = (C.c_void_p * n)(*([h.value] * n))
    caches = (_lib.KVCacheC * n)(*[_lib.KVCacheC(FAKE, FAKE, FAKE, hl.ctypes.data_as(C.POINTER(C.c_int32)), 1, 64)
                                   for _ in range(n)])
    out = C.c_void_p()
    need = L.ds_stack_state_bytes(2)
    assert need > 0 and L.ds_stack_state_bytes(0) == 0
    # the tag packs layer * 8 + phase into 12 bits: 511 layers at most
    assert L.ds_stack_create(handles, caches, 512, 1, None, C.c_void_p(FAKE), 1 << 30, C.byref(out)) == _lib.DS_ERR_UNSUPPORTED
    assert L.ds_stack_create(handles, caches, n, 1, None, C.c_void_p(FAKE), 1 << 30, C.byref(out)) == _lib.DS_ERR_UNSUPPORTED
    assert "511" in L.ds_last_error().decode()
    assert L.ds_stack_create(handles, caches, 0, 1, None, C.c_void_p(FAKE), 1 << 30, C.byref(out)) == _lib.DS_ERR_SHAPE
    assert L.ds_stack_create(handles, caches, 2, 1, None, None, need, C.byref(out)) == _lib.DS_ERR_NULL
    assert L.ds_stack_create(handles, caches, 2, 1, None, C.c_void_p(FAKE + 8), need, C.byref(out)) == _lib.DS_ERR_ALIGN
    assert L.ds_stack_create(handles, caches, 2, 1, None, C.c_void_p(FAKE), need - 1, C.byref(out)) == _lib.DS_ERR_WORKSPACE
    assert L.ds_stack_create(handles, caches, 2, 5, None, C.c_void_p(FAKE), need, C.byref(out)) == _lib.DS_ERR_UNSUPPORTED
    assert not out.value
    L.ds_layer_destroy(h)
    # LM head descriptions are checked before any device work too (on a stack-compatible layer)
    rc, h2 = _create(_desc(hidden=512, heads=4, ffn=1024), _weights())
    assert rc == 0
    handles = (C.c_void_p * 2)(h2.value, h2.value)
    bad = [_lib.LmHeadC(FAKE, FAKE, None, None, 100), _lib.LmHeadC(FAKE, FAKE, FAKE + 8, None, 100),
           _lib.LmHeadC(FAKE, FAKE, FAKE, FAKE, 100), _lib.LmHeadC(FAKE, FAKE, FAKE, None, 0),
           _lib.LmHeadC(FAKE, FAKE, FAKE, None, 1 << 21)]
    codes = [_lib.DS_ERR_NULL, _lib.DS_ERR_ALIGN, _lib.DS_ERR_DTYPE, _lib.DS_ERR_SHAPE, _lib.DS_ERR_SHAPE]
    for head, code in zip(bad, codes):
        rc = L.ds_stack_create(handles, caches, 2, 1, C.byref(head), C.c_void_p(FAKE), need, C.byref(out))
        assert rc == code, (rc, L.ds_last_error())
    assert not out.value
    # an int8 kv cache: the stack needs its row scales, and fp16 activations
    rc, h8 = _create(_desc(hidden=512, heads=4, ffn=1024, kv_dtype=_lib.DS_I8), _weights())
    assert rc == 0, L.ds_last_error()
    handles8 = (C.c_void_p * 2)(h8.value, h8.value)
    assert L.ds_stack_create(handles8, caches, 2, 1, None, C.c_void_p(FAKE), need, C.byref(out)) == _lib.DS_ERR_NULL
    assert "k_scale" in L.ds_last_error().decode()
    scaled = (_lib.KVCacheC * 2)(*[_lib.KVCacheC(FAKE, FAKE, FAKE, hl.ctypes.data_as(C.POINTER(C.c_int32)), 1, 64,
                                                 FAKE + 8, FAKE) for _ in range(2)])
    assert L.ds_stack_create(handles8, scaled, 2, 1, None, C.c_void_p(FAKE), need, C.byref(out)) == _lib.DS_ERR_ALIGN
    # scales on the caches of layers whose cache is not int8
    assert L.ds_stack_create(handles, scaled, 2, 1, None, C.c_void_p(FAKE), need, C.byref(out)) == _lib.DS_ERR_DTYPE
    L.ds_layer_destroy(h8)
    rc, hb = _create(_desc(hidden=512, heads=4, ffn=1024, weight_dtype=3, act_dtype=3, kv_dtype=_lib.DS_I8), _weights())
    assert rc == 0, L.ds_last_error()
    handlesb = (C.c_void_p * 2)(hb.value, hb.value)
    # bf16 activations over int8 caches pass the type check; the misaligned scale is what fails
    assert L.ds_stack_create(handlesb, scaled, 2, 1, None, C.c_void_p(FAKE), need, C.byref(out)) == _lib.DS_ERR_ALIGN
    assert not out.value
    L.ds_layer_destroy(hb)
    L.ds_layer_destroy(h2)


def test_layer_close_is_idempotent():
    cfg = tg.make_config(hidden=256, heads=2, ffn=512, dtype="fp16")
    rc, h = _create(_desc(), _weights())
    assert rc == 0
    _lib.lib().ds_layer_destroy(h)
    assert _lib.lib().ds_layer_destroy(None) == 0
    assert cfg.quant_group_mlp == 0


# ------------------------------------------------------------------ the MoE expert FF (host checks)
def _moe_desc(**kw):
    d = dict(hidden=256, ffn=512, experts=8, top_k=2, weight_dtype=1, act_dtype=1, quant_group=0, ln_eps=1e-5,
             gelu_tanh=0, residual=0, combine=0)
    d.update(kw)
    return _lib.MoeDescC(**d)


def _moe_weights(int8=False, residual=False, **over):
    w = {n: FAKE for n in ("ln_g", "ln_b", "w_gate", "w1", "b1", "w2", "b2")}
    if int8:
        w.update(s1=FAKE, s2=FAKE)
    if residual:
        w.update(r_w1=FAKE, r_b1=FAKE, r_w2=FAKE, r_b2=FAKE)
        if int8:
            w.update(r_s1=FAKE, r_s2=FAKE)
    w.update(over)
    return _lib.MoeWeightsC(*[w.get(n) for n in _lib.MOE_WEIGHT_FIELDS])


def _moe_create(desc, weights):
    h = C.c_void_p()
    rc = _lib.lib().ds_moe_create(C.byref(desc), C.byref(weights), C.byref(h))
    return rc, h


@pytest.mark.parametrize("kw,code", [
    (dict(hidden=200), _lib.DS_ERR_SHAPE),
    (dict(ffn=0), _lib.DS_ERR_SHAPE),
    (dict(experts=0), _lib.DS_ERR_SHAPE),
    (dict(experts=1024), _lib.DS_ERR_SHAPE),
    (dict(top_k=0), _lib.DS_ERR_SHAPE),
    (dict(top_k=9, experts=16), _lib.DS_ERR_SHAPE),
    (dict(top_k=3, experts=2), _lib.DS_ERR_SHAPE),
    (dict(weight_dtype=1, act_dtype=3), _lib.DS_ERR_DTYPE),
    (dict(weight_dtype=0, act_dtype=1), _lib.DS_ERR_DTYPE),
    (dict(quant_group=64), _lib.DS_ERR_DTYPE),
    (dict(weight_dtype=2, act_dtype=1, quant_group=24), _lib.DS_ERR_SHAPE),
    (dict(weight_dtype=2, act_dtype=1, quant_group=0), _lib.DS_ERR_SHAPE),
    (dict(ln_eps=0.0), _lib.DS_ERR_SHAPE),
    (dict(combine=2), _lib.DS_ERR_SHAPE),
    (dict(residual=1), _lib.DS_ERR_NULL),      # the residual type without its MLP
])
def test_moe_create_rejects_bad_descriptions(kw, code):
    rc, h = _moe_create(_moe_desc(**kw), _moe_weights(int8=kw.get("weight_dtype") == 2))
    assert rc == code, (rc, _lib.lib().ds_last_error())
    assert not h.value


def test_moe_create_checks_pointers_and_accepts_valid_blocks():
    assert _moe_create(_moe_desc(), _moe_weights(w1=None))[0] == _lib.DS_ERR_NULL
    assert _moe_create(_moe_desc(), _moe_weights(w2=FAKE + 4))[0] == _lib.DS_ERR_ALIGN
    assert _moe_create(_moe_desc(), _moe_weights(s1=FAKE))[0] == _lib.DS_ERR_DTYPE          # scales on fp16
    assert _moe_create(_moe_desc(), _moe_weights(residual=True))[0] == _lib.DS_ERR_SHAPE    # MLP on a standard MoE
    assert _moe_create(_moe_desc(weight_dtype=2, quant_group=64), _moe_weights(int8=True, s2=None))[0] == _lib.DS_ERR_NULL
    for d, w in ((_moe_desc(), _moe_weights()),
                 (_moe_desc(residual=1, combine=1, gelu_tanh=1), _moe_weights(residual=True)),
                 (_moe_desc(weight_dtype=2, quant_group=32, residual=1), _moe_weights(int8=True, residual=True)),
                 (_moe_desc(weight_dtype=3, act_dtype=3, experts=1023, top_k=8), _moe_weights()),
                 (_moe_desc(weight_dtype=0, act_dtype=0, experts=1, top_k=1), _moe_weights())):
        rc, h = _moe_create(d, w)
        assert rc == 0, _lib.lib().ds_last_error()
        L = _lib.lib()
        assert L.ds_moe_workspace_bytes(h, 1) > 0 and L.ds_moe_workspace_bytes(h, 0) == 0
        slots = d.top_k + d.residual
        assert L.ds_moe_workspace_bytes(h, 4096 // slots) > 0 and L.ds_moe_workspace_bytes(h, 4096 // slots + 1) == 0
        # forward: argument errors before anything is enqueued
        ws = L.ds_moe_workspace_bytes(h, 2)
        assert L.ds_moe_forward(h, FAKE, FAKE, 0, None, None, FAKE, ws, None) == _lib.DS_ERR_SHAPE
        assert L.ds_moe_forward(h, FAKE, FAKE, 4096 // slots + 1, None, None, FAKE, ws, None) == _lib.DS_ERR_SHAPE
        assert L.ds_moe_forward(h, None, FAKE, 2, None, None, FAKE, ws, None) == _lib.DS_ERR_NULL
        assert L.ds_moe_forward(h, FAKE + 2, FAKE, 2, None, None, FAKE, ws, None) == _lib.DS_ERR_ALIGN
        assert L.ds_moe_forward(h, FAKE, FAKE, 2, None, None, FAKE, ws - 1, None) == _lib.DS_ERR_WORKSPACE
        L.ds_moe_destroy(h)
