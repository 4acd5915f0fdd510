"""GPU parity of the MFMA (many-row) path against the oracle: fp16 and bf16 layers with at least 16
rows per step run LayerNorm rows, the fused-epilogue GEMMs and flash attention on matrix cores.

Shapes span several GEMM tiles (128 rows by 160/256/320 columns) with ragged row and column tails,
several 64-key attention tiles, past rows that are not a multiple of 64, head_dim 64 and 128, and
both mask settings. The causal mask is also checked by construction: changing prompt row t' leaves
every output row t < t' bit-identical.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from tests._common import TOL, filled_caches, gpu_layer_and_oracle_weights, rel_l2

pytestmark = pytest.mark.gpu


def _wl(**kw):
    base = dict(hidden=256, heads=2, head_dim=128, ffn=768, weight_dtype="f16", act_dtype="f16", batch=2, past=0)
    base.update(kw)
    return dataclasses.replace(syn.WORKLOADS["c1"], **base)


CASES = {
    # rows 200: two row tiles, the second 72 rows; qkv N=768, ff1 N=768, ff2 K=768
    "d128-b2-s100": (_wl(cfg_id=201), 100, 0),
    # past rows 33 before 70 new ones: keys span two tiles with a ragged end; N=960 (3*320) and 640
    "d64-b3-s70-p33": (_wl(hidden=320, heads=5, head_dim=64, ffn=640, batch=3, cfg_id=202), 70, 33),
    # K=2048 for FF2 (64 k-steps), 512 rows, heads of 128
    "d128-b2-s256": (_wl(hidden=512, heads=4, ffn=2048, cfg_id=203), 256, 0),
    # exactly 16 rows: the smallest MFMA-path step
    "d128-b1-s16-p5": (_wl(batch=1, cfg_id=204), 16, 5),
}


AFFINE = dict(ln_std=0.2, bias_std=0.1)


def _prefill_case(wl, S, P0, **cfg_kw):
    wl = dataclasses.replace(wl, past=P0, seq=S)
    cap = ((P0 + S + 1 + 63) // 64) * 64
    gl, ow = gpu_layer_and_oracle_weights(wl, 0, **cfg_kw)
    kv, ok, ov, lens = filled_caches(wl, 0, gl, past=P0, cap=cap)
    x = syn.normal((wl.batch, S, wl.hidden), 1.0, wl.cfg_id, syn.X_LAYER, 7, "cuda").to(gl.cfg.torch_act_dtype)
    return wl, gl, ow, kv, ok, ov, lens, x


# per-layer LayerNorm affine and larger biases, with both GeLU forms
CASES.update({
    "d128-b2-s100-affine-tanh": (_wl(cfg_id=209, **AFFINE), 100, 0),
    "d64-b3-s70-p33-affine": (_wl(hidden=320, heads=5, head_dim=64, ffn=640, batch=3, cfg_id=210, **AFFINE), 70, 33),
})
TANH = {"d128-b2-s100-affine-tanh"}


def _check_prefill(name, wl, S, P0, tanh):
    wl, gl, ow, kv, ok, ov, lens, x = _prefill_case(wl, S, P0, gelu_tanh=tanh)
    print(f"case {name}: B={wl.batch} S={S} P0={P0} H={wl.hidden} F={wl.ffn} d={wl.head_dim} tanh={tanh}", flush=True)
    y = gl.prefill(kv, x)
    torch.cuda.synchronize()
    desc = oracle.Desc(wl.hidden, wl.heads, wl.head_dim, wl.ffn, gelu_tanh=tanh)
    yo = oracle.layer_forward(desc, ow, ok, ov, lens, x.double().cpu().numpy())
    yd, xd = y.double().cpu().numpy(), x.double().cpu().numpy()
    err, err_d = rel_l2(yd, yo), rel_l2(yd - xd, yo - xd)
    print(f"  rel L2 {err:.3e}, of y - x {err_d:.3e}", flush=True)
    tol = TOL[wl.act_dtype]
    assert err <= tol and err_d <= tol, (err, err_d)
    n = P0 + S
    assert rel_l2(kv.k.double().cpu().numpy()[:, :, :n], ok[:, :, :n]) <= tol
    assert rel_l2(kv.v.double().cpu().numpy()[:, :, :n], ov[:, :, :n]) <= tol
    assert kv.lengths() == [n] * wl.batch


@pytest.mark.parametrize("cfg", [0, 1, 2])
@pytest.mark.parametrize("name", ["d128-b2-s256", "d64-b3-s70-p33-affine", "d128-b2-s100-affine-tanh"])
def test_prefill_each_gemm_configuration_matches_oracle(name, cfg, monkeypatch):
    """Every GEMM tile configuration (0: 128 x 160 two-stage, 1: 128 x 160 three-stage with two wave
    groups, 2: 256 x 256 eight waves) forced on all four products of small shapes, whose automatic
    choice would not take it, against the oracle; ragged row and column tiles included."""
    monkeypatch.setenv("DS_GEMM_CONFIG", str(cfg))
    wl, S, P0 = CASES[name]
    _check_prefill(f"{name} config {cfg}", wl, S, P0, name in TANH)


@pytest.mark.parametrize("name", list(CASES))
def test_prefill_mfma_matches_oracle(name):
    wl, S, P0 = CASES[name]
    tanh = name in TANH
    wl, gl, ow, kv, ok, ov, lens, x = _prefill_case(wl, S, P0, gelu_tanh=tanh)
    print(f"case {name}: B={wl.batch} S={S} P0={P0} H={wl.hidden} F={wl.ffn} d={wl.head_dim}", flush=True)
    y = gl.prefill(kv, x)
    torch.cuda.synchronize()
    desc = oracle.Desc(wl.hidden, wl.heads, wl.head_dim, wl.ffn, gelu_tanh=tanh)
    yo = oracle.layer_forward(desc, ow, ok, ov, lens, x.double().cpu().numpy())
    err = rel_l2(y.double().cpu().numpy(), yo)
    assert err <= TOL["f16"], err
    # the same metric on the layer's update y - x, a stricter view of the computed part
    xd = x.double().cpu().numpy()
    assert rel_l2(y.double().cpu().numpy() - xd, yo - xd) <= TOL["f16"]
    n = P0 + S
    assert rel_l2(kv.k.double().cpu().numpy()[:, :, :n], ok[:, :, :n]) <= TOL["f16"]
    assert rel_l2(kv.v.double().cpu().numpy()[:, :, :n], ov[:, :, :n]) <= TOL["f16"]
    assert kv.lengths() == [n] * wl.batch
    assert torch.isfinite(y).all()


def test_prefill_mfma_without_mask_matches_oracle():
    wl, S, P0 = _wl(cfg_id=205, batch=2), 40, 10
    wl, gl, ow, kv, ok, ov, lens, x = _prefill_case(wl, S, P0, triangular_masking=False)
    y = gl.prefill(kv, x)
    torch.cuda.synchronize()
    desc = oracle.Desc(wl.hidden, wl.heads, wl.head_dim, wl.ffn, triangular_masking=False)
    yo = oracle.layer_forward(desc, ow, ok, ov, lens, x.double().cpu().numpy())
    assert rel_l2(y.double().cpu().numpy(), yo) <= TOL["f16"]


def test_prefill_mfma_is_causal_bitwise():
    wl, S, P0 = _wl(cfg_id=206, batch=1), 96, 0
    wl, gl, ow, kv, ok, ov, lens, x = _prefill_case(wl, S, P0)
    y1 = gl.prefill(kv, x).clone()
    tp = 70
    x2 = x.clone()
    x2[:, tp] = -x2[:, tp] + 0.5
    kv2, _, _, _ = filled_caches(wl, 0, gl, past=P0, cap=kv.capacity)
    y2 = gl.prefill(kv2, x2)
    torch.cuda.synchronize()
    assert torch.equal(y1[:, :tp], y2[:, :tp])
    assert not torch.equal(y1[:, tp:], y2[:, tp:])


def test_prefill_then_decode_matches_longer_prefill():
    """prefill(S) then decode of row S equals the last row of prefill(S+1) (GPU both ways)."""
    wl, S, P0 = _wl(cfg_id=207, batch=2), 40, 0
    wl, gl, ow, kv, ok, ov, lens, x = _prefill_case(wl, S + 1, P0)
    y_full = gl.prefill(kv, x)
    kv2, _, _, _ = filled_caches(wl, 0, gl, past=P0, cap=kv.capacity)
    gl.prefill(kv2, x[:, :S].contiguous())
    y_last = gl.decode(kv2, x[:, S].contiguous())
    torch.cuda.synchronize()
    assert rel_l2(y_last.double().cpu().numpy(), y_full[:, S].double().cpu().numpy()) <= TOL["f16"]


def test_large_batch_decode_uses_mfma_path_and_matches_oracle():
    """A decode step of 24 sequences (24 rows) takes the MFMA path; check it against the oracle."""
    wl = _wl(cfg_id=208, batch=24, hidden=320, heads=5, head_dim=64, ffn=640, past=77)
    gl, ow = gpu_layer_and_oracle_weights(wl, 0)
    kv, ok, ov, lens = filled_caches(wl, 0, gl, past=77, cap=128)
    x = syn.normal((wl.batch, wl.hidden), 1.0, wl.cfg_id, syn.X_LAYER, 0, "cuda").to(torch.float16)
    y = gl.decode(kv, x)
    torch.cuda.synchronize()
    desc = oracle.Desc(wl.hidden, wl.heads, wl.head_dim, wl.ffn)
    yo = oracle.layer_forward(desc, ow, ok, ov, lens, x.double().cpu().numpy()[:, None, :])[:, 0]
    assert rel_l2(y.double().cpu().numpy(), yo) <= TOL["f16"]


# bf16 weights and activations on the same kernels (the 16-bit type is a template parameter of the
# LayerNorm, GEMM and attention kernels): ragged tiles, head_dim 64 and 128, past rows, K = 2048
BF16 = dict(weight_dtype="bf16", act_dtype="bf16")
BF16_CASES = {
    "bf16-d128-b2-s100-affine-tanh": (_wl(cfg_id=241, **BF16, **AFFINE), 100, 0, True),
    "bf16-d64-b3-s70-p33-affine": (_wl(hidden=320, heads=5, head_dim=64, ffn=640, batch=3, cfg_id=242, **BF16,
                                       **AFFINE), 70, 33, False),
    "bf16-d128-b2-s256": (_wl(hidden=512, heads=4, ffn=2048, cfg_id=243, **BF16), 256, 0, False),
}


@pytest.mark.parametrize("cfg", [None, 0, 1, 2])
@pytest.mark.parametrize("name", list(BF16_CASES))
def test_prefill_mfma_bf16_matches_oracle(name, cfg, monkeypatch):
    """bf16 prefill on matrix cores (automatic tile choice, then each configuration forced) against
    the oracle, within the bf16 tolerance."""
    if cfg is not None:
        monkeypatch.setenv("DS_GEMM_CONFIG", str(cfg))
    wl, S, P0, tanh = BF16_CASES[name]
    _check_prefill(f"{name} config {cfg}", wl, S, P0, tanh)


def test_bf16_many_rows_take_the_mfma_kernels():
    """A bf16 prefill of 2 x 40 rows runs the MFMA path's launches (separate LayerNorm launches,
    which the per-row path does not make) and matches the untimed step bit for bit."""
    wl, S, P0 = _wl(cfg_id=244, batch=2, **BF16), 40, 6
    wl, gl, ow, kv, ok, ov, lens, x = _prefill_case(wl, S, P0)
    y1 = gl.prefill(kv, x)
    kv2, _, _, _ = filled_caches(wl, 0, gl, past=P0, cap=kv.capacity)
    y2 = torch.empty_like(y1)
    timed = gl.time_kernels(kv2, x, y2)
    torch.cuda.synchronize()
    assert [p for p, _ in timed] == ["ln1", "qkv", "attn", "o", "ln2", "ff1", "ff2"]
    assert torch.equal(y1, y2) and torch.equal(kv.k, kv2.k) and torch.equal(kv.v, kv2.v)


# int8 weights (codes with fp16 group scales) above the skinny kernel's 16 rows: each matrix is
# dequantized into fp16 just before its MFMA product; groups of 64, 128 with 64 in the MLP, and 32
I8 = dict(weight_dtype="i8", act_dtype="f16")
I8_CASES = {
    "i8-g64-d128-b2-s100-affine": (_wl(group=64, cfg_id=251, **I8, **AFFINE), 100, 0, False),
    "i8-g128-mlp64-d64-b3-s70-p33-tanh": (_wl(hidden=512, heads=8, head_dim=64, ffn=1024, batch=3, group=128,
                                              group_mlp=64, cfg_id=252, **I8, **AFFINE), 70, 33, True),
    "i8-g32-d128-b1-s17-p5": (_wl(batch=1, group=32, cfg_id=253, **I8), 17, 5, False),
}


@pytest.mark.parametrize("name", list(I8_CASES))
def test_prefill_mfma_int8_weights_matches_oracle(name):
    wl, S, P0, tanh = I8_CASES[name]
    _check_prefill(name, wl, S, P0, tanh)


def test_int8_prefill_takes_the_mfma_kernels():
    """An int8 prefill of 2 x 40 rows runs the MFMA path's launches (separate LayerNorm launches,
    which the per-row path does not make) and matches the untimed step bit for bit."""
    wl, S, P0 = _wl(cfg_id=254, batch=2, group=64, **I8), 40, 6
    wl, gl, ow, kv, ok, ov, lens, x = _prefill_case(wl, S, P0)
    y1 = gl.prefill(kv, x)
    kv2, _, _, _ = filled_caches(wl, 0, gl, past=P0, cap=kv.capacity)
    y2 = torch.empty_like(y1)
    timed = gl.time_kernels(kv2, x, y2)
    torch.cuda.synchronize()
    assert [p for p, _ in timed] == ["ln1", "qkv", "attn", "o", "ln2", "ff1", "ff2"]
    assert torch.equal(y1, y2) and torch.equal(kv.k, kv2.k) and torch.equal(kv.v, kv2.v)
