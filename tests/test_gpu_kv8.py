"""The int8 KV cache (kv_dtype DS_I8: int8 codes with one fp16 scale per cached row of one head)
against the oracle's kv_int8 reading, on the per-layer decode and prefill paths.

Appended rows come from fp16/bf16 values both sides see exactly, so their codes and scales are
compared bit for bit with the oracle's row quantizer. The rows a step writes come from the step's
own K/V projection (fp32 on the GPU, double in the oracle): a code may differ by one where the
quantizer's rounding is a near tie, so those rows are compared as dequantized values.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
import transformer_gpt_layer_amd as tg
from tests._common import TOL, TORCH, gpu_layer_and_oracle_weights, kv8_caches, rel_l2

pytestmark = pytest.mark.gpu


def _wl(**kw):
    return dataclasses.replace(syn.WORKLOADS["c1"], **kw)


CASES = {
    "f16-d128-b1": _wl(hidden=256, heads=2, head_dim=128, ffn=768, weight_dtype="f16", act_dtype="f16", batch=1,
                       past=70, cfg_id=601),
    "f16-d64-b3-affine": _wl(hidden=512, heads=8, head_dim=64, ffn=1024, weight_dtype="f16", act_dtype="f16", batch=3,
                             past=129, cfg_id=602, ln_std=0.2, bias_std=0.1),
    "i8w-d128-b9": _wl(hidden=512, heads=4, head_dim=128, ffn=1024, weight_dtype="i8", act_dtype="f16", group=64,
                       batch=9, past=300, cfg_id=603),
    "bf16-d128-b2-affine": _wl(hidden=512, heads=4, head_dim=128, ffn=2048, weight_dtype="bf16", act_dtype="bf16",
                               batch=2, past=45, cfg_id=604, ln_std=0.2, bias_std=0.1),
    # wide enough that the few-row products split K over workgroups and that attention takes
    # 256-position chunks (15 rows x 32 heads)
    "f16-d64-b15-h2048": _wl(hidden=2048, heads=32, head_dim=64, ffn=4096, weight_dtype="f16", act_dtype="f16",
                             batch=15, past=300, cfg_id=605),
}


@pytest.mark.parametrize("name", list(CASES))
def test_decode_with_int8_kv_matches_oracle(name):
    wl = CASES[name]
    tanh = "affine" in name
    print(f"[kv8 decode] {name}: {wl}", flush=True)
    gl, ow = gpu_layer_and_oracle_weights(wl, 0, gelu_tanh=tanh, kv_dtype="int8")
    kv, ok, ov, lens = kv8_caches(wl, 0, gl)
    desc = oracle.Desc(wl.hidden, wl.heads, wl.head_dim, wl.ffn, gelu_tanh=tanh, kv_int8=True)
    act = TORCH[wl.act_dtype]
    for step in range(2):
        x = syn.normal((wl.batch, wl.hidden), 1.0, wl.cfg_id, syn.X_LAYER, step, "cuda").to(act)
        y = gl.decode(kv, x)
        torch.cuda.synchronize()
        xd = x.double().cpu().numpy()
        P = int(lens[0])
        yo = oracle.layer_forward(desc, ow, ok, ov, lens, xd[:, None])[:, 0]
        yd = y.double().cpu().numpy()
        err, err_d = rel_l2(yd, yo), rel_l2(yd - xd, yo - xd)
        kd, vd = kv.dequantized()
        ek = rel_l2(kd[:, :, P].double().cpu().numpy(), ok[:, :, P])
        ev = rel_l2(vd[:, :, P].double().cpu().numpy(), ov[:, :, P])
        print(f"  step {step}: rel L2 {err:.3e}, of y - x {err_d:.3e}; new rows K {ek:.3e} V {ev:.3e}", flush=True)
        tol = TOL[wl.act_dtype]
        assert err <= tol and err_d <= tol and ek <= tol and ev <= tol
        # the new rows are int8 codes with one scale per row: max |code| is 127 where amax > 0
        codes = kv.k[:, :, P].cpu().numpy().astype(int)
        assert np.all(np.abs(codes).max(-1) == 127)
        assert kv.lengths() == [P + 1] * wl.batch


@pytest.mark.parametrize("name", ["f16-d64-b3-affine", "bf16-d128-b2-affine", "i8w-d128-b9"])
def test_int8_kv_decode_takes_the_skinny_mfma_path(name):
    """Decode with an int8 cache and at most 15 rows runs the skinny MFMA launches (with their own
    LayerNorm launches; the new k and v rows are quantized inside the QKV part), with the same
    outputs and cache bytes as the untimed step."""
    wl = CASES[name]
    gl, _ = gpu_layer_and_oracle_weights(wl, 0, gelu_tanh="affine" in name, kv_dtype="int8")
    kv1, *_ = kv8_caches(wl, 0, gl)
    kv2, *_ = kv8_caches(wl, 0, gl)
    x = syn.normal((wl.batch, wl.hidden), 1.0, wl.cfg_id, syn.X_LAYER, 0, "cuda").to(TORCH[wl.act_dtype])
    y1 = gl.decode(kv1, x)
    y2 = torch.empty_like(y1)
    timed = gl.time_kernels(kv2, x, y2)
    torch.cuda.synchronize()
    assert [p for p, _ in timed] == ["ln1", "qkv", "attn", "o", "ln2", "ff1", "ff2"]
    assert torch.equal(y1, y2) and torch.equal(kv1.k, kv2.k) and torch.equal(kv1.v, kv2.v)
    assert kv1.lengths() == kv2.lengths()


# few rows (the skinny products and the flash attention) and 16 or more (the MFMA GEMMs): the
# attention dequantizes the int8 K and V rows while staging them; several 64-key tiles, both
# head widths, fp16 and bf16
@pytest.mark.parametrize("name,S,P0", [("f16-d128-b1", 6, 5), ("f16-d64-b3-affine", 4, 0),
                                       ("f16-d64-b3-affine", 40, 7), ("f16-d128-b1", 70, 0),
                                       ("bf16-d128-b2-affine", 30, 9)])
def test_prefill_with_int8_kv_matches_oracle(name, S, P0):
    wl = CASES[name]
    gl, ow = gpu_layer_and_oracle_weights(wl, 0, gelu_tanh="affine" in name, kv_dtype="int8")
    kv, ok, ov, lens = kv8_caches(wl, 0, gl, past=P0, cap=(P0 + S + 63) // 64 * 64)
    x = syn.normal((wl.batch, S, wl.hidden), 1.0, wl.cfg_id, syn.X_LAYER, 7, "cuda").to(TORCH[wl.act_dtype])
    y = gl.prefill(kv, x)
    torch.cuda.synchronize()
    desc = oracle.Desc(wl.hidden, wl.heads, wl.head_dim, wl.ffn, gelu_tanh="affine" in name, kv_int8=True)
    yo = oracle.layer_forward(desc, ow, ok, ov, lens, x.double().cpu().numpy())
    yd, xd = y.double().cpu().numpy(), x.double().cpu().numpy()
    err, err_d = rel_l2(yd, yo), rel_l2(yd - xd, yo - xd)
    kd, vd = kv.dequantized()
    ek = rel_l2(kd[:, :, :P0 + S].double().cpu().numpy(), ok[:, :, :P0 + S])
    ev = rel_l2(vd[:, :, :P0 + S].double().cpu().numpy(), ov[:, :, :P0 + S])
    print(f"  prefill {name} S={S} P0={P0}: rel L2 {err:.3e}, of y - x {err_d:.3e}, cache K {ek:.3e} V {ev:.3e}",
          flush=True)
    tol = TOL[wl.act_dtype]
    assert err <= tol and err_d <= tol and ek <= tol and ev <= tol
    assert kv.lengths() == [P0 + S] * wl.batch


def test_int8_kv_scale_pointers_are_checked():
    wl = CASES["f16-d128-b1"]
    gl, _ = gpu_layer_and_oracle_weights(wl, 0, kv_dtype="int8")
    kv = tg.KVCache(1, wl.heads, 64, wl.head_dim, torch.int8, "cuda")
    kv.k_scale = None
    with pytest.raises(ValueError, match="k_scale"):
        gl.decode(kv, torch.zeros((1, wl.hidden), dtype=torch.float16, device="cuda"))
    gl16, _ = gpu_layer_and_oracle_weights(wl, 0)
    kv8 = tg.KVCache(1, wl.heads, 64, wl.head_dim, torch.int8, "cuda")
    with pytest.raises(ValueError, match="not int8"):
        gl16.decode(kv8, torch.zeros((1, wl.hidden), dtype=torch.float16, device="cuda"))
