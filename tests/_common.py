"""Shared test plumbing: seeded inputs for both sides, GPU layer construction, error metrics.

The GPU side gets device tensors in its dtypes; the oracle gets exactly the same values widened
to float64. No expected value here comes from the GPU path.
"""
import numpy as np
import torch

import synthetic as syn

# relative L2 bars: fp32 configs, fp16-activation configs, bf16 configs
TOL = {"f32": 1e-4, "f16": 1e-2, "bf16": 4e-2}
TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def gpu_layer_and_oracle_weights(wl: syn.Workload, layer: int, device="cuda", check_quant=True, **cfg_kw):
    """Builds a library Layer for one layer of the workload and the oracle's float64 weights
    (same values). For int8 the GPU quantizer makes the codes, and the oracle quantizer makes its
    own from the same float32 draws; the two are compared bit for bit."""
    import oracle
    import transformer_gpt_layer_amd as tg

    w32 = syn.layer_weights_f32(wl, layer, device)
    act = TORCH[wl.act_dtype]
    i8 = wl.weight_dtype == "i8"
    cfg = tg.make_config(hidden=wl.hidden, heads=wl.heads, ffn=wl.ffn,
                         dtype={"f32": "fp32", "f16": "fp16", "i8": "int8", "bf16": "bf16"}[wl.weight_dtype],
                         quant_group=wl.group if i8 else None,
                         quant_group_mlp=wl.group_mlp if i8 and wl.group_mlp else None, **cfg_kw)
    gw, ow = {}, {}
    for name, t in w32.items():
        if name.startswith("w_"):
            if i8:
                G = wl.group_mlp if wl.group_mlp and name in ("w_ff1", "w_ff2") else wl.group
                q, s = tg.quantize_i8(t.contiguous(), G)
                gw[name], gw["s" + name[1:]] = q, s
                if check_quant:
                    oq, os_ = oracle.quantize_i8(t.cpu().numpy(), G)
                    assert np.array_equal(q.cpu().numpy(), oq), f"int8 codes of {name} differ from the oracle"
                    assert np.array_equal(s.cpu().view(torch.int16).numpy().view(np.uint16), os_), \
                        f"fp16 scales of {name} differ from the oracle"
                    ow[name] = oracle.dequantize_i8(oq, os_, G)
                else:
                    ow[name] = oracle.dequantize_i8(q.cpu().numpy(), s.cpu().view(torch.int16).numpy().view(np.uint16), G)
            else:
                gw[name] = t.to(act).contiguous()
                ow[name] = gw[name].double().cpu().numpy()
        else:
            gw[name] = t.to(act).contiguous()
            ow[name] = gw[name].double().cpu().numpy()
    return tg.Layer(cfg, gw), ow


def filled_caches(wl: syn.Workload, layer: int, gl, device="cuda", past=None, cap=None, batch=None):
    """A GPU KVCache holding `past` seeded rows (appended through ds_kv_append) and the oracle's
    float64 copy of the same values."""
    import transformer_gpt_layer_amd as tg

    B = wl.batch if batch is None else batch
    P = wl.past if past is None else past
    cap = wl.capacity if cap is None else cap
    act = TORCH[wl.act_dtype]
    kv = tg.KVCache(B, wl.heads, cap, wl.head_dim, act, device)
    ok = np.zeros((B, wl.heads, cap, wl.head_dim))
    ov = np.zeros_like(ok)
    if P > 0:
        kp = syn.normal((B, P, wl.hidden), 1.0, wl.cfg_id, layer, syn.K_PAST, device).to(act)
        vp = syn.normal((B, P, wl.hidden), 1.0, wl.cfg_id, layer, syn.V_PAST, device).to(act)
        gl.kv_append(kv, kp.contiguous(), vp.contiguous())
        kh = kp.double().cpu().numpy().reshape(B, P, wl.heads, wl.head_dim).transpose(0, 2, 1, 3)
        vh = vp.double().cpu().numpy().reshape(B, P, wl.heads, wl.head_dim).transpose(0, 2, 1, 3)
        ok[:, :, :P] = kh
        ov[:, :, :P] = vh
    lens = np.full(B, P, dtype=np.int32)
    return kv, ok, ov, lens


def kv8_caches(wl, layer, gl, past=None, cap=None, batch=None):
    """A GPU int8 KV cache holding `past` seeded rows (appended through ds_kv_append, which
    quantizes them) and the oracle's float64 cache of the dequantized rows; the GPU's codes and
    scales are checked bit for bit against the oracle's row quantizer on the same values."""
    import oracle
    import transformer_gpt_layer_amd as tg

    B = wl.batch if batch is None else batch
    P = wl.past if past is None else past
    cap = wl.capacity if cap is None else cap
    act = TORCH[wl.act_dtype]
    kv = tg.KVCache(B, wl.heads, cap, wl.head_dim, torch.int8, "cuda")
    ok = np.zeros((B, wl.heads, cap, wl.head_dim))
    ov = np.zeros_like(ok)
    if P > 0:
        kp = syn.normal((B, P, wl.hidden), 1.0, wl.cfg_id, layer, syn.K_PAST, "cuda").to(act)
        vp = syn.normal((B, P, wl.hidden), 1.0, wl.cfg_id, layer, syn.V_PAST, "cuda").to(act)
        gl.kv_append(kv, kp.contiguous(), vp.contiguous())
        torch.cuda.synchronize()
        for src, codes, scales, dst in ((kp, kv.k, kv.k_scale, ok), (vp, kv.v, kv.v_scale, ov)):
            rows = src.double().cpu().numpy().reshape(B, P, wl.heads, wl.head_dim).transpose(0, 2, 1, 3)
            q, s = oracle.quantize_rows_i8(rows)
            assert np.array_equal(codes[:, :, :P].cpu().numpy(), q), "appended int8 codes differ from the oracle"
            sb = scales[:, :, :P].cpu().view(torch.int16).numpy().view(np.uint16)
            assert np.array_equal(sb, s), "appended fp16 row scales differ from the oracle"
            dst[:, :, :P] = q.astype(np.float64) * oracle.fp16_to_double(s)[..., None]
    lens = np.full(B, P, dtype=np.int32)
    return kv, ok, ov, lens
