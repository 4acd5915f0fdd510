"""Seeded synthetic inputs and the workload shapes.

This module draws random numbers and names shapes; it holds none of the layer's arithmetic. Both
the oracle side (tests, CPU baseline) and the GPU side (tests, benchmark, smoke check) take their
inputs from here.

Recipe (the pages' workloads are trained GPT-2 / GPT-Neo / Turing-NLG / GPT-3-like models whose
weights are not available; seeded draws of the same shapes stand in for them):
  weights ~ N(0, 0.02), biases ~ N(0, bias_std) (0.01 by default), LayerNorm gamma = 1 and
  beta = 0 by default, activations x ~ N(0, 1), past K/V cache rows ~ N(0, 1).
Parity cases that must see the LayerNorm affine map set ln_std > 0: gamma ~ 1 + N(0, ln_std) and
beta ~ N(0, ln_std), drawn per layer (the seed includes the layer), so that a kernel which ignores
gamma/beta, or reads another layer's or the other LayerNorm's, gives a visibly different result.
Draws are float32 from torch's generator on the requested device, seeded from
(config id, layer, tensor id) through numpy's SeedSequence; the caller rounds them to the
target dtype (round to nearest even). A given key always yields the same tensor on a given
device type; CPU and GPU generators yield different (equally distributed) streams, so a parity
test draws once and hands the same values to both sides.
"""
from dataclasses import dataclass, field

import numpy as np
import torch

# tensor ids
LN1_G, LN1_B, W_QKV, B_QKV, W_O, B_O, LN2_G, LN2_B, W_FF1, B_FF1, W_FF2, B_FF2, K_PAST, V_PAST = range(14)
LNF_G, LNF_B, W_VOCAB = 14, 15, 16
X_LAYER = 65535     # layer slot used for the stack input x
HEAD_LAYER = 65534  # layer slot of the final LayerNorm and the LM head
GPT_NEO_VOCAB = 50257  # the GPT-2 BPE vocabulary of the GPT-Neo-2.7B example

WEIGHT_NAMES = ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_o", "b_o",
                "ln2_g", "ln2_b", "w_ff1", "b_ff1", "w_ff2", "b_ff2")


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    hidden: int
    heads: int
    head_dim: int
    ffn: int
    layers: int
    weight_dtype: str  # "f32" | "f16" | "i8" | "bf16"
    act_dtype: str     # "f32" | "f16" | "bf16"
    batch: int
    past: int          # filled cache rows before the step (decode) or P0 (prefill)
    seq: int = 1       # new rows per sequence: 1 for decode, S for prefill
    group: int = 0     # int8 group size along the reduction dimension
    group_mlp: int = 0  # int8 group size of the MLP matrices (0: group)
    ln_std: float = 0.0     # > 0: LayerNorm gamma ~ 1 + N(0, ln_std), beta ~ N(0, ln_std)
    bias_std: float = 0.01  # biases ~ N(0, bias_std)
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def capacity(self) -> int:
        # room for the past rows, this step's rows, and a little headroom, rounded to 64 rows
        need = self.past + self.seq + 1
        return (need + 63) // 64 * 64


WORKLOADS = {
    # one pre-LN layer, fp32, tiny: the parity case
    "c1": Workload("c1-fp32-h256", 1, 256, 4, 64, 1024, 1, "f32", "f32", 1, 32),
    # GPT-Neo-2.7B-shaped stack, fp16, batch-1 decode against 512 past rows
    "c2": Workload("c2-gptneo2.7b-f16-b1-p512", 2, 2560, 20, 128, 10240, 32, "f16", "f16", 1, 512),
    # 13B-shaped stack, fp16, batch-8 decode against 1024 past rows
    "c3": Workload("c3-13b-f16-b8-p1024", 3, 5120, 40, 128, 20480, 40, "f16", "f16", 8, 1024),
    # 13B shapes, int8 weights (group 64, fp16 scales), fp16 activations, batch 1 and 8
    "c4b1": Workload("c4-13b-i8g64-b1-p1024", 4, 5120, 40, 128, 20480, 40, "i8", "f16", 1, 1024, group=64),
    "c4b8": Workload("c4-13b-i8g64-b8-p1024", 4, 5120, 40, 128, 20480, 40, "i8", "f16", 8, 1024, group=64),
    # mlp_extra_grouping: twice the groups (size 32) in the two MLP matrices
    "c4b1m32": Workload("c4-13b-i8g64-mlp32-b1-p1024", 8, 5120, 40, 128, 20480, 40, "i8", "f16", 1, 1024, group=64,
                        group_mlp=32),
    # prefill on the GPT-Neo-2.7B shapes: batch 4 x 512 prompt rows, causal
    "c5": Workload("c5-gptneo2.7b-f16-prefill-b4s512", 5, 2560, 20, 128, 10240, 32, "f16", "f16", 4, 0, seq=512),
    # the C2 decode step in the other precisions the config table names: bf16 weights and
    # activations, and fp16 with an int8 KV cache (one int8 row and fp16 scale per cached head row)
    "c2bf16": Workload("c2-gptneo2.7b-bf16-b1-p512", 6, 2560, 20, 128, 10240, 32, "bf16", "bf16", 1, 512),
    "c2kv8": Workload("c2-gptneo2.7b-f16-kv8-b1-p512", 7, 2560, 20, 128, 10240, 32, "f16", "f16", 1, 512,
                      extra={"kv_dtype": "int8"}),
    # the C5 prefill in bf16 weights and activations, with an int8 KV cache, and with int8 weights
    "c5bf16": Workload("c5-gptneo2.7b-bf16-prefill-b4s512", 9, 2560, 20, 128, 10240, 32, "bf16", "bf16", 4, 0,
                       seq=512),
    "c5kv8": Workload("c5-gptneo2.7b-f16-kv8-prefill-b4s512", 10, 2560, 20, 128, 10240, 32, "f16", "f16", 4, 0,
                      seq=512, extra={"kv_dtype": "int8"}),
    "c5i8": Workload("c5-gptneo2.7b-i8g64-prefill-b4s512", 11, 2560, 20, 128, 10240, 32, "i8", "f16", 4, 0,
                     seq=512, group=64),
}


def seed_of(cfg_id: int, layer: int, tensor_id: int) -> int:
    ss = np.random.SeedSequence([cfg_id, layer, tensor_id])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def normal(shape, std: float, cfg_id: int, layer: int, tensor_id: int, device="cpu") -> torch.Tensor:
    """float32 N(0, std^2) draws of the given shape, seeded by (cfg_id, layer, tensor_id)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(cfg_id, layer, tensor_id))
    t = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    return t.mul_(std) if std != 1.0 else t


def layer_weights_f32(wl: Workload, layer: int, device="cpu") -> dict:
    """The twelve float32 parameter tensors of one layer (weights [N,K] row-major)."""
    H, F, c, bs = wl.hidden, wl.ffn, wl.cfg_id, wl.bias_std

    def gamma(tid):
        if wl.ln_std <= 0:
            return torch.ones(H, device=device)
        return normal((H,), wl.ln_std, c, layer, tid, device).add_(1.0)

    def beta(tid):
        if wl.ln_std <= 0:
            return torch.zeros(H, device=device)
        return normal((H,), wl.ln_std, c, layer, tid, device)

    return {
        "ln1_g": gamma(LN1_G), "ln1_b": beta(LN1_B),
        "w_qkv": normal((3 * H, H), 0.02, c, layer, W_QKV, device),
        "b_qkv": normal((3 * H,), bs, c, layer, B_QKV, device),
        "w_o": normal((H, H), 0.02, c, layer, W_O, device),
        "b_o": normal((H,), bs, c, layer, B_O, device),
        "ln2_g": gamma(LN2_G), "ln2_b": beta(LN2_B),
        "w_ff1": normal((F, H), 0.02, c, layer, W_FF1, device),
        "b_ff1": normal((F,), bs, c, layer, B_FF1, device),
        "w_ff2": normal((H, F), 0.02, c, layer, W_FF2, device),
        "b_ff2": normal((H,), bs, c, layer, B_FF2, device),
    }


def past_kv_f32(wl: Workload, layer: int, device="cpu"):
    """float32 [B, heads, past, head_dim] draws for the filled cache rows (K and V)."""
    shape = (wl.batch, wl.heads, wl.past, wl.head_dim)
    return (normal(shape, 1.0, wl.cfg_id, layer, K_PAST, device),
            normal(shape, 1.0, wl.cfg_id, layer, V_PAST, device))


def stack_input_f32(wl: Workload, device="cpu", step: int = 0) -> torch.Tensor:
    """float32 [B, T, H] N(0,1) input rows of the stack."""
    return normal((wl.batch, wl.seq, wl.hidden), 1.0, wl.cfg_id, X_LAYER, step, device)


def lm_head_f32(wl: Workload, vocab: int, device="cpu") -> dict:
    """float32 final LayerNorm (gamma, beta as for the layers of this workload) and LM head weight
    [vocab, hidden] ~ N(0, 0.02)."""
    H, c = wl.hidden, wl.cfg_id
    if wl.ln_std > 0:
        g = normal((H,), wl.ln_std, c, HEAD_LAYER, LNF_G, device).add_(1.0)
        b = normal((H,), wl.ln_std, c, HEAD_LAYER, LNF_B, device)
    else:
        g, b = torch.ones(H, device=device), torch.zeros(H, device=device)
    return {"ln_g": g, "ln_b": b, "w": normal((vocab, H), 0.02, c, HEAD_LAYER, W_VOCAB, device)}


# ---------------------------------------------------------------- the MoE expert FF
# tensor ids of the MoE block (layer slot = the block's index)
MOE_LN_G, MOE_LN_B, W_GATE, W_EXP1, B_EXP1, W_EXP2, B_EXP2, W_RES1, B_RES1, W_RES2, B_RES2, X2_IN = range(20, 32)


@dataclass(frozen=True)
class MoeWorkload:
    """One MoE expert-FF block ("DeepSpeed MoE 大规模稀疏模型推理实战指南": experts per MoE layer,
    types standard / residual). Gate weights ~ N(0, gate_std^2), gate_std = 1/sqrt(hidden) by
    default so that the gate logits of a LayerNorm-ed row are about N(0, 1); expert and residual
    weights ~ N(0, 0.02), biases ~ N(0, bias_std); x2 ~ N(0, 1)."""
    name: str
    cfg_id: int
    hidden: int
    ffn: int
    experts: int
    top_k: int
    tokens: int
    weight_dtype: str   # "f32" | "f16" | "i8" | "bf16"
    act_dtype: str      # "f32" | "f16" | "bf16"
    group: int = 0
    residual: bool = False
    combine: int = 0
    ln_std: float = 0.0
    bias_std: float = 0.01
    gate_std: float = 0.0   # 0: 1/sqrt(hidden)


MOE_WORKLOADS = {
    # the MoE page's 52B model: a 1.3B dense backbone (24 layers, hidden 2048) with 128 experts per
    # MoE layer; expert FF width 4 x hidden (the GPT convention; the page gives no width); top-1
    "moe-1.3b-e128": MoeWorkload("moe-1.3b-e128-f16-top1-t8", 30, 2048, 8192, 128, 1, 8, "f16", "f16"),
    "moe-1.3b-e128-t1": MoeWorkload("moe-1.3b-e128-f16-top1-t1", 30, 2048, 8192, 128, 1, 1, "f16", "f16"),
}


def moe_weights_f32(mw: MoeWorkload, device="cpu", block: int = 0) -> dict:
    """float32 tensors of one MoE block: ln_g, ln_b [H], w_gate [E,H], w1 [E,F,H], b1 [E,F],
    w2 [E,H,F], b2 [E,H], and r_w1 [F,H], r_b1 [F], r_w2 [H,F], r_b2 [H] for the residual type."""
    H, F, E, c, bs = mw.hidden, mw.ffn, mw.experts, mw.cfg_id, mw.bias_std
    gs = mw.gate_std if mw.gate_std > 0 else 1.0 / float(np.sqrt(H))
    if mw.ln_std > 0:
        g = normal((H,), mw.ln_std, c, block, MOE_LN_G, device).add_(1.0)
        b = normal((H,), mw.ln_std, c, block, MOE_LN_B, device)
    else:
        g, b = torch.ones(H, device=device), torch.zeros(H, device=device)
    w = {"ln_g": g, "ln_b": b, "w_gate": normal((E, H), gs, c, block, W_GATE, device),
         "w1": normal((E, F, H), 0.02, c, block, W_EXP1, device), "b1": normal((E, F), bs, c, block, B_EXP1, device),
         "w2": normal((E, H, F), 0.02, c, block, W_EXP2, device), "b2": normal((E, H), bs, c, block, B_EXP2, device)}
    if mw.residual:
        w.update({"r_w1": normal((F, H), 0.02, c, block, W_RES1, device), "r_b1": normal((F,), bs, c, block, B_RES1, device),
                  "r_w2": normal((H, F), 0.02, c, block, W_RES2, device), "r_b2": normal((H,), bs, c, block, B_RES2, device)})
    return w


def moe_input_f32(mw: MoeWorkload, device="cpu", step: int = 0) -> torch.Tensor:
    """float32 [T, H] N(0, 1) rows of the residual stream entering the block."""
    return normal((mw.tokens, mw.hidden), 1.0, mw.cfg_id, X_LAYER, X2_IN + 64 * step, device)
