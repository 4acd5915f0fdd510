"""GPU parity of the HIP layer against the oracle (run on an MI355X).

Inputs are seeded synthetic draws (synthetic.py); both sides receive the same values. Sizes span
several tiles and ragged tails (batch not a multiple of the batch tile, past lengths not multiples
of the attention chunk, rows not multiples of the row tile).
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from tests._common import TOL, TORCH, filled_caches, gpu_layer_and_oracle_weights, rel_l2

pytestmark = pytest.mark.gpu


def _wl(base, **kw):
    return dataclasses.replace(syn.WORKLOADS[base] if isinstance(base, str) else base, **kw)


def _run_decode(wl, layer=0, past=None, batch=None, cap=None, gelu_tanh=False):
    gl, ow = gpu_layer_and_oracle_weights(wl, layer, gelu_tanh=gelu_tanh)
    B = wl.batch if batch is None else batch
    kv, ok, ov, lens = filled_caches(wl, layer, gl, past=past, batch=B, cap=cap)
    x = syn.normal((B, wl.hidden), 1.0, wl.cfg_id, syn.X_LAYER, layer).to(gl.cfg.torch_act_dtype)
    x = x.cuda() if not x.is_cuda else x
    y = gl.decode(kv, x)
    torch.cuda.synchronize()
    desc = oracle.Desc(wl.hidden, wl.heads, wl.head_dim, wl.ffn, gelu_tanh=gelu_tanh)
    yo = oracle.layer_forward(desc, ow, ok, ov, lens, x.double().cpu().numpy()[:, None, :])[:, 0]
    return gl, kv, x, y, yo, ok, ov, lens


SMALL = {
    "c1": _wl("c1"),
    "f32-d128-b3": _wl("c1", hidden=256, heads=2, head_dim=128, ffn=512, batch=3, past=37, cfg_id=101),
    "f16-d128-b3": _wl("c1", hidden=256, heads=2, head_dim=128, ffn=768, weight_dtype="f16", act_dtype="f16",
                       batch=3, past=70, cfg_id=102),
    "f16-d64-b9": _wl("c1", hidden=320, heads=5, head_dim=64, ffn=640, weight_dtype="f16", act_dtype="f16",
                      batch=9, past=129, cfg_id=103),
    "i8-d128-b5": _wl("c1", hidden=512, heads=4, head_dim=128, ffn=1024, weight_dtype="i8", act_dtype="f16",
                      group=64, batch=5, past=65, cfg_id=104),
    "i8-d64-b1-k256": _wl("c1", hidden=256, heads=4, head_dim=64, ffn=512, weight_dtype="i8", act_dtype="f16",
                          group=64, batch=1, past=3, cfg_id=105),
    # wide enough that the few-row products split K over workgroups (O by 4, FF2 by 8 for fp16)
    # and that attention takes 256-position chunks (15 rows x 32 heads)
    "f16-d64-b15-h2048": _wl("c1", hidden=2048, heads=32, head_dim=64, ffn=4096, weight_dtype="f16", act_dtype="f16",
                             batch=15, past=300, cfg_id=106),
    "i8-d64-b15-h2048": _wl("c1", hidden=2048, heads=32, head_dim=64, ffn=8192, weight_dtype="i8", act_dtype="f16",
                            group=64, batch=15, past=301, cfg_id=107),
    # bf16 weights and activations (the skinny MFMA path with bf16 operands below 16 rows), one case
    # wide enough to split K over workgroups and to take 256-position attention chunks
    "bf16-d128-b3": _wl("c1", hidden=256, heads=2, head_dim=128, ffn=768, weight_dtype="bf16", act_dtype="bf16",
                        batch=3, past=70, cfg_id=140),
    "bf16-d64-b9": _wl("c1", hidden=320, heads=5, head_dim=64, ffn=640, weight_dtype="bf16", act_dtype="bf16",
                       batch=9, past=129, cfg_id=141),
    "bf16-d64-b15-h2048": _wl("c1", hidden=2048, heads=32, head_dim=64, ffn=4096, weight_dtype="bf16",
                              act_dtype="bf16", batch=15, past=300, cfg_id=144),
}

# Per-layer LayerNorm gamma ~ 1 + N(0, 0.2), beta ~ N(0, 0.2) and biases ~ N(0, 0.1), on every
# decode path (fp32 GEMV, fp16 and int8 skinny MFMA with one and with several activation rows),
# with the erf and the tanh GeLU: a kernel that drops or swaps an affine vector or a bias, or uses
# the other GeLU form, moves y - x far past the bar.
AFFINE = dict(ln_std=0.2, bias_std=0.1)
CASES = {name: (wl, False) for name, wl in SMALL.items()}
CASES.update({
    "f32-affine": (_wl(SMALL["c1"], cfg_id=121, **AFFINE), False),
    "f32-affine-tanh": (_wl(SMALL["f32-d128-b3"], cfg_id=122, **AFFINE), True),
    "f16-affine-b3": (_wl(SMALL["f16-d128-b3"], cfg_id=123, **AFFINE), False),
    "f16-affine-tanh-b9": (_wl(SMALL["f16-d64-b9"], cfg_id=124, **AFFINE), True),
    "f16-affine-tanh-b1": (_wl(SMALL["f16-d128-b3"], batch=1, cfg_id=125, **AFFINE), True),
    "i8-affine-tanh-b5": (_wl(SMALL["i8-d128-b5"], cfg_id=126, **AFFINE), True),
    "i8-affine-b1": (_wl(SMALL["i8-d64-b1-k256"], cfg_id=127, **AFFINE), False),
    "i8-affine-tanh-b15": (_wl(SMALL["i8-d64-b15-h2048"], cfg_id=128, **AFFINE), True),
    # finer int8 groups (mlp_extra_grouping halves the MLP group; other group sizes): the per-row
    # GEMV path with a scale group per matrix, at one and at several activation rows
    "i8-g64-mlp32-b1": (_wl(SMALL["i8-d128-b5"], group_mlp=32, batch=1, cfg_id=129, **AFFINE), False),
    "i8-g32-b8": (_wl(SMALL["i8-d128-b5"], group=32, ffn=1536, batch=8, cfg_id=130, **AFFINE), True),
    "i8-g128-mlp64-b3": (_wl("c1", hidden=1024, heads=8, head_dim=128, ffn=2048, weight_dtype="i8", act_dtype="f16",
                             group=128, group_mlp=64, batch=3, past=40, cfg_id=131, **AFFINE), False),
    "bf16-affine-tanh-b1": (_wl(SMALL["bf16-d128-b3"], batch=1, cfg_id=142, **AFFINE), True),
    "bf16-affine-b4-h1024": (_wl("c1", hidden=1024, heads=8, head_dim=128, ffn=4096, weight_dtype="bf16",
                                 act_dtype="bf16", batch=4, past=300, cfg_id=143, **AFFINE), False),
    "i8-g16-mlp48-b2": (_wl("c1", hidden=768, heads=12, head_dim=64, ffn=1536, weight_dtype="i8", act_dtype="f16",
                            group=16, group_mlp=48, batch=2, past=21, cfg_id=132, **AFFINE), True),
})


@pytest.mark.parametrize("name", list(CASES))
def test_decode_matches_oracle(name):
    wl, tanh = CASES[name]
    print(f"[decode parity] {name}: {wl} gelu_tanh={tanh}", flush=True)
    gl, kv, x, y, yo, ok, ov, lens = _run_decode(wl, gelu_tanh=tanh)
    err = rel_l2(y.double().cpu().numpy(), yo)
    print(f"  rel L2 = {err:.3e}", flush=True)
    assert err <= TOL[wl.act_dtype], err
    # the layer's own contribution (y - x) is the stricter view: the residual stream hides errors
    xd = x.double().cpu().numpy()
    err_d = rel_l2(y.double().cpu().numpy() - xd, yo - xd)
    print(f"  rel L2 of y - x = {err_d:.3e}", flush=True)
    assert err_d <= TOL[wl.act_dtype], err_d
    # the new K/V rows landed at row `past` of every head, and the lengths advanced
    P = wl.past
    kg = kv.k.double().cpu().numpy()
    vg = kv.v.double().cpu().numpy()
    assert rel_l2(kg[:, :, P], ok[:, :, P]) <= TOL[wl.act_dtype]
    assert rel_l2(vg[:, :, P], ov[:, :, P]) <= TOL[wl.act_dtype]
    assert np.array_equal(kg[:, :, :P], ok[:, :, :P]) and np.array_equal(vg[:, :, :P], ov[:, :, :P])
    assert not kg[:, :, P + 1:].any()
    assert kv.lengths() == [P + 1] * wl.batch and list(kv.h_len) == [P + 1] * wl.batch


def test_decode_single_key_cache():
    # P = 0: every head attends to its own new key only
    wl = _wl(SMALL["f16-d128-b3"], past=0, cfg_id=110)
    gl, kv, x, y, yo, *_ = _run_decode(wl)
    assert rel_l2(y.double().cpu().numpy(), yo) <= TOL["f16"]


def single_key_layer(wl, layer=0):
    """A layer whose step reduces to y = x + ctx when the cache is empty: W_o = I, W_ff1 = W_ff2 = 0
    and zero biases (W_qkv and the LayerNorm vectors stay seeded draws). With one key the softmax
    weight is exactly 1, so ctx is the new value row itself, and every later step adds exact zeros
    or multiplies by exactly one."""
    import transformer_gpt_layer_amd as tg
    act = TORCH[wl.act_dtype]
    w = {k: v.to(act).contiguous() for k, v in syn.layer_weights_f32(wl, layer, "cuda").items()}
    H, F = wl.hidden, wl.ffn
    w["w_o"] = torch.eye(H, dtype=act, device="cuda")
    w["w_ff1"] = torch.zeros((F, H), dtype=act, device="cuda")
    w["w_ff2"] = torch.zeros((H, F), dtype=act, device="cuda")
    for n in ("b_qkv", "b_o", "b_ff1", "b_ff2"):
        w[n] = torch.zeros_like(w[n])
    cfg = tg.make_config(hidden=H, heads=wl.heads, ffn=F, dtype={"f32": "fp32", "f16": "fp16"}[wl.weight_dtype])
    return tg.Layer(cfg, w)


@pytest.mark.parametrize("name", ["c1", "f16-d128-b3", "f16-d64-b9", "f16-d64-b15-h2048"])
def test_decode_single_key_is_exactly_the_value_row(name):
    """P = 0 with W_o = I and a zero MLP: y = x + v exactly (in the activation type), v being the
    value row the step wrote into the cache."""
    wl = _wl(SMALL[name], past=0, ln_std=0.2)
    gl = single_key_layer(wl)
    act = TORCH[wl.act_dtype]
    kv = __import__("transformer_gpt_layer_amd").KVCache(wl.batch, wl.heads, 64, wl.head_dim, act, "cuda")
    x = syn.normal((wl.batch, wl.hidden), 1.0, wl.cfg_id, syn.X_LAYER, 5, "cuda").to(act)
    y = gl.decode(kv, x)
    torch.cuda.synchronize()
    v = kv.v[:, :, 0].reshape(wl.batch, wl.hidden)       # heads concatenated
    want = (x.float() + v.float()).to(act)
    assert torch.count_nonzero(v) > 0
    assert torch.equal(y, want), (y.float() - want.float()).abs().max().item()
    assert kv.lengths() == [1] * wl.batch


def test_decode_batch_independent_and_deterministic():
    wl = SMALL["f16-d64-b9"]
    gl, ow = gpu_layer_and_oracle_weights(wl, 0)
    x = syn.normal((wl.batch, wl.hidden), 1.0, wl.cfg_id, syn.X_LAYER, 0, "cuda").half()
    kv, *_ = filled_caches(wl, 0, gl)
    y = gl.decode(kv, x)
    kv2, *_ = filled_caches(wl, 0, gl)
    y2 = gl.decode(kv2, x)
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "run-to-run results differ"
    for b in (0, 4, 8):
        kv1, *_ = filled_caches(wl, 0, gl, batch=1)
        # sequence b's past rows are the draws of batch row b
        kv1.k.copy_(kv.k[b:b + 1]); kv1.v.copy_(kv.v[b:b + 1])
        kv1.set_lengths([wl.past])
        y1 = gl.decode(kv1, x[b:b + 1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(y1[0], y[b]), f"sequence {b} depends on the rest of the batch"


def test_decode_sequence_of_steps_tracks_oracle():
    # four consecutive decode steps on one cache, each checked against the oracle
    wl = SMALL["f16-d128-b3"]
    gl, ow = gpu_layer_and_oracle_weights(wl, 0)
    kv, ok, ov, lens = filled_caches(wl, 0, gl)
    desc = oracle.Desc(wl.hidden, wl.heads, wl.head_dim, wl.ffn)
    for step in range(4):
        x = syn.normal((wl.batch, wl.hidden), 1.0, wl.cfg_id, syn.X_LAYER, 10 + step, "cuda").half()
        y = gl.decode(kv, x)
        yo = oracle.layer_forward(desc, ow, ok, ov, lens, x.double().cpu().numpy()[:, None])[:, 0]
        assert rel_l2(y.double().cpu().numpy(), yo) <= TOL["f16"], step
    assert kv.lengths() == list(lens)


def test_quantizer_and_dequant_bit_exact():
    import transformer_gpt_layer_amd as tg
    w = syn.normal((300, 1024), 0.02, 7, 0, 0, "cuda")
    w[5, 64:128] = 0.0
    w[9, 3] = 1.5
    q, s = tg.quantize_i8(w, 64)
    oq, os_ = oracle.quantize_i8(w.cpu().numpy(), 64)
    assert np.array_equal(q.cpu().numpy(), oq)
    assert np.array_equal(s.cpu().view(torch.int16).numpy().view(np.uint16), os_)
    deq = tg.dequantize_i8(q, s, 64).cpu().numpy()
    ref = oracle.dequantize_i8(oq, os_, 64).astype(np.float32)   # q*s is exact in float32
    assert np.array_equal(deq.view(np.uint32), ref.view(np.uint32))


def test_kv_full_raises_before_launch():
    wl = SMALL["f16-d128-b3"]
    gl, _ = gpu_layer_and_oracle_weights(wl, 0)
    kv, *_ = filled_caches(wl, 0, gl, past=wl.capacity - 1)
    x = torch.zeros((wl.batch, wl.hidden), dtype=torch.float16, device="cuda")
    gl.decode(kv, x)  # fills the last row
    with pytest.raises(OverflowError):
        gl.decode(kv, x)
    assert kv.lengths() == [wl.capacity] * wl.batch


def test_read_probe_reads_every_word():
    """The bandwidth probe's digest is the XOR of every 32-bit word of the buffer: two full passes
    of its grid (2048 workgroups x 2048 16-byte pieces), then five whole workgroup spans and a
    ragged tail of 3 x 256 + 37 pieces."""
    import transformer_gpt_layer_amd as tg
    g = torch.Generator().manual_seed(11)
    words = 4 * (2 * 2048 * 2048 + 5 * 2048 + 3 * 256 + 37)
    host = torch.randint(-2**31, 2**31 - 1, (words,), dtype=torch.int32, generator=g)
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    tg.read_probe(host.cuda(), out)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert int(out.cpu().numpy().view(np.uint32)[0]) == int(want)


@pytest.mark.parametrize("name,S,P0,tanh", [("f16-d128-b3", 7, 5, False), ("f32-d128-b3", 5, 0, False),
                                             ("i8-d128-b5", 4, 9, False), ("f16-affine-b3", 5, 3, True),
                                             ("f32-affine-tanh", 6, 2, True), ("i8-affine-tanh-b5", 3, 4, True),
                                             ("bf16-d128-b3", 6, 4, False), ("bf16-affine-tanh-b1", 5, 2, True)])
def test_prefill_matches_oracle(name, S, P0, tanh):
    wl = CASES[name][0]
    gl, ow = gpu_layer_and_oracle_weights(wl, 0, gelu_tanh=tanh)
    kv, ok, ov, lens = filled_caches(wl, 0, gl, past=P0)
    x = syn.normal((wl.batch, S, wl.hidden), 1.0, wl.cfg_id, syn.X_LAYER, 3, "cuda").to(gl.cfg.torch_act_dtype)
    y = gl.prefill(kv, x)
    desc = oracle.Desc(wl.hidden, wl.heads, wl.head_dim, wl.ffn, gelu_tanh=tanh)
    yo = oracle.layer_forward(desc, ow, ok, ov, lens, x.double().cpu().numpy())
    yd, xd = y.double().cpu().numpy(), x.double().cpu().numpy()
    assert rel_l2(yd, yo) <= TOL[wl.act_dtype]
    assert rel_l2(yd - xd, yo - xd) <= TOL[wl.act_dtype]
    kg = kv.k.double().cpu().numpy()
    vg = kv.v.double().cpu().numpy()
    assert rel_l2(kg[:, :, :P0 + S], ok[:, :, :P0 + S]) <= TOL[wl.act_dtype]
    assert rel_l2(vg[:, :, :P0 + S], ov[:, :, :P0 + S]) <= TOL[wl.act_dtype]
    assert kv.lengths() == [P0 + S] * wl.batch


@pytest.mark.parametrize("name,parts", [
    ("f16-d64-b9", ["ln1", "qkv", "attn", "o", "ln2", "ff1", "ff2"]),
    ("bf16-d64-b9", ["ln1", "qkv", "attn", "o", "ln2", "ff1", "ff2"]),
    ("c1", ["qkv", "attn", "o", "ff1", "ff2", "len"]),
])
def test_time_kernels_runs_the_same_step(name, parts):
    """The timing aid runs exactly the decode step (same outputs, same cache rows, same lengths) and
    names its kernel launches in order."""
    wl = SMALL[name]
    gl, _ = gpu_layer_and_oracle_weights(wl, 0)
    x = syn.normal((wl.batch, wl.hidden), 1.0, wl.cfg_id, syn.X_LAYER, 0, "cuda").to(gl.cfg.torch_act_dtype)
    kv1, *_ = filled_caches(wl, 0, gl)
    y1 = gl.decode(kv1, x)
    kv2, *_ = filled_caches(wl, 0, gl)
    y2 = torch.empty_like(y1)
    timed = gl.time_kernels(kv2, x, y2)
    torch.cuda.synchronize()
    assert [p for p, _ in timed] == parts
    assert all(ms > 0 for _, ms in timed)
    assert torch.equal(y1, y2) and torch.equal(kv1.k, kv2.k) and torch.equal(kv1.v, kv2.v)
    assert kv1.lengths() == kv2.lengths()
