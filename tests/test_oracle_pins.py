"""Pins of the oracle to things other than itself (CPU only).

Each test checks the oracle against a closed form, an invariant, a hand-worked example
(tests/golden/) or an independent library routine (torch float64 on the CPU), chosen so that a
plausible mistake -- a dropped bias, a wrong sign or index, a transposed operand, an off-by-one in
the mask, a wrong variance or scale -- fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


# ------------------------------------------------------------------ LayerNorm
@pytest.mark.parametrize("n", [4, 63, 256, 2560])
def test_layernorm_mean_zero_and_closed_form_variance(n):
    x = rng.normal(0.3, 1.7, n)
    out = oracle.layernorm(x, np.ones(n), np.zeros(n), 1e-5)
    var = np.mean((x - x.mean()) ** 2)  # biased variance of the input
    assert abs(out.mean()) < 1e-12
    # with gamma=1, beta=0 the output variance is var/(var+eps) exactly
    assert abs(np.mean(out ** 2) - var / (var + 1e-5)) < 1e-12


def test_layernorm_hand_example():
    # [1,2,3,4]: mean 2.5, biased variance 1.25
    out = oracle.layernorm(np.array([1.0, 2, 3, 4]), np.ones(4), np.zeros(4), 1e-5)
    expect = (np.array([1.0, 2, 3, 4]) - 2.5) / math.sqrt(1.25 + 1e-5)
    assert np.max(np.abs(out - expect)) < 1e-15


def test_layernorm_affine_and_torch():
    n = 96
    x, g, b = rng.normal(size=n), rng.normal(size=n), rng.normal(size=n)
    plain = oracle.layernorm(x, np.ones(n), np.zeros(n), 1e-5)
    out = oracle.layernorm(x, g, b, 1e-5)
    assert np.max(np.abs(out - (plain * g + b))) < 1e-13
    ref = Fn.layer_norm(torch.tensor(x), (n,), torch.tensor(g), torch.tensor(b), 1e-5).numpy()
    assert np.max(np.abs(out - ref)) < 1e-13


# ------------------------------------------------------------------ GEMV
@pytest.mark.parametrize("n,k", [(1, 1), (3, 65), (63, 64), (64, 3), (65, 63)])
def test_linear_small_integers_exact(n, k):
    # small integers make every product and partial sum exact in double
    w = rng.integers(-5, 6, (n, k)).astype(np.float64)
    x = rng.integers(-5, 6, k).astype(np.float64)
    b = rng.integers(-5, 6, n).astype(np.float64)
    out = oracle.linear(w, b, x)
    ref = (torch.tensor(w) @ torch.tensor(x) + torch.tensor(b)).numpy()
    assert np.array_equal(out, ref)


def test_linear_closed_forms():
    k = 37
    x = rng.normal(size=k)
    assert np.array_equal(oracle.linear(np.eye(k), None, x), x)                # identity
    ones = oracle.linear(np.ones((5, k)), np.arange(5.0), np.arange(1.0, k + 1))
    assert np.array_equal(ones, k * (k + 1) / 2 + np.arange(5.0))              # sum 1..k + bias
    # a non-square shape catches a transposed operand: row o of [n,k] meets x
    w = np.zeros((3, k))
    w[2, 5] = 1.0
    assert np.array_equal(oracle.linear(w, None, x), np.array([0.0, 0.0, x[5]]))


def test_linear_matches_torch_float64():
    w, x, b = rng.normal(size=(70, 129)), rng.normal(size=129), rng.normal(size=70)
    ref = Fn.linear(torch.tensor(x), torch.tensor(w), torch.tensor(b)).numpy()
    assert np.max(np.abs(oracle.linear(w, b, x) - ref)) < 1e-13


# ------------------------------------------------------------------ GeLU
def test_gelu_textbook_values():
    # GeLU(u) = u * Phi(u); Phi(1) = 0.8413447460685429, Phi(2) = 0.9772498680518208 (normal table)
    assert oracle.gelu(np.array([0.0]))[0] == 0.0
    assert abs(oracle.gelu(np.array([1.0]))[0] - 0.8413447460685429) < 1e-15
    assert abs(oracle.gelu(np.array([-1.0]))[0] - (-1.0 + 0.8413447460685429)) < 1e-15
    assert abs(oracle.gelu(np.array([2.0]))[0] - 2 * 0.9772498680518208) < 1e-15


def test_gelu_odd_identity_and_torch():
    u = rng.normal(0, 3, 200)
    g, gm = oracle.gelu(u), oracle.gelu(-u)
    assert np.max(np.abs(g - gm - u)) < 1e-14      # u Phi(u) - (-u) Phi(-u) = u since Phi(u) + Phi(-u) = 1
    ref = Fn.gelu(torch.tensor(u)).numpy()
    assert np.max(np.abs(g - ref)) < 1e-14
    ref_t = Fn.gelu(torch.tensor(u), approximate="tanh").numpy()
    assert np.max(np.abs(oracle.gelu(u, tanh_form=True) - ref_t)) < 1e-14


# ------------------------------------------------------------------ softmax / attention
def test_softmax_invariants():
    s = rng.normal(size=50)
    p = oracle.softmax(s)
    assert abs(p.sum() - 1.0) < 1e-14
    assert np.max(np.abs(oracle.softmax(s + 123.25) - p)) < 1e-15   # shift invariance
    one = oracle.softmax(np.array([0.0, 1000.0, 0.0]))
    assert np.array_equal(one, np.array([0.0, 1.0, 0.0]))
    assert np.max(np.abs(p - torch.softmax(torch.tensor(s), 0).numpy())) < 1e-15


def test_attend_single_key_and_identical_keys():
    d = 64
    q, k, v = rng.normal(size=d), rng.normal(size=(1, d)), rng.normal(size=(1, d))
    assert np.array_equal(oracle.attend(q, k, v), v[0])          # one key: weight exactly 1
    keys = np.tile(rng.normal(size=d), (7, 1))
    vals = rng.normal(size=(7, d))
    assert np.max(np.abs(oracle.attend(q, keys, vals) - vals.mean(0))) < 1e-15


def test_attend_matches_sdpa():
    d, n = 128, 33
    q, k, v = rng.normal(size=d), rng.normal(size=(n, d)), rng.normal(size=(n, d))
    ref = Fn.scaled_dot_product_attention(torch.tensor(q)[None, None], torch.tensor(k)[None],
                                          torch.tensor(v)[None]).numpy()[0, 0]
    assert np.max(np.abs(oracle.attend(q, k, v) - ref)) < 1e-14


# ------------------------------------------------------------------ fp16 and the quantizer
def test_fp16_golden_cases():
    cases = json.load(open(os.path.join(GOLD, "fp16_rounding.json")))["cases"]
    for c in cases:
        assert int(oracle.fp16_from_double(np.array([c["x"]]))[0]) == c["bits"], c


def test_fp16_matches_numpy_rounding():
    # numpy's float64 -> float16 cast is round-to-nearest-even; probe normals, subnormals,
    # exact midpoints between neighbours, and the overflow boundary
    v = np.concatenate([rng.normal(0, 1, 2000), rng.normal(0, 1e-5, 500), rng.normal(0, 3e4, 500)])
    h = np.arange(0, 0x7bff, 37, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (h[:-1] + np.nextafter(h[:-1].astype(np.float16), np.float16(np.inf)).astype(np.float64)) / 2
    v = np.concatenate([v, mids, -mids, [65504.0, 65519.0, 65520.0, 1e6, 0.0]])
    ours = oracle.fp16_from_double(v)
    ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)
    # and every non-NaN bit pattern widens to numpy's value
    allh = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    back = oracle.fp16_to_double(allh)
    ref_back = allh.view(np.float16).astype(np.float64)
    ok = ~np.isnan(ref_back)
    assert np.array_equal(back[ok], ref_back[ok]) and np.all(np.isnan(back[~ok]))


def test_quantizer_golden_examples():
    gold = json.load(open(os.path.join(GOLD, "quant_group_examples.json")))
    G = gold["group"]
    for c in gold["cases"]:
        w = np.zeros((1, G), dtype=np.float32)
        w[0, :len(c["w_head"])] = c["w_head"]
        q, s = oracle.quantize_i8(w, G)
        assert int(s[0, 0]) == c["scale_bits"], c["name"]
        assert oracle.fp16_to_double(s)[0, 0] == c["scale_value"]
        assert list(q[0, :len(c["q_head"])]) == c["q_head"], c["name"]
        assert not q[0, len(c["q_head"]):].any()


@pytest.mark.parametrize("G", [64, 32, 16])
def test_quantizer_bounds_and_idempotence(G):
    w = (rng.normal(0, 0.02, (48, 256))).astype(np.float32)
    w[3, 64:128] = 0.0                      # one all-zero group (whole groups at every G here)
    w[5, 7] = 0.9                           # one outlier
    q, s = oracle.quantize_i8(w, G)
    assert s.shape == (48, 256 // G)
    sv = oracle.fp16_to_double(s)
    deq = oracle.dequantize_i8(q, s, G)
    per = np.repeat(sv, G, axis=1)
    assert np.all(np.abs(w.astype(np.float64) - deq) <= per / 2 * (1 + 1e-12))   # |w - q s| <= s/2
    assert np.all(np.abs(q.astype(int)) <= 127)
    amax = np.abs(w.reshape(48, 256 // G, G)).max(-1)
    qmax = np.abs(q.astype(int).reshape(48, 256 // G, G)).max(-1)
    assert np.all(qmax[amax > 0] == 127) and np.all(qmax[amax == 0] == 0)
    assert np.all(sv[3, 64 // G:128 // G] == 0.0)
    # dequantized values are exact in float32, and quantizing them again returns (q, s)
    assert np.array_equal(deq.astype(np.float32).astype(np.float64), deq)
    q2, s2 = oracle.quantize_i8(deq.astype(np.float32), G)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


def test_quantizer_group_32_boundaries():
    """Groups of 32 along K (the finer MLP groups): each half of a 64-wide row gets its own scale.
    amax = f32(0.127) gives the scale 1049 * 2^-20 (fp16 bits 0x1419, the golden 'rounded scale'
    case); amax = f32(0.254), exactly twice that, gives exactly twice the scale (0x1819: one binade
    up, same significand). So 0.127 codes as 127 in the first group and as round(63.47) = 63 in the
    second, and as 63 under a single group of 64."""
    w = np.zeros((1, 64), np.float32)
    w[0, 0], w[0, 32], w[0, 33] = 0.127, 0.254, 0.127
    q, s = oracle.quantize_i8(w, 32)
    assert [int(v) for v in s[0]] == [0x1419, 0x1819]
    assert (int(q[0, 0]), int(q[0, 32]), int(q[0, 33])) == (127, 127, 63)
    assert np.count_nonzero(q) == 3
    q64, s64 = oracle.quantize_i8(w, 64)
    assert [int(v) for v in s64[0]] == [0x1819]
    assert (int(q64[0, 0]), int(q64[0, 32]), int(q64[0, 33])) == (63, 127, 63)


# ------------------------------------------------------------------ the whole layer
def _rand_layer(H, nh, F, seed, zero=()):
    r = np.random.default_rng(seed)
    w = {"ln1_g": r.normal(1, 0.1, H), "ln1_b": r.normal(0, 0.1, H),
         "w_qkv": r.normal(0, 0.05, (3 * H, H)), "b_qkv": r.normal(0, 0.1, 3 * H),
         "w_o": r.normal(0, 0.05, (H, H)), "b_o": r.normal(0, 0.1, H),
         "ln2_g": r.normal(1, 0.1, H), "ln2_b": r.normal(0, 0.1, H),
         "w_ff1": r.normal(0, 0.05, (F, H)), "b_ff1": r.normal(0, 0.1, F),
         "w_ff2": r.normal(0, 0.05, (H, F)), "b_ff2": r.normal(0, 0.1, H)}
    for z in zero:
        w[z] = np.zeros_like(w[z])
    return w


def _cache(B, nh, cap, d, past, seed):
    r = np.random.default_rng(seed)
    k = np.zeros((B, nh, cap, d))
    v = np.zeros((B, nh, cap, d))
    k[:, :, :past] = r.normal(size=(B, nh, past, d))
    v[:, :, :past] = r.normal(size=(B, nh, past, d))
    return k, v, np.full(B, past, dtype=np.int32)


def _torch_layer(w, kpast, vpast, x, causal=True):
    """float64 composition of torch library ops: layer_norm, linear, SDPA, gelu."""
    t = {n: torch.tensor(a) for n, a in w.items()}
    B, T, H = x.shape
    nh, P, d = kpast.shape[1], kpast.shape[2], kpast.shape[3]
    xt = torch.tensor(x)
    h = Fn.layer_norm(xt, (H,), t["ln1_g"], t["ln1_b"], 1e-5)
    z = Fn.linear(h, t["w_qkv"], t["b_qkv"])
    q, k, v = z[..., :H], z[..., H:2 * H], z[..., 2 * H:]
    sh = lambda a: a.reshape(B, T, nh, d).permute(0, 2, 1, 3)
    K = torch.cat([torch.tensor(kpast), sh(k)], 2)
    V = torch.cat([torch.tensor(vpast), sh(v)], 2)
    mask = None
    if causal:
        pos_q = torch.arange(T)[:, None] + P
        mask = torch.arange(P + T)[None, :] <= pos_q
    ctx = Fn.scaled_dot_product_attention(sh(q), K, V, attn_mask=mask)
    ctx = ctx.permute(0, 2, 1, 3).reshape(B, T, H)
    x2 = xt + Fn.linear(ctx, t["w_o"], t["b_o"])
    g = Fn.gelu(Fn.linear(Fn.layer_norm(x2, (H,), t["ln2_g"], t["ln2_b"], 1e-5), t["w_ff1"], t["b_ff1"]))
    return (x2 + Fn.linear(g, t["w_ff2"], t["b_ff2"])).numpy(), K.numpy(), V.numpy()


@pytest.mark.parametrize("B,T,past,causal", [(1, 1, 32, True), (2, 5, 7, True), (2, 4, 3, False), (1, 6, 0, True)])
def test_layer_matches_torch_composition(B, T, past, causal):
    H, nh, F = 64, 4, 128
    d = H // nh
    w = _rand_layer(H, nh, F, 5)
    k, v, lens = _cache(B, nh, past + T + 2, d, past, 6)
    x = np.random.default_rng(7).normal(size=(B, T, H))
    kpast, vpast = k[:, :, :past].copy(), v[:, :, :past].copy()
    desc = oracle.Desc(H, nh, d, F, triangular_masking=causal)
    y = oracle.layer_forward(desc, w, k, v, lens, x)
    ref, K, V = _torch_layer(w, kpast, vpast, x, causal)
    assert np.max(np.abs(y - ref)) < 1e-12
    assert np.max(np.abs(k[:, :, :past + T] - K)) < 1e-13 and np.max(np.abs(v[:, :, :past + T] - V)) < 1e-13
    assert np.all(lens == past + T)


def test_layer_zero_weights_is_identity():
    H, nh, F = 64, 2, 96
    w = _rand_layer(H, nh, F, 1, zero=("w_qkv", "b_qkv", "w_o", "b_o", "w_ff1", "b_ff1", "w_ff2", "b_ff2"))
    k, v, lens = _cache(1, nh, 16, H // nh, 9, 2)
    x = np.random.default_rng(3).normal(size=(1, 1, H))
    y = oracle.layer_forward(oracle.Desc(H, nh, H // nh, F), w, k, v, lens, x)
    assert np.array_equal(y, x)


def test_layer_output_projections_zero_gives_biases():
    H, nh, F = 64, 2, 96
    w = _rand_layer(H, nh, F, 4, zero=("w_o", "w_ff2"))
    k, v, lens = _cache(2, nh, 16, H // nh, 5, 2)
    x = np.random.default_rng(3).normal(size=(2, 3, H))
    y = oracle.layer_forward(oracle.Desc(H, nh, H // nh, F), w, k, v, lens, x)
    assert np.array_equal(y, (x + w["b_o"]) + w["b_ff2"])


def test_layer_batch_independence():
    H, nh, F = 64, 4, 128
    w = _rand_layer(H, nh, F, 8)
    k, v, lens = _cache(3, nh, 20, H // nh, 6, 9)
    x = np.random.default_rng(10).normal(size=(3, 2, H))
    kk, vv, ll = k.copy(), v.copy(), lens.copy()
    y = oracle.layer_forward(oracle.Desc(H, nh, H // nh, F), w, k, v, lens, x)
    for b in range(3):
        k1, v1, l1 = kk[b:b + 1].copy(), vv[b:b + 1].copy(), ll[b:b + 1].copy()
        y1 = oracle.layer_forward(oracle.Desc(H, nh, H // nh, F), w, k1, v1, l1, x[b:b + 1])
        assert np.array_equal(y1, y[b:b + 1])


def test_layer_causal_zero_leakage_and_prefill_decode_consistency():
    H, nh, F, S = 64, 4, 128, 9
    desc = oracle.Desc(H, nh, H // nh, F)
    w = _rand_layer(H, nh, F, 11)
    x = np.random.default_rng(12).normal(size=(1, S, H))
    k, v, lens = _cache(1, nh, 16, H // nh, 0, 0)
    y = oracle.layer_forward(desc, w, k, v, lens, x)
    # perturbing row 6 leaves rows 0..5 bit-identical
    x2 = x.copy()
    x2[0, 6] += 1.0
    k2, v2, l2 = _cache(1, nh, 16, H // nh, 0, 0)
    y2 = oracle.layer_forward(desc, w, k2, v2, l2, x2)
    assert np.array_equal(y[0, :6], y2[0, :6]) and not np.array_equal(y[0, 6], y2[0, 6])
    # prefill of S-1 rows, then one decode row, reproduces the last row of prefill(S)
    k3, v3, l3 = _cache(1, nh, 16, H // nh, 0, 0)
    oracle.layer_forward(desc, w, k3, v3, l3, x[:, :S - 1])
    ylast = oracle.layer_forward(desc, w, k3, v3, l3, x[:, S - 1:])
    assert np.max(np.abs(ylast[0, 0] - y[0, S - 1])) < 1e-12
    assert np.max(np.abs(k3 - k)) < 1e-13


def test_layer_stage_outputs_consistent():
    H, nh, F = 64, 4, 128
    desc = oracle.Desc(H, nh, H // nh, F)
    w = _rand_layer(H, nh, F, 13)
    k, v, lens = _cache(1, nh, 12, H // nh, 4, 14)
    x = np.random.default_rng(15).normal(size=(1, 1, H))
    y, st = oracle.layer_forward(desc, w, k, v, lens, x, stages=True)
    ref = Fn.layer_norm(torch.tensor(x), (H,), torch.tensor(w["ln1_g"]), torch.tensor(w["ln1_b"]), 1e-5).numpy()
    assert np.max(np.abs(st["ln1"] - ref)) < 1e-13
    assert np.max(np.abs(st["x2"] - (x + st["ctx"] @ w["w_o"].T + w["b_o"]))) < 1e-12
    assert np.max(np.abs(st["act"] - Fn.gelu(torch.tensor(st["ff1"])).numpy())) < 1e-13
    assert np.max(np.abs(y - (st["x2"] + st["act"] @ w["w_ff2"].T + w["b_ff2"]))) < 1e-12


def test_layer_rejects_overflow():
    H, nh, F = 64, 4, 128
    w = _rand_layer(H, nh, F, 1)
    k, v, lens = _cache(1, nh, 8, H // nh, 8, 2)
    with pytest.raises(ValueError):
        oracle.layer_forward(oracle.Desc(H, nh, H // nh, F), w, k, v, lens, np.zeros((1, 1, H)))


# ------------------------------------------------------------------ the ends of a generation step
def test_argmax_golden_cases():
    gold = json.load(open(os.path.join(GOLD, "argmax_examples.json")))
    for case in gold["cases"]:
        assert oracle.argmax(np.array(case["values"])) == case["index"], case["note"]


def test_argmax_matches_numpy_and_takes_the_first_tie():
    # numpy's argmax returns the first position of the maximum, the same rule
    for n in (1, 2, 7, 64, 50257):
        v = rng.normal(size=n)
        assert oracle.argmax(v) == int(np.argmax(v))
        w = v.copy()
        i, j = sorted(rng.choice(n, size=2, replace=False)) if n > 1 else (0, 0)
        w[i] = w[j] = v.max() + 1.0   # an exact tie at the top
        assert oracle.argmax(w) == i


def _alternating(H, a):
    """y = [a, -a, a, -a, ...]: mean 0, biased variance a^2, so LN(y) = y / sqrt(a^2 + eps)."""
    y = np.empty(H)
    y[0::2], y[1::2] = a, -a
    return y


def test_lm_head_closed_form_with_small_integer_weights():
    H, V, a, eps = 8, 5, 1.5, 1e-5
    w = rng.integers(-3, 4, size=(V, H)).astype(np.float64)
    y = _alternating(H, a)
    logits = oracle.lm_head(y, np.ones(H), np.zeros(H), w, eps)
    sign = np.array([1.0, -1.0] * (H // 2))
    expect = (a / math.sqrt(a * a + eps)) * (w @ sign)   # integer sums, one scale
    assert np.max(np.abs(logits - expect)) < 1e-13
    # gamma = 0: the normalized row drops out and the logits are W beta, exactly (small integers)
    beta = rng.integers(-2, 3, size=H).astype(np.float64)
    assert np.array_equal(oracle.lm_head(y, np.zeros(H), beta, w, eps), w @ beta)
    # a transposed or shifted weight would break the per-row one-hot picks
    eye = np.zeros((H, H))
    eye[np.arange(H), (np.arange(H) + 3) % H] = 2.0
    picked = oracle.lm_head(y, np.ones(H), np.zeros(H), eye, eps)
    assert np.max(np.abs(picked - 2.0 * np.roll(y, -3) / math.sqrt(a * a + eps))) < 1e-13


def test_lm_head_matches_torch_float64_and_greedy_choice():
    H, V = 64, 300
    y = rng.normal(size=H)
    g, b = 1.0 + 0.2 * rng.normal(size=H), 0.2 * rng.normal(size=H)
    w = 0.02 * rng.normal(size=(V, H))
    ref = torch.from_numpy(w) @ Fn.layer_norm(torch.from_numpy(y), (H,), torch.from_numpy(g), torch.from_numpy(b), 1e-5)
    logits = oracle.lm_head(y, g, b, w)
    assert np.max(np.abs(logits - ref.numpy())) < 1e-13
    assert oracle.argmax(logits) == int(torch.argmax(ref))


# ------------------------------------------------------------------ the MoE expert FF
def _rand_moe(H, F, E, seed, residual=False):
    r = np.random.default_rng(seed)
    w = {"ln_g": r.normal(1, 0.1, H), "ln_b": r.normal(0, 0.1, H), "w_gate": r.normal(0, 0.3, (E, H)),
         "w1": r.normal(0, 0.05, (E, F, H)), "b1": r.normal(0, 0.1, (E, F)),
         "w2": r.normal(0, 0.05, (E, H, F)), "b2": r.normal(0, 0.1, (E, H))}
    if residual:
        w.update({"r_w1": r.normal(0, 0.05, (F, H)), "r_b1": r.normal(0, 0.1, F),
                  "r_w2": r.normal(0, 0.05, (H, F)), "r_b2": r.normal(0, 0.1, H)})
    return w


def _dense_ffn_via_layer(x2, ln_g, ln_b, w1, b1, w2, b2, tanh=False):
    """x2 + W2 GeLU(W1 LN(x2) + b1) + b2 through the (separately pinned) layer oracle: with
    W_o = 0 and b_o = 0 the attention adds nothing, so x2 = x and the layer's region 3 and 4 are
    exactly the dense FF of x2."""
    T, H = x2.shape
    F = w1.shape[0]
    lw = _rand_layer(H, 2, F, 99, zero=("w_o", "b_o"))
    lw.update({"ln2_g": ln_g, "ln2_b": ln_b, "w_ff1": w1, "b_ff1": b1, "w_ff2": w2, "b_ff2": b2})
    kc, vc = np.zeros((T, 2, 4, H // 2)), np.zeros((T, 2, 4, H // 2))
    lens = np.zeros(T, dtype=np.int32)
    return oracle.layer_forward(oracle.Desc(H, 2, H // 2, F, gelu_tanh=tanh), lw, kc, vc, lens, x2[:, None, :])[:, 0]


@pytest.mark.parametrize("tanh", [False, True])
def test_moe_single_expert_is_the_dense_ffn(tanh):
    H, F = 16, 24
    w = _rand_moe(H, F, 1, 31)
    x2 = rng.normal(0, 1, (3, H))
    y, sel, wgt = oracle.moe_forward(w, x2, top_k=1, gelu_tanh=tanh)
    ref = _dense_ffn_via_layer(x2, w["ln_g"], w["ln_b"], w["w1"][0], w["b1"][0], w["w2"][0], w["b2"][0], tanh)
    assert np.all(sel == 0) and np.all(wgt == 1.0)
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-13)


def test_moe_identical_experts_reduce_to_the_dense_ffn():
    # the combine weights sum to 1 whichever experts are chosen: renormalized top-2, or every
    # expert with its softmax probability
    H, F, E = 16, 20, 4
    one = _rand_moe(H, F, 1, 32)
    w = dict(one, w_gate=rng.normal(0, 1, (E, H)))
    for n in ("w1", "b1", "w2", "b2"):
        w[n] = np.repeat(one[n], E, axis=0)
    x2 = rng.normal(0, 1, (5, H))
    ref = _dense_ffn_via_layer(x2, w["ln_g"], w["ln_b"], one["w1"][0], one["b1"][0], one["w2"][0], one["b2"][0])
    y2, _, wgt2 = oracle.moe_forward(w, x2, top_k=2, combine=0)
    yall, _, wgta = oracle.moe_forward(w, x2, top_k=E, combine=1)
    np.testing.assert_allclose(wgt2.sum(1), 1.0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(wgta.sum(1), 1.0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(y2, ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(yall, ref, rtol=0, atol=1e-13)


def test_moe_permuting_the_experts_permutes_the_choice_only():
    H, F, E, k = 12, 16, 6, 2
    w = _rand_moe(H, F, E, 33)
    x2 = rng.normal(0, 1, (7, H))
    y, sel, wgt = oracle.moe_forward(w, x2, top_k=k)
    perm = np.array([3, 0, 5, 1, 4, 2])         # new expert i is old expert perm[i]
    wp = dict(w)
    for n in ("w_gate", "w1", "b1", "w2", "b2"):
        wp[n] = w[n][perm]
    yp, selp, wgtp = oracle.moe_forward(wp, x2, top_k=k)
    assert np.array_equal(perm[selp], sel)
    # equal up to the order of the softmax denominator's sum
    np.testing.assert_allclose(wgtp, wgt, rtol=1e-14)
    np.testing.assert_allclose(yp, y, rtol=0, atol=1e-14)
    # the chosen experts are the k most probable, most probable first
    for t in range(x2.shape[0]):
        h = oracle.layernorm(x2[t], w["ln_g"], w["ln_b"])
        p = oracle.softmax(w["w_gate"] @ h)
        order = sorted(range(E), key=lambda e: (-p[e], e))
        assert list(sel[t]) == order[:k]


def test_moe_gate_by_hand():
    """H = 4, x2 = (1, -1, 1, -1): LN gives h = x2 / sqrt(1 + eps) (mean 0, variance 1). Gate row e
    is c_e (1, -1, 1, -1) / 4, so logit_e = c_e / sqrt(1 + eps) with c = (0, 2, 1, 2, -1). The two
    largest are the tied experts 1 and 3, taken in index order, each with renormalized weight 1/2.
    Every expert has W1 = W2 = 0 and b1 = 0 (GeLU(0) = 0), so FF_e(h) = b2_e, the e-th basis
    vector times (e + 1): y = x2 + (2 e_1 + 4 e_3) / 2 = (1, 0, 1, 1)."""
    H, F, E = 4, 3, 5
    c = np.array([0.0, 2.0, 1.0, 2.0, -1.0])
    s = np.array([1.0, -1.0, 1.0, -1.0])
    b2 = np.zeros((E, H))
    for e in range(E):
        b2[e, e % H] = e + 1
    w = {"ln_g": np.ones(H), "ln_b": np.zeros(H), "w_gate": np.outer(c, s) / 4,
         "w1": np.zeros((E, F, H)), "b1": np.zeros((E, F)), "w2": np.zeros((E, H, F)), "b2": b2}
    x2 = s[None, :]
    y, sel, wgt = oracle.moe_forward(w, x2, top_k=2, combine=0)
    assert list(sel[0]) == [1, 3] and list(wgt[0]) == [0.5, 0.5]
    np.testing.assert_allclose(y[0], [1.0, 0.0, 1.0, 1.0], rtol=0, atol=1e-15)
    # combine 1: the softmax probabilities themselves, exp(2a) / sum_e exp(c_e a), a = 1/sqrt(1+eps)
    a = 1 / math.sqrt(1 + 1e-5)
    p1 = math.exp(2 * a) / (1 + 2 * math.exp(2 * a) + math.exp(a) + math.exp(-a))
    y1, sel1, wgt1 = oracle.moe_forward(w, x2, top_k=2, combine=1)
    assert list(sel1[0]) == [1, 3]
    np.testing.assert_allclose(wgt1[0], [p1, p1], rtol=1e-14)
    np.testing.assert_allclose(y1[0], s + p1 * (2 * np.eye(H)[1] + 4 * np.eye(H)[3]), rtol=0, atol=1e-14)
    # top-1 with the tie: the smaller index
    _, selt, _ = oracle.moe_forward(w, x2, top_k=1)
    assert int(selt[0, 0]) == 1


def test_moe_residual_type_adds_the_dense_mlp():
    H, F, E = 16, 24, 3
    w = _rand_moe(H, F, E, 34, residual=True)
    x2 = rng.normal(0, 1, (4, H))
    y_res, sel, wgt = oracle.moe_forward(w, x2, top_k=2)
    std = {k: v for k, v in w.items() if not k.startswith("r_")}
    y_std, sel2, _ = oracle.moe_forward(std, x2, top_k=2)
    assert np.array_equal(sel, sel2)
    dense = _dense_ffn_via_layer(x2, w["ln_g"], w["ln_b"], w["r_w1"], w["r_b1"], w["r_w2"], w["r_b2"])
    np.testing.assert_allclose(y_res - y_std, dense - x2, rtol=0, atol=1e-13)


def test_moe_forced_selection():
    H, F, E = 8, 8, 4
    w = _rand_moe(H, F, E, 35)
    x2 = rng.normal(0, 1, (3, H))
    y, sel, wgt = oracle.moe_forward(w, x2, top_k=2)
    yf, self_, wgtf = oracle.moe_forward(w, x2, top_k=2, force_sel=sel)
    assert np.array_equal(y, yf) and np.array_equal(sel, self_) and np.array_equal(wgt, wgtf)
    other = (sel + 1) % E
    yo, selo, _ = oracle.moe_forward(w, x2, top_k=2, force_sel=other)
    assert np.array_equal(selo, other) and not np.allclose(yo, y)
    with pytest.raises(ValueError):
        oracle.moe_forward(w, x2, top_k=2, force_sel=np.full((3, 2), E))


# ------------------------------------------------------------------ the int8 KV cache reading
def test_kv_row_quantizer_matches_the_weight_quantizer():
    # on float32 rows the per-row quantizer is the (pinned) group quantizer with one group per row
    x = rng.normal(0, 1.3, (9, 128)).astype(np.float32)
    x[4] = 0.0
    q, s = oracle.quantize_rows_i8(x.astype(np.float64))
    qw, sw = oracle.quantize_i8(x, 128)
    assert np.array_equal(q, qw) and np.array_equal(s, sw[:, 0])
    assert s[4] == 0 and not q[4].any()


def test_kv_row_quantizer_by_hand():
    """amax 1.0: scale = fp16(1/127) = (1 + 8/1024) 2^-7 = 0.00787353515625 (bits 0x2008: 1/127
    lies 8.06 steps of 2^-17 above 2^-7). Codes: 1.0 / s = 127.008 -> 127, 0.3 / s = 38.10 -> 38,
    -0.5 / s = -63.504 -> -64, 0.125 / s = 15.876 -> 16."""
    q, s = oracle.quantize_rows_i8(np.array([[1.0, 0.3, -0.5, 0.125, 0.0, 0.0, 0.0, 0.0]]))
    assert int(s[0]) == 0x2008
    assert list(q[0, :5]) == [127, 38, -64, 16, 0]


def _kv_layer_case(H=64, nh=2, F=96, B=2, P=5, seed=40):
    w = _rand_layer(H, nh, F, seed)
    d = H // nh
    kc, vc, _ = _cache(B, nh, P + 3, d, P, seed + 1)
    x = rng.normal(0, 1, (B, 1, H))
    return w, kc, vc, x, d


def test_layer_int8_kv_with_exactly_representable_rows_is_the_fp_layer():
    # new K/V rows from the bias alone (W_qkv's K and V rows zero), each row holding 127 * 2^-4
    # and other multiples of 2^-4: the scale is 2^-4 exactly and every code exact, so the int8
    # cache holds the same values and the layer gives the same output bit for bit
    H, nh, F, B, P = 64, 2, 96, 2, 5
    w, kc, vc, x, d = _kv_layer_case(H, nh, F, B, P)
    w["w_qkv"][H:] = 0.0
    codes = rng.integers(-127, 128, 2 * H)
    codes[::d] = 127
    w["b_qkv"][H:] = codes * 2.0 ** -4
    out = []
    for kv8 in (False, True):
        k2, v2, lens = kc.copy(), vc.copy(), np.full(B, P, dtype=np.int32)
        y = oracle.layer_forward(oracle.Desc(H, nh, d, F, kv_int8=kv8), w, k2, v2, lens, x)
        out.append((y, k2, v2))
    assert np.array_equal(out[0][0], out[1][0])
    assert np.array_equal(out[0][1], out[1][1]) and np.array_equal(out[0][2], out[1][2])


def test_layer_int8_kv_cache_holds_the_quantized_rows():
    H, nh, F, B, P = 64, 2, 96, 2, 5
    w, kc, vc, x, d = _kv_layer_case(H, nh, F, B, P, seed=41)
    k_fp, v_fp, lens = kc.copy(), vc.copy(), np.full(B, P, dtype=np.int32)
    y_fp = oracle.layer_forward(oracle.Desc(H, nh, d, F), w, k_fp, v_fp, lens, x)
    k8, v8, lens = kc.copy(), vc.copy(), np.full(B, P, dtype=np.int32)
    y8 = oracle.layer_forward(oracle.Desc(H, nh, d, F, kv_int8=True), w, k8, v8, lens, x)
    for fp, c8 in ((k_fp, k8), (v_fp, v8)):
        q, s = oracle.quantize_rows_i8(fp[:, :, P])
        want = q.astype(np.float64) * oracle.fp16_to_double(s)[..., None]
        assert np.array_equal(c8[:, :, P], want)                  # the new row: q * s
        assert np.array_equal(c8[:, :, :P], fp[:, :, :P])          # the past rows untouched
    # the attention sees the quantized rows: close to the fp layer, not equal
    assert not np.array_equal(y8, y_fp) and np.allclose(y8, y_fp, rtol=0, atol=5e-2)
