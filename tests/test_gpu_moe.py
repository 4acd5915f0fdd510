"""The MoE expert FF (ds_moe_*) against the oracle's moe_forward on the same seeded inputs.

The gate decides in fp32 from the LayerNorm rows rounded to the activation type; the oracle decides
in double from exact rows. Where the two choose different experts, the test accepts it only as a
near tie (the oracle's probabilities of the two choices agree to within the gate's rounding) and
then checks y against the oracle run on the GPU's choice (force_sel), so the products and the
combination are always compared element by element.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
import transformer_gpt_layer_amd as tg
from tests._common import TOL, TORCH, rel_l2

pytestmark = pytest.mark.gpu

DT = {"f32": "fp32", "f16": "fp16", "i8": "int8", "bf16": "bf16"}
# how far apart (absolute, in probability) two choices may be and still count as a tie decided by
# rounding: the gate's logits move by about |logit| x the activation type's unit roundoff
TIE = {"f32": 1e-5, "f16": 4e-3, "bf16": 3e-2}
U = {"f32": 2.0 ** -24, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}  # unit roundoff of the activation type


def _mw(**kw):
    base = syn.MoeWorkload("moe-test", 500, 256, 512, 4, 2, 3, "f16", "f16")
    return dataclasses.replace(base, **kw)


def gpu_moe_and_oracle(mw, gelu_tanh=False, device="cuda"):
    """A library MoE over the workload's weights and the oracle's float64 copies of the same values
    (int8: the GPU quantizer's codes, checked bit for bit against the oracle's quantizer)."""
    w32 = syn.moe_weights_f32(mw, device)
    act, wdt = TORCH[mw.act_dtype], TORCH.get(mw.weight_dtype)
    gw, ow = {}, {}
    for n, t in w32.items():
        if n in ("w1", "w2", "r_w1", "r_w2"):
            if mw.weight_dtype == "i8":
                t2 = t.reshape(-1, t.shape[-1]).contiguous()
                q, s = tg.quantize_i8(t2, mw.group)
                oq, os_ = oracle.quantize_i8(t2.cpu().numpy(), mw.group)
                assert np.array_equal(q.cpu().numpy(), oq), f"int8 codes of {n} differ from the oracle"
                sb = s.cpu().view(torch.int16).numpy().view(np.uint16)
                assert np.array_equal(sb, os_), f"fp16 scales of {n} differ from the oracle"
                gw[n] = q.reshape(t.shape)
                gw[n.replace("w", "s", 1)] = s.reshape(t.shape[:-1] + (t.shape[-1] // mw.group,))
                ow[n] = oracle.dequantize_i8(oq, os_, mw.group).reshape(t.shape)
            else:
                gw[n] = t.to(wdt).contiguous()
                ow[n] = gw[n].double().cpu().numpy()
        else:
            gw[n] = t.to(act).contiguous()
            ow[n] = gw[n].double().cpu().numpy()
    moe = tg.MoE(mw.hidden, mw.ffn, mw.experts, mw.top_k, gw, dtype=DT[mw.weight_dtype],
                 quant_group=mw.group if mw.weight_dtype == "i8" else None, gelu_tanh=gelu_tanh, combine=mw.combine)
    return moe, ow


def oracle_probs(ow, xd):
    out = []
    for row in xd:
        h = oracle.layernorm(row, ow["ln_g"], ow["ln_b"])
        out.append(oracle.softmax(oracle.linear(ow["w_gate"], None, h)))
    return np.array(out)


def check_step(mw, moe, ow, x, gelu_tanh, label):
    y, sel, wgt = moe.forward(x, routing=True)
    torch.cuda.synchronize()
    xd = x.double().cpu().numpy()
    yo, selo, _ = oracle.moe_forward(ow, xd, top_k=mw.top_k, gelu_tanh=gelu_tanh, combine=mw.combine)
    sg = sel.cpu().numpy()
    assert sg.min() >= 0 and sg.max() < mw.experts
    assert all(len(set(r)) == mw.top_k for r in sg), "an expert chosen twice for one token"
    diff = np.flatnonzero((sg != selo).any(1))
    if diff.size:
        p = oracle_probs(ow, xd)
        for t in diff:
            got, want = np.sort(p[t][sg[t]])[::-1], np.sort(p[t][selo[t]])[::-1]
            assert np.all(np.abs(got - want) <= TIE[mw.act_dtype]), (label, t, sg[t], selo[t], got, want)
        assert diff.size <= max(1, mw.tokens // 8), (label, "too many near ties", diff.size)
    yf, self_, wgtf = oracle.moe_forward(ow, xd, top_k=mw.top_k, gelu_tanh=gelu_tanh, combine=mw.combine, force_sel=sg)
    yd = y.double().cpu().numpy()
    err, err_d = rel_l2(yd, yf), rel_l2(yd - xd, yf - xd)
    werr = float(np.abs(wgt.cpu().numpy() - wgtf).max())
    print(f"  {label}: rel L2 {err:.3e}, of y - x {err_d:.3e}, weights max |diff| {werr:.2e}, "
          f"{diff.size} near ties", flush=True)
    # y is stored in the activation type: its rounding (RMS u/sqrt(3) of |y|) is the floor of the
    # y - x view, large when the block's contribution is a small part of y (raw probabilities over
    # many experts); that view's bar is twice the floor, and never below the dtype's bar
    tol = TOL[mw.act_dtype]
    floor = U[mw.act_dtype] / np.sqrt(3) * np.sqrt(np.mean(yf ** 2) / np.mean((yf - xd) ** 2))
    assert err <= tol and err_d <= max(tol, 2 * floor), (label, err, err_d, floor)
    assert werr <= TIE[mw.act_dtype] * 2, (label, werr)
    return sg


CASES = {
    "f16-e4-k2-t3": _mw(),
    "f16-e16-k1-t8-residual-tanh": (_mw(experts=16, top_k=1, tokens=8, residual=True, cfg_id=501, ln_std=0.2), True),
    "bf16-e8-k2-t5-combine1": _mw(experts=8, tokens=5, weight_dtype="bf16", act_dtype="bf16", combine=1, cfg_id=502),
    "i8-e4-k2-t8-g64": _mw(experts=4, tokens=8, weight_dtype="i8", act_dtype="f16", group=64, cfg_id=503, bias_std=0.1),
    "i8-e6-k3-t4-g32-residual": _mw(experts=6, top_k=3, tokens=4, weight_dtype="i8", act_dtype="f16", group=32,
                                    residual=True, cfg_id=504),
    "f32-e5-k2-t2": _mw(experts=5, tokens=2, weight_dtype="f32", act_dtype="f32", cfg_id=505),
    # many tokens per expert: every expert takes its tokens in several tiles of 8
    "f16-e2-k1-t37": _mw(experts=2, top_k=1, tokens=37, hidden=512, ffn=1024, cfg_id=506),
    "f16-e1-k1-t4": _mw(experts=1, top_k=1, tokens=4, cfg_id=507),
    # more than 64 experts (several per gate lane), eight per token, and more than 256 experts
    # (several per routing thread)
    "f16-e130-k8-t16": _mw(experts=130, top_k=8, tokens=16, hidden=128, ffn=256, cfg_id=508),
    "bf16-e300-k2-t3-residual": _mw(experts=300, top_k=2, tokens=3, hidden=128, ffn=128, weight_dtype="bf16",
                                    act_dtype="bf16", residual=True, cfg_id=509),
    "f16-e64-k2-t1-wide": _mw(experts=64, top_k=2, tokens=1, hidden=1024, ffn=4096, cfg_id=510),
}


@pytest.mark.parametrize("name", list(CASES))
def test_moe_matches_oracle(name):
    case = CASES[name]
    mw, tanh = case if isinstance(case, tuple) else (case, False)
    print(f"[moe parity] {name}: {mw} gelu_tanh={tanh}", flush=True)
    moe, ow = gpu_moe_and_oracle(mw, gelu_tanh=tanh)
    act = TORCH[mw.act_dtype]
    with moe:
        for step in range(2):
            x = syn.moe_input_f32(mw, "cuda", step).to(act)
            check_step(mw, moe, ow, x, tanh, f"step {step}")


def test_moe_output_may_alias_input_and_is_deterministic():
    mw = _mw(experts=8, tokens=6, cfg_id=511)
    moe, ow = gpu_moe_and_oracle(mw)
    with moe:
        x = syn.moe_input_f32(mw, "cuda").half()
        y1 = moe.forward(x)
        y2 = moe.forward(x)
        xa = x.clone()
        ws = moe.workspace(mw.tokens)
        moe.forward(xa, y=xa, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2) and torch.equal(y1, xa)


def test_moe_time_kernels_runs_the_same_step():
    mw = _mw(experts=8, tokens=4, cfg_id=512)
    moe, ow = gpu_moe_and_oracle(mw)
    with moe:
        x = syn.moe_input_f32(mw, "cuda").half()
        ms = moe.time_kernels(x)
        assert list(ms) == ["gate", "route", "ff1", "ff2", "combine"] and all(v > 0 for v in ms.values())
        y = moe.forward(x)
        torch.cuda.synchronize()
        assert torch.isfinite(y.float()).all()


def test_moe_full_size_sampled():
    """The MoE page's 1.3B + MoE-128 block at its real shapes (hidden 2048, 128 experts of width
    8192, top-1) for 8 tokens, in the launch configuration the benchmark times. The oracle runs on
    the experts the GPU chose only (copied to the host with the gate), every token and element."""
    mw = syn.MOE_WORKLOADS["moe-1.3b-e128"]
    print(f"[moe full size] {mw}", flush=True)
    w32 = syn.moe_weights_f32(mw, "cuda")
    gw = {n: t.half().contiguous() for n, t in w32.items()}
    del w32
    torch.cuda.empty_cache()
    moe = tg.MoE(mw.hidden, mw.ffn, mw.experts, mw.top_k, gw, dtype="fp16")
    with moe:
        x = syn.moe_input_f32(mw, "cuda").half()
        y, sel, wgt = moe.forward(x, routing=True)
        torch.cuda.synchronize()
        sg = sel.cpu().numpy()
        used = sorted(set(int(e) for e in sg.ravel()))
        print(f"  experts chosen: {used}", flush=True)
        # the gate over all experts (for the choice), the chosen experts' weights only (for y):
        # with top-1 and renormalized weights the chosen expert's weight is 1 whatever the others
        ow_gate = {"ln_g": gw["ln_g"].double().cpu().numpy(), "ln_b": gw["ln_b"].double().cpu().numpy(),
                   "w_gate": gw["w_gate"].double().cpu().numpy()}
        xd = x.double().cpu().numpy()
        p = oracle_probs(ow_gate, xd)
        top = p.argmax(1)
        for t in range(mw.tokens):
            assert sg[t, 0] == top[t] or abs(p[t, sg[t, 0]] - p[t, top[t]]) <= TIE["f16"], (t, sg[t], top[t])
        idx = torch.tensor(used, device="cuda")
        ow = dict(ow_gate, w_gate=ow_gate["w_gate"][used])
        for n in ("w1", "b1", "w2", "b2"):
            ow[n] = gw[n].index_select(0, idx).double().cpu().numpy()
        local = np.searchsorted(np.array(used), sg)
        yf, _, _ = oracle.moe_forward(ow, xd, top_k=1, force_sel=local)
        yd = y.double().cpu().numpy()
        err, err_d = rel_l2(yd, yf), rel_l2(yd - xd, yf - xd)
        print(f"  rel L2 {err:.3e}, of y - x {err_d:.3e}", flush=True)
        assert err <= TOL["f16"] and err_d <= TOL["f16"]
        assert np.allclose(wgt.cpu().numpy(), 1.0)
