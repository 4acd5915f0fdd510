"""GPU parity of the generation step's ends in the persistent kernel: the final LayerNorm, the LM
head and the greedy choice (ds_stack_forward_generate) against the oracle.

The logits are compared with the oracle's to the fp16 (or fp32) bar. The token is an integer that
floating point decides, so it is checked in the kernel's own precision: it must be the first
position of the largest fp32 logit the kernel returned. It must also be the oracle's choice whenever
the oracle's two largest logits are further apart than the logits' error, and otherwise a logit
within that distance of the oracle's largest. An exact-tie case (logits that are small integers in
any summation order) pins the tie rule: the smallest position wins.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
import transformer_gpt_layer_amd as tg
from tests._common import TOL, TORCH, rel_l2
from tests.test_gpu_stack import build, oracle_step

pytestmark = pytest.mark.gpu


def _wl(**kw):
    return dataclasses.replace(syn.WORKLOADS["c1"], **kw)


def gpu_head(wl, vocab, cfg):
    """Device head tensors and the oracle's float64 copies of exactly the same values."""
    h32 = syn.lm_head_f32(wl, vocab, "cuda")
    act = TORCH[wl.act_dtype]
    head = {"ln_g": h32["ln_g"].to(act).contiguous(), "ln_b": h32["ln_b"].to(act).contiguous()}
    if wl.weight_dtype == "i8":
        q, s = tg.quantize_i8(h32["w"].contiguous(), wl.group)
        oq, os_ = oracle.quantize_i8(h32["w"].cpu().numpy(), wl.group)
        assert np.array_equal(q.cpu().numpy(), oq)
        assert np.array_equal(s.cpu().view(torch.int16).numpy().view(np.uint16), os_)
        head["w"], head["s"] = q, s
        ow = oracle.dequantize_i8(oq, os_, wl.group)
    else:
        head["w"] = h32["w"].to(act).contiguous()
        ow = head["w"].double().cpu().numpy()
    ohead = {"ln_g": head["ln_g"].double().cpu().numpy(), "ln_b": head["ln_b"].double().cpu().numpy(), "w": ow}
    return head, ohead


def check_tokens(logits_gpu, tokens_gpu, logits_ora, margin):
    lg = logits_gpu.double().cpu().numpy()
    tk = tokens_gpu.cpu().numpy()
    for b in range(lg.shape[0]):
        # the kernel's choice in the kernel's precision: the first position of its largest logit
        first = int(np.flatnonzero(lg[b] == lg[b].max())[0])
        assert int(tk[b]) == first, (b, int(tk[b]), first)
        lo = logits_ora[b]
        top2 = np.sort(lo)[-2:]
        if top2[1] - top2[0] > 2 * margin:
            assert int(tk[b]) == oracle.argmax(lo), (b, int(tk[b]), oracle.argmax(lo), top2)
        else:
            assert lo[int(tk[b])] >= lo.max() - 2 * margin


CASES = {
    # (workload, layers, vocab, gelu_tanh): vocabularies that leave ragged row tiles on 256 workgroups
    "f16-d128-b1-L2-v1000": (_wl(hidden=512, heads=4, head_dim=128, ffn=1024, weight_dtype="f16", act_dtype="f16",
                                 batch=1, past=40, cfg_id=401, ln_std=0.2, bias_std=0.1), 2, 1000, False),
    "f16-d64-b3-L2-v777": (_wl(hidden=1024, heads=16, head_dim=64, ffn=2048, weight_dtype="f16", act_dtype="f16",
                               batch=3, past=21, cfg_id=402, ln_std=0.2), 2, 777, True),
    "i8-d128-b1-L2-v3001": (_wl(hidden=1024, heads=8, head_dim=128, ffn=2048, weight_dtype="i8", act_dtype="f16",
                                group=64, batch=1, past=9, cfg_id=403, ln_std=0.2, bias_std=0.1), 2, 3001, False),
    "i8-d128-b4-L2-v300": (_wl(hidden=1024, heads=8, head_dim=128, ffn=2048, weight_dtype="i8", act_dtype="f16",
                               group=64, batch=4, past=70, cfg_id=404, ln_std=0.2), 2, 300, True),
    "f32-d64-b1-L2-v129": (_wl(cfg_id=405, ln_std=0.2, bias_std=0.1), 2, 129, False),
    "bf16-d128-b1-L2-v1000": (_wl(hidden=512, heads=4, head_dim=128, ffn=1024, weight_dtype="bf16", act_dtype="bf16",
                                  batch=1, past=40, cfg_id=408, ln_std=0.2, bias_std=0.1), 2, 1000, True),
    # finer MLP groups: the LM head keeps the attention group
    "i8-d128-b2-L2-v500-mlp32": (_wl(hidden=1024, heads=8, head_dim=128, ffn=2048, weight_dtype="i8", act_dtype="f16",
                                     group=64, group_mlp=32, batch=2, past=30, cfg_id=407, ln_std=0.2), 2, 500, False),
}


@pytest.mark.parametrize("name", list(CASES))
def test_generate_matches_oracle(name):
    wl, L, V, tanh = CASES[name]
    print(f"[generate parity] {name}: {wl} layers={L} vocab={V}", flush=True)
    gls, ows, kvs, oks, ovs, lens = build(wl, L, gelu_tanh=tanh)
    head, ohead = gpu_head(wl, V, gls[0].cfg)
    tol = TOL[wl.act_dtype]
    with tg.Stack(gls, kvs, max_batch=wl.batch, head=head) as st:
        ws = st.workspace(wl.batch)
        for step in range(3):
            x = syn.normal((wl.batch, wl.hidden), 1.0, wl.cfg_id, syn.X_LAYER, step, "cuda").to(gls[0].cfg.torch_act_dtype)
            if step == 1:
                # a plain decode step between two generation steps (the argmax slots alternate)
                st.decode(x, workspace=ws)
                st.check()
                oracle_step(wl, ows, oks, ovs, lens, x.double().cpu().numpy(), gelu_tanh=tanh)
                continue
            y, logits, tokens = st.generate(x, workspace=ws)
            st.check()
            yo = oracle_step(wl, ows, oks, ovs, lens, x.double().cpu().numpy(), gelu_tanh=tanh)
            assert rel_l2(y.double().cpu().numpy(), yo) <= tol
            lo = np.stack([oracle.lm_head(yo[b], ohead["ln_g"], ohead["ln_b"], ohead["w"]) for b in range(wl.batch)])
            err = rel_l2(logits.double().cpu().numpy(), lo)
            print(f"  step {step}: logits rel L2 {err:.3e}, tokens {tokens.tolist()}", flush=True)
            assert err <= tol, err
            margin = float(np.max(np.abs(logits.double().cpu().numpy() - lo)))
            check_tokens(logits, tokens, lo, max(margin, 1e-6))
            for kv in kvs:
                assert kv.lengths() == [wl.past + step + 1] * wl.batch
        # without storing the logits: the same tokens
        for kv in kvs:
            kv.set_lengths([wl.past + 2] * wl.batch)
        for l in range(L):
            lens[l][:] = wl.past + 2
        x = syn.normal((wl.batch, wl.hidden), 1.0, wl.cfg_id, syn.X_LAYER, 2, "cuda").to(gls[0].cfg.torch_act_dtype)
        y2, none, tokens2 = st.generate(x, logits=False, workspace=ws)
        st.check()
        assert none is None and torch.equal(tokens2, tokens) and torch.equal(y2, y)


@pytest.mark.parametrize("dt,batch", [("f16", 1), ("f16", 4), ("i8", 2)])
def test_generate_tie_takes_the_first_position(dt, batch):
    """gamma_f = 0 and beta_f = 1 make the normalized row exactly all ones, so each logit is the
    sum of its weight row: small integers, exact in any order. Rows 37, 200 and 901 tie at the
    largest sum; the token must be 37 for every sequence."""
    H = 1024 if dt == "i8" else 512   # int8 stacks take widths that are multiples of 1024
    wl = _wl(hidden=H, heads=H // 128, head_dim=128, ffn=2 * H, weight_dtype=dt, act_dtype="f16",
             group=64 if dt == "i8" else 0, batch=batch, past=5, cfg_id=406)
    gls, ows, kvs, *_ = build(wl, 1)
    V = 1024
    w = torch.zeros(V, H)
    for r in range(V):
        w[r, : r % 5] = 1.0                      # row sums 0..4
    for r in (37, 200, 901):
        w[r, :8] = 1.0                           # row sum 8: the largest
    head = {"ln_g": torch.zeros(H, dtype=torch.float16, device="cuda"),
            "ln_b": torch.ones(H, dtype=torch.float16, device="cuda")}
    if dt == "i8":
        q, s = tg.quantize_i8(w.cuda().contiguous(), 64)
        head["w"], head["s"] = q, s
        deq = oracle.dequantize_i8(q.cpu().numpy(), s.cpu().view(torch.int16).numpy().view(np.uint16), 64)
        want_sums = deq.sum(axis=1)
    else:
        head["w"] = w.half().cuda().contiguous()
        want_sums = w.double().numpy().sum(axis=1)
    assert oracle.argmax(want_sums) == 37
    x = syn.normal((batch, H), 1.0, wl.cfg_id, syn.X_LAYER, 0, "cuda").half()
    with tg.Stack(gls, kvs, max_batch=batch, head=head) as st:
        y, logits, tokens = st.generate(x)
        st.check()
    lg = logits.double().cpu().numpy()
    for b in range(batch):
        assert np.array_equal(lg[b], want_sums), np.abs(lg[b] - want_sums).max()
    assert tokens.tolist() == [37] * batch


def test_generate_requires_a_head():
    wl = _wl(hidden=512, heads=4, head_dim=128, ffn=1024, weight_dtype="f16", act_dtype="f16", batch=1, past=5,
             cfg_id=407)
    gls, ows, kvs, *_ = build(wl, 1)
    with tg.Stack(gls, kvs, max_batch=1) as st:
        x = torch.zeros((1, wl.hidden), dtype=torch.float16, device="cuda")
        with pytest.raises(ValueError):
            st.generate(x)
        tok = torch.zeros(4, dtype=torch.int32, device="cuda")
        rc = tg._lib.lib().ds_stack_forward_generate(st._handle(), tg._lib.ptr(x), tg._lib.ptr(x), None,
                                                      tg._lib.ptr(tok), 1, tg._lib.ptr(x), 16, None)
        assert rc == tg._lib.DS_ERR_UNSUPPORTED
