"""GPU parity of the persistent multi-layer decode (ds_stack_*) against the oracle.

Every layer of the stack is checked through the oracle run layer by layer on the same seeded
inputs; consecutive steps check that the cache lengths and new rows carry over between launches.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
import transformer_gpt_layer_amd as tg
from tests._common import TOL, filled_caches, gpu_layer_and_oracle_weights, rel_l2

pytestmark = pytest.mark.gpu


def _wl(base, **kw):
    return dataclasses.replace(syn.WORKLOADS[base] if isinstance(base, str) else base, **kw)


def build(wl, layers, past=None, batch=None):
    B = wl.batch if batch is None else batch
    gls, ows, kvs, oks, ovs, lens = [], [], [], [], [], []
    for l in range(layers):
        gl, ow = gpu_layer_and_oracle_weights(wl, l)
        kv, ok, ov, ln = filled_caches(wl, l, gl, past=past, batch=B)
        gls.append(gl); ows.append(ow); kvs.append(kv); oks.append(ok); ovs.append(ov); lens.append(ln)
    return gls, ows, kvs, oks, ovs, lens


def oracle_step(wl, ows, oks, ovs, lens, x):
    desc = oracle.Desc(wl.hidden, wl.heads, wl.head_dim, wl.ffn)
    h = x[:, None, :]
    for l in range(len(ows)):
        h = oracle.layer_forward(desc, ows[l], oks[l], ovs[l], lens[l], h)
    return h[:, 0]


CASES = {
    "f16-d128-b1-L3": (_wl("c1", hidden=512, heads=4, head_dim=128, ffn=2048, weight_dtype="f16", act_dtype="f16",
                           batch=1, past=45, cfg_id=201), 3),
    "f16-d64-b3-L2": (_wl("c1", hidden=1024, heads=16, head_dim=64, ffn=1536, weight_dtype="f16", act_dtype="f16",
                          batch=3, past=70, cfg_id=202), 2),
    "i8-d128-b2-L2": (_wl("c1", hidden=1024, heads=8, head_dim=128, ffn=3072, weight_dtype="i8", act_dtype="f16",
                          group=64, batch=2, past=33, cfg_id=203), 2),
    "f32-d64-b1-L2": (_wl("c1", cfg_id=204), 2),
}


@pytest.mark.parametrize("name", list(CASES))
def test_stack_decode_matches_oracle(name):
    wl, L = CASES[name]
    print(f"[stack parity] {name}: {wl} layers={L}", flush=True)
    gls, ows, kvs, oks, ovs, lens = build(wl, L)
    st = tg.Stack(gls, kvs, max_batch=wl.batch)
    print(f"  workgroups {st.groups}", flush=True)
    ws = st.workspace(wl.batch)
    for step in range(3):
        x = syn.normal((wl.batch, wl.hidden), 1.0, wl.cfg_id, syn.X_LAYER, step, "cuda").to(gls[0].cfg.torch_act_dtype)
        y = st.decode(x, workspace=ws)
        st.check()
        yo = oracle_step(wl, ows, oks, ovs, lens, x.double().cpu().numpy())
        err = rel_l2(y.double().cpu().numpy(), yo)
        print(f"  step {step}: rel L2 {err:.3e}", flush=True)
        assert err <= TOL[wl.act_dtype], (step, err)
        for l in range(L):
            assert kvs[l].lengths() == [wl.past + step + 1] * wl.batch
            P = wl.past + step
            assert rel_l2(kvs[l].k.double().cpu().numpy()[:, :, P], oks[l][:, :, P]) <= TOL[wl.act_dtype]
            assert rel_l2(kvs[l].v.double().cpu().numpy()[:, :, P], ovs[l][:, :, P]) <= TOL[wl.act_dtype]


def test_stack_matches_per_layer_path_and_is_deterministic():
    wl, L = CASES["f16-d64-b3-L2"]
    gls, ows, kvs, *_ = build(wl, L)
    x = syn.normal((wl.batch, wl.hidden), 1.0, wl.cfg_id, syn.X_LAYER, 9, "cuda").half()
    st = tg.Stack(gls, kvs, max_batch=wl.batch)
    y1 = st.decode(x)
    st.check()
    for kv in kvs:
        kv.set_lengths([wl.past] * wl.batch)
    y2 = st.decode(x)
    st.check()
    assert torch.equal(y1, y2), "persistent decode is not run-to-run deterministic"
    for kv in kvs:
        kv.set_lengths([wl.past] * wl.batch)
    h = x
    for l in range(L):
        h = gls[l].decode(kvs[l], h)
    torch.cuda.synchronize()
    assert rel_l2(y1.double().cpu().numpy(), h.double().cpu().numpy()) <= 2e-3


def test_stack_barrier_timeout_is_reported_and_recovers():
    # a 1 us barrier limit makes the waits expire: every workgroup leaves the launch, the error is
    # reported once, the state is reset, and the next step with the normal limit is correct
    wl, L = CASES["f16-d128-b1-L3"]
    gls, ows, kvs, oks, ovs, lens = build(wl, L)
    st = tg.Stack(gls, kvs, max_batch=1)
    x = syn.normal((1, wl.hidden), 1.0, wl.cfg_id, syn.X_LAYER, 0, "cuda").half()
    st.set_timeout_us(1)
    st.decode(x)
    with pytest.raises(RuntimeError, match="timed out"):
        st.check()
    st.set_timeout_us(2_000_000)
    for l, kv in enumerate(kvs):
        kv.set_lengths([wl.past])
    y = st.decode(x)
    st.check()
    yo = oracle_step(wl, ows, oks, ovs, lens, x.double().cpu().numpy())
    assert rel_l2(y.double().cpu().numpy(), yo) <= TOL["f16"]


def test_stack_kv_full_raises():
    wl, L = CASES["f16-d128-b1-L3"]
    gls, ows, kvs, *_ = build(wl, 1, past=wl.capacity - 1)
    st = tg.Stack(gls, kvs, max_batch=1)
    x = torch.zeros((1, wl.hidden), dtype=torch.float16, device="cuda")
    st.decode(x)
    st.check()
    with pytest.raises(OverflowError):
        st.decode(x)
