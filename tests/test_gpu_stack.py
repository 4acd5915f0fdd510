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
from tests._common import TOL, TORCH, filled_caches, gpu_layer_and_oracle_weights, kv8_caches, rel_l2

pytestmark = pytest.mark.gpu


def _wl(base, **kw):
    return dataclasses.replace(syn.WORKLOADS[base] if isinstance(base, str) else base, **kw)


def build(wl, layers, past=None, batch=None, gelu_tanh=False, cap=None, kv8=False):
    B = wl.batch if batch is None else batch
    gls, ows, kvs, oks, ovs, lens = [], [], [], [], [], []
    for l in range(layers):
        if kv8:
            gl, ow = gpu_layer_and_oracle_weights(wl, l, gelu_tanh=gelu_tanh, kv_dtype="int8")
            kv, ok, ov, ln = kv8_caches(wl, l, gl, past=past, batch=B, cap=cap)
        else:
            gl, ow = gpu_layer_and_oracle_weights(wl, l, gelu_tanh=gelu_tanh)
            kv, ok, ov, ln = filled_caches(wl, l, gl, past=past, batch=B, cap=cap)
        gls.append(gl); ows.append(ow); kvs.append(kv); oks.append(ok); ovs.append(ov); lens.append(ln)
    return gls, ows, kvs, oks, ovs, lens


def oracle_step(wl, ows, oks, ovs, lens, x, gelu_tanh=False, kv8=False):
    desc = oracle.Desc(wl.hidden, wl.heads, wl.head_dim, wl.ffn, gelu_tanh=gelu_tanh, kv_int8=kv8)
    h = x[:, None, :]
    for l in range(len(ows)):
        h = oracle.layer_forward(desc, ows[l], oks[l], ovs[l], lens[l], h)
    return h[:, 0]


AFFINE = dict(ln_std=0.2, bias_std=0.1)
# (workload, layers, gelu_tanh). The affine cases draw LayerNorm gamma ~ 1 + N(0, 0.2), beta ~
# N(0, 0.2) and biases ~ N(0, 0.1) per layer, so that reading another layer's or the other
# LayerNorm's parameters (the stack fetches them per layer and phase) changes the result.
CASES = {
    "f16-d128-b1-L3": (_wl("c1", hidden=512, heads=4, head_dim=128, ffn=2048, weight_dtype="f16", act_dtype="f16",
                           batch=1, past=45, cfg_id=201), 3, False),
    "f16-d64-b3-L2": (_wl("c1", hidden=1024, heads=16, head_dim=64, ffn=1536, weight_dtype="f16", act_dtype="f16",
                          batch=3, past=70, cfg_id=202), 2, False),
    "i8-d128-b2-L2": (_wl("c1", hidden=1024, heads=8, head_dim=128, ffn=3072, weight_dtype="i8", act_dtype="f16",
                          group=64, batch=2, past=33, cfg_id=203), 2, False),
    "f32-d64-b1-L2": (_wl("c1", cfg_id=204), 2, False),
    "f16-d128-b1-L3-affine": (_wl("c1", hidden=512, heads=4, head_dim=128, ffn=2048, weight_dtype="f16",
                                  act_dtype="f16", batch=1, past=45, cfg_id=211, **AFFINE), 3, False),
    "f16-d64-b4-L3-affine-tanh": (_wl("c1", hidden=1024, heads=16, head_dim=64, ffn=1536, weight_dtype="f16",
                                      act_dtype="f16", batch=4, past=70, cfg_id=212, **AFFINE), 3, True),
    "i8-d128-b1-L3-affine-tanh": (_wl("c1", hidden=1024, heads=8, head_dim=128, ffn=3072, weight_dtype="i8",
                                      act_dtype="f16", group=64, batch=1, past=33, cfg_id=213, **AFFINE), 3, True),
    "i8-d128-b3-L3-affine": (_wl("c1", hidden=1024, heads=8, head_dim=128, ffn=2048, weight_dtype="i8",
                                 act_dtype="f16", group=64, batch=3, past=65, cfg_id=214, **AFFINE), 3, False),
    "f32-d64-b1-L3-affine-tanh": (_wl("c1", cfg_id=215, **AFFINE), 3, True),
    # bf16 weights and activations: one batch row with the LayerNorm in registers, two rows
    # through LDS with groups of five slices, and the four-row tile at head_dim 64
    "bf16-d128-b1-L3-affine-tanh": (_wl("c1", hidden=512, heads=4, head_dim=128, ffn=2048, weight_dtype="bf16",
                                        act_dtype="bf16", batch=1, past=45, cfg_id=224, **AFFINE), 3, True),
    "bf16-d128-b2-L2-g5": (_wl("c1", hidden=2560, heads=20, head_dim=128, ffn=5120, weight_dtype="bf16",
                               act_dtype="bf16", batch=2, past=70, cfg_id=225, **AFFINE), 2, False),
    "bf16-d64-b4-L2": (_wl("c1", hidden=1024, heads=16, head_dim=64, ffn=1536, weight_dtype="bf16",
                           act_dtype="bf16", batch=4, past=33, cfg_id=226, **AFFINE), 2, False),
    # int8 with a finer MLP group (mlp_extra_grouping) and with groups of 32 throughout
    "i8-d128-b1-L2-g64-mlp32": (_wl("c1", hidden=1024, heads=8, head_dim=128, ffn=2048, weight_dtype="i8",
                                    act_dtype="f16", group=64, group_mlp=32, batch=1, past=50, cfg_id=222, **AFFINE),
                                2, False),
    "i8-d128-b3-L2-g32": (_wl("c1", hidden=1024, heads=8, head_dim=128, ffn=3072, weight_dtype="i8",
                              act_dtype="f16", group=32, batch=3, past=20, cfg_id=223, **AFFINE), 2, True),
    # widths whose rows hold a multiple of 5 slices: the workers consume groups of 5 slices
    "f16-d128-b2-L3-g5": (_wl("c1", hidden=2560, heads=20, head_dim=128, ffn=5120, weight_dtype="f16",
                              act_dtype="f16", batch=2, past=70, cfg_id=217, **AFFINE), 3, True),
    "f16-d128-b1-L2-g5": (_wl("c1", hidden=2560, heads=20, head_dim=128, ffn=2560, weight_dtype="f16",
                              act_dtype="f16", batch=1, past=130, cfg_id=218, **AFFINE), 2, False),
    "i8-d128-b1-L2-g5": (_wl("c1", hidden=5120, heads=40, head_dim=128, ffn=5120, weight_dtype="i8",
                             act_dtype="f16", group=64, batch=1, past=33, cfg_id=219, **AFFINE), 2, False),
    "f32-d128-b1-L2-g5": (_wl("c1", hidden=1280, heads=10, head_dim=128, ffn=2560, weight_dtype="f32",
                              act_dtype="f32", batch=1, past=20, cfg_id=220, **AFFINE), 2, True),
    # more attention items than workgroups (several per workgroup): each later item's rows arrive
    # through the LDS prefetch; fp16 at head_dim 128 over two sequences, bf16 at head_dim 64
    "f16-d128-b2-L2-long": (_wl("c1", hidden=2560, heads=20, head_dim=128, ffn=5120, weight_dtype="f16",
                                act_dtype="f16", batch=2, past=900, cfg_id=227, **AFFINE), 2, False),
    "bf16-d64-b1-L2-long": (_wl("c1", hidden=1024, heads=16, head_dim=64, ffn=2048, weight_dtype="bf16",
                                act_dtype="bf16", batch=1, past=1100, cfg_id=228, **AFFINE), 2, True),
    "i8-d128-b1-L2-long": (_wl("c1", hidden=5120, heads=40, head_dim=128, ffn=5120, weight_dtype="i8",
                               act_dtype="f16", group=64, batch=1, past=700, cfg_id=229, **AFFINE), 2, False),
}


@pytest.mark.parametrize("name", list(CASES))
def test_stack_decode_matches_oracle(name):
    wl, L, tanh = CASES[name]
    print(f"[stack parity] {name}: {wl} layers={L} gelu_tanh={tanh}", flush=True)
    gls, ows, kvs, oks, ovs, lens = build(wl, L, gelu_tanh=tanh)
    with tg.Stack(gls, kvs, max_batch=wl.batch) as st:
        print(f"  workgroups {st.groups}", flush=True)
        ws = st.workspace(wl.batch)
        for step in range(3):
            x = syn.normal((wl.batch, wl.hidden), 1.0, wl.cfg_id, syn.X_LAYER, step, "cuda").to(gls[0].cfg.torch_act_dtype)
            y = st.decode(x, workspace=ws)
            st.check()
            xd = x.double().cpu().numpy()
            yo = oracle_step(wl, ows, oks, ovs, lens, xd, gelu_tanh=tanh)
            yd = y.double().cpu().numpy()
            err, err_d = rel_l2(yd, yo), rel_l2(yd - xd, yo - xd)
            print(f"  step {step}: rel L2 {err:.3e}, of y - x {err_d:.3e}", flush=True)
            assert err <= TOL[wl.act_dtype] and err_d <= TOL[wl.act_dtype], (step, err, err_d)
            for l in range(L):
                assert kvs[l].lengths() == [wl.past + step + 1] * wl.batch
                P = wl.past + step
                assert rel_l2(kvs[l].k.double().cpu().numpy()[:, :, P], oks[l][:, :, P]) <= TOL[wl.act_dtype]
                assert rel_l2(kvs[l].v.double().cpu().numpy()[:, :, P], ovs[l][:, :, P]) <= TOL[wl.act_dtype]


# int8 KV caches (one fp16 scale per cached row of one head): the attention item that holds a
# sequence's new row quantizes it and writes the cache. Past lengths 63 and 127 put the new rows
# of consecutive steps on both sides of a chunk boundary.
KV8_CASES = {
    "f16-d128-b1-L3-affine-kv8": (_wl("c1", hidden=512, heads=4, head_dim=128, ffn=2048, weight_dtype="f16",
                                      act_dtype="f16", batch=1, past=63, cfg_id=231, **AFFINE), 3, False),
    "i8-d64-b3-L2-tanh-kv8": (_wl("c1", hidden=1024, heads=16, head_dim=64, ffn=2048, weight_dtype="i8",
                                  act_dtype="f16", group=64, batch=3, past=70, cfg_id=232, **AFFINE), 2, True),
    "f16-d128-b2-L2-g5-kv8": (_wl("c1", hidden=2560, heads=20, head_dim=128, ffn=5120, weight_dtype="f16",
                                  act_dtype="f16", batch=2, past=127, cfg_id=233, **AFFINE), 2, False),
    "i8-d128-b1-L2-g5-kv8": (_wl("c1", hidden=5120, heads=40, head_dim=128, ffn=5120, weight_dtype="i8",
                                 act_dtype="f16", group=64, batch=1, past=5, cfg_id=234, **AFFINE), 2, False),
    # bf16 weights and activations over int8 caches
    "bf16-d64-b3-L2-tanh-kv8": (_wl("c1", hidden=1024, heads=16, head_dim=64, ffn=2048, weight_dtype="bf16",
                                    act_dtype="bf16", batch=3, past=41, cfg_id=236, **AFFINE), 2, True),
    "bf16-d128-b1-L2-g5-kv8": (_wl("c1", hidden=2560, heads=20, head_dim=128, ffn=5120, weight_dtype="bf16",
                                   act_dtype="bf16", batch=1, past=90, cfg_id=237, **AFFINE), 2, False),
}


@pytest.mark.parametrize("name", list(KV8_CASES))
def test_stack_decode_with_int8_kv_matches_oracle(name):
    wl, L, tanh = KV8_CASES[name]
    print(f"[stack int8 kv parity] {name}: {wl} layers={L} gelu_tanh={tanh}", flush=True)
    gls, ows, kvs, oks, ovs, lens = build(wl, L, gelu_tanh=tanh, kv8=True)
    with tg.Stack(gls, kvs, max_batch=wl.batch) as st:
        ws = st.workspace(wl.batch)
        for step in range(3):
            x = syn.normal((wl.batch, wl.hidden), 1.0, wl.cfg_id, syn.X_LAYER, step, "cuda").to(TORCH[wl.act_dtype])
            y = st.decode(x, workspace=ws)
            st.check()
            xd = x.double().cpu().numpy()
            yo = oracle_step(wl, ows, oks, ovs, lens, xd, gelu_tanh=tanh, kv8=True)
            yd = y.double().cpu().numpy()
            err, err_d = rel_l2(yd, yo), rel_l2(yd - xd, yo - xd)
            P = wl.past + step
            news = []
            for l in range(L):
                assert kvs[l].lengths() == [P + 1] * wl.batch
                kd, vd = kvs[l].dequantized()
                news.append(rel_l2(kd[:, :, P].double().cpu().numpy(), oks[l][:, :, P]))
                news.append(rel_l2(vd[:, :, P].double().cpu().numpy(), ovs[l][:, :, P]))
                codes = torch.cat([kvs[l].k[:, :, P], kvs[l].v[:, :, P]], 1).cpu().numpy().astype(int)
                assert np.all(np.abs(codes).max(-1) == 127), "a new row's codes do not reach 127"
            print(f"  step {step}: rel L2 {err:.3e}, of y - x {err_d:.3e}; new rows worst {max(news):.3e}", flush=True)
            tol = TOL[wl.act_dtype]
            assert err <= tol and err_d <= tol and max(news) <= tol, (step, err, err_d, news)


def test_stack_with_int8_kv_matches_the_per_layer_path():
    """The stack and the per-layer path on the same int8 caches: the same codes for rows whose
    quantization is not a near tie, and outputs within the activation type's rounding."""
    wl = _wl("c1", hidden=1024, heads=8, head_dim=128, ffn=2048, weight_dtype="f16", act_dtype="f16", batch=2,
             past=40, cfg_id=235, **AFFINE)
    L = 2
    gls, ows, kvs, oks, ovs, lens = build(wl, L, kv8=True)
    _, _, kvs2, _, _, _ = build(wl, L, kv8=True)
    x = syn.normal((wl.batch, wl.hidden), 1.0, wl.cfg_id, syn.X_LAYER, 0, "cuda").half()
    with tg.Stack(gls, kvs, max_batch=wl.batch) as st:
        y = st.decode(x)
        st.check()
    h = x
    for l in range(L):
        h = gls[l].decode(kvs2[l], h)
    torch.cuda.synchronize()
    err = rel_l2(y.double().cpu().numpy(), h.double().cpu().numpy())
    print(f"  stack vs per-layer: rel L2 {err:.3e}", flush=True)
    assert err <= 2e-3
    for l in range(L):
        for a, b in ((kvs[l].k, kvs2[l].k), (kvs[l].v, kvs2[l].v)):
            d = (a[:, :, wl.past].int() - b[:, :, wl.past].int()).abs()
            assert int(d.max()) <= 1 and float((d > 0).float().mean()) < 0.05
        assert torch.equal(kvs[l].k[:, :, :wl.past], kvs2[l].k[:, :, :wl.past])


def test_stack_ragged_lengths_in_a_large_cache():
    """Sequences of lengths 150, 40 and 1 in caches of 2048 rows: the attention items cover the
    chunks that hold keys of the longest sequence only, and the shorter sequences skip the chunks
    past their own keys."""
    wl = _wl("c1", hidden=1024, heads=8, head_dim=128, ffn=2048, weight_dtype="f16", act_dtype="f16", batch=3,
             past=150, cfg_id=221, **AFFINE)
    L, want = 2, [150, 40, 1]
    gls, ows, kvs, oks, ovs, lens = build(wl, L, cap=2048)
    for kv, ln in zip(kvs, lens):
        kv.set_lengths(want)
        ln[:] = want
    with tg.Stack(gls, kvs, max_batch=wl.batch) as st:
        ws = st.workspace(wl.batch)
        for step in range(2):
            x = syn.normal((wl.batch, wl.hidden), 1.0, wl.cfg_id, syn.X_LAYER, step, "cuda").half()
            y = st.decode(x, workspace=ws)
            st.check()
            yo = oracle_step(wl, ows, oks, ovs, lens, x.double().cpu().numpy())
            yd = y.double().cpu().numpy()
            for b in range(wl.batch):
                err = rel_l2(yd[b], yo[b])
                print(f"  step {step} sequence {b} (length {want[b] + step}): rel L2 {err:.3e}", flush=True)
                assert err <= TOL["f16"], (step, b, err)
            for l in range(L):
                assert kvs[l].lengths() == [n + step + 1 for n in want]


@pytest.mark.parametrize("dt,batch", [("f16", 1), ("f16", 3), ("f32", 1)])
def test_stack_single_key_is_exactly_the_value_row(dt, batch):
    """One layer, empty cache, W_o = I and a zero MLP: the persistent step gives y = x + v exactly,
    v being the value row it wrote into the cache (softmax weight exactly 1)."""
    from tests.test_gpu_parity import single_key_layer
    wl = _wl("c1", hidden=512, heads=4, head_dim=128, ffn=1024, weight_dtype=dt, act_dtype=dt, batch=batch,
             past=0, cfg_id=216, ln_std=0.2)
    gl = single_key_layer(wl)
    act = gl.cfg.torch_act_dtype
    kv = tg.KVCache(batch, wl.heads, 64, wl.head_dim, act, "cuda")
    x = syn.normal((batch, wl.hidden), 1.0, wl.cfg_id, syn.X_LAYER, 1, "cuda").to(act)
    with tg.Stack([gl], [kv], max_batch=batch) as st:
        y = st.decode(x)
        st.check()
    v = kv.v[:, :, 0].reshape(batch, wl.hidden)
    want = (x.float() + v.float()).to(act)
    assert torch.count_nonzero(v) > 0
    assert torch.equal(y, want), (y.float() - want.float()).abs().max().item()


def test_stack_matches_per_layer_path_and_is_deterministic():
    wl, L, _ = CASES["f16-d64-b3-L2"]
    gls, ows, kvs, *_ = build(wl, L)
    x = syn.normal((wl.batch, wl.hidden), 1.0, wl.cfg_id, syn.X_LAYER, 9, "cuda").half()
    st = tg.Stack(gls, kvs, max_batch=wl.batch)
    y1 = st.decode(x)
    st.check()
    for kv in kvs:
        kv.set_lengths([wl.past] * wl.batch)
    y2 = st.decode(x)
    st.check()
    st.close()
    assert torch.equal(y1, y2), "persistent decode is not run-to-run deterministic"
    for kv in kvs:
        kv.set_lengths([wl.past] * wl.batch)
    h = x
    for l in range(L):
        h = gls[l].decode(kvs[l], h)
    torch.cuda.synchronize()
    assert rel_l2(y1.double().cpu().numpy(), h.double().cpu().numpy()) <= 2e-3


def test_stack_barrier_timeout_is_reported_and_recovers():
    # a 1 us limit on the kernel's own bounded waits makes them expire: every workgroup leaves the
    # launch and the error is reported. A step enqueued before the check leaves at once (the error
    # flag is still raised) and changes nothing. The check resets the state and hands the host
    # length mirrors the device's lengths, and the next step with the normal limit is correct.
    wl, L, _ = CASES["f16-d128-b1-L3"]
    gls, ows, kvs, oks, ovs, lens = build(wl, L)
    st = tg.Stack(gls, kvs, max_batch=1)
    x = syn.normal((1, wl.hidden), 1.0, wl.cfg_id, syn.X_LAYER, 0, "cuda").half()
    st.set_timeout_us(1)
    st.decode(x)
    st.set_timeout_us(2_000_000)
    sentinel = torch.full_like(x, 7.0)
    y_skip = st.decode(x, y=sentinel.clone())
    torch.cuda.synchronize()
    assert torch.equal(y_skip, sentinel), "a launch after an unreported timeout must store nothing"
    assert [list(kv.h_len) for kv in kvs] == [[wl.past + 2]] * L   # advanced at enqueue
    with pytest.raises(RuntimeError, match="timed out"):
        st.check()
    for kv in kvs:
        assert kv.lengths() == [wl.past] and list(kv.h_len) == [wl.past]
    y = st.decode(x)
    st.check()
    st.close()
    yo = oracle_step(wl, ows, oks, ovs, lens, x.double().cpu().numpy())
    assert rel_l2(y.double().cpu().numpy(), yo) <= TOL["f16"]


def test_stack_kv_full_raises():
    wl, L, _ = CASES["f16-d128-b1-L3"]
    gls, ows, kvs, *_ = build(wl, 1, past=wl.capacity - 1)
    with tg.Stack(gls, kvs, max_batch=1) as st:
        x = torch.zeros((1, wl.hidden), dtype=torch.float16, device="cuda")
        st.decode(x)
        st.check()
        with pytest.raises(OverflowError):
            st.decode(x)


def test_two_stacks_sharing_one_workspace():
    """Two stacks on one workspace, alternating: the workspace is cleared when its user changes, so
    no value of one stack's launches can pass as the other's. Each result equals that stack's
    result on a workspace of its own."""
    wl, L, _ = CASES["f16-d64-b3-L2"]
    a = build(wl, L)
    b = build(_wl(wl, cfg_id=222), L)
    sa = tg.Stack(a[0], a[2], max_batch=wl.batch)
    sb = tg.Stack(b[0], b[2], max_batch=wl.batch)
    shared = sa.workspace(wl.batch)
    x = syn.normal((wl.batch, wl.hidden), 1.0, wl.cfg_id, syn.X_LAYER, 4, "cuda").half()
    outs = []
    for st, parts in ((sa, a), (sb, b), (sa, a), (sb, b)):
        for kv in parts[2]:
            kv.set_lengths([wl.past] * wl.batch)
        outs.append(st.decode(x, workspace=shared))
        st.check()
    for st, parts, y in ((sa, a, outs[2]), (sb, b, outs[3])):
        for kv in parts[2]:
            kv.set_lengths([wl.past] * wl.batch)
        ref = st.decode(x, workspace=st.workspace(wl.batch))
        st.check()
        assert torch.equal(y, ref)
    assert torch.equal(outs[0], outs[2]) and torch.equal(outs[1], outs[3])
    assert not torch.equal(outs[0], outs[1])
    sa.close()
    sb.close()
