"""The no-allocation decode entry point (ds_stack_forward_decode_static) against the entry point it
varies (ds_stack_forward_decode with a caller workspace), through the C ABI.

Two calls in a row on one stack, the second with a smaller input (fewer sequences), each compared
with the workspace entry point on the same inputs and cache state: outputs and the new cache rows
must be identical (same kernel, same arithmetic), and both match the oracle to the fp16 bar. A
second stack then runs on the same static scratch, which the library must clear for it.
"""
import dataclasses

import numpy as np
import pytest
import torch

import synthetic as syn
import transformer_gpt_layer_amd as tg
from tests._common import TOL, filled_caches, gpu_layer_and_oracle_weights, rel_l2

pytestmark = pytest.mark.gpu


def _stack(wl, layers):
    gls, ows, kvs, oks, ovs, lens = [], [], [], [], [], []
    for l in range(layers):
        gl, ow = gpu_layer_and_oracle_weights(wl, l)
        kv, ok, ov, ln = filled_caches(wl, l, gl)
        gls.append(gl); ows.append(ow); kvs.append(kv); oks.append(ok); ovs.append(ov); lens.append(ln)
    return gls, ows, kvs, oks, ovs, lens


def _reset(kvs, past, batch):
    for kv in kvs:
        kv.set_lengths([past] * batch)


def test_static_scratch_decode_matches_workspace_decode():
    import oracle
    wl = dataclasses.replace(syn.WORKLOADS["c1"], hidden=1024, heads=8, head_dim=128, ffn=2048, weight_dtype="f16",
                             act_dtype="f16", batch=3, past=50, cfg_id=301, ln_std=0.2, bias_std=0.1)
    L = 2
    gls, ows, kvs, oks, ovs, lens = _stack(wl, L)
    st = tg.Stack(gls, kvs, max_batch=wl.batch)
    assert st.workspace_bytes(wl.batch) <= tg._lib.lib().ds_stack_workspace_bytes(st._handle(), wl.batch)
    for step, batch in enumerate((3, 2)):     # the second call has fewer sequences
        x = syn.normal((batch, wl.hidden), 1.0, wl.cfg_id, syn.X_LAYER, step, "cuda").half()
        print(f"[no-alloc] call {step}: batch {batch}", flush=True)
        _reset(kvs, wl.past, wl.batch)
        y_ws = st.decode(x, workspace=st.workspace(batch))
        st.check()
        rows_ws = [(kv.k[:batch, :, wl.past].clone(), kv.v[:batch, :, wl.past].clone()) for kv in kvs]
        _reset(kvs, wl.past, wl.batch)
        y_st = torch.full_like(x, float("nan"))
        st.decode_static(x, y_st)
        st.check()
        assert torch.equal(y_st, y_ws), (y_st.float() - y_ws.float()).abs().max().item()
        for kv, (k0, v0) in zip(kvs, rows_ws):
            assert torch.equal(kv.k[:batch, :, wl.past], k0) and torch.equal(kv.v[:batch, :, wl.past], v0)
            assert kv.lengths()[:batch] == [wl.past + 1] * batch
        # and the oracle, layer after layer, on the same inputs
        desc = oracle.Desc(wl.hidden, wl.heads, wl.head_dim, wl.ffn)
        h = x.double().cpu().numpy()[:, None, :]
        for l in range(L):
            ok, ov = oks[l][:batch].copy(), ovs[l][:batch].copy()
            h = oracle.layer_forward(desc, ows[l], ok, ov, np.full(batch, wl.past, dtype=np.int32), h)
        assert rel_l2(y_st.double().cpu().numpy(), h[:, 0]) <= TOL["f16"]
    # another stack on the same static scratch: the library clears it for the new user
    wl2 = dataclasses.replace(wl, cfg_id=302)
    g2, o2, k2, *_ = _stack(wl2, L)
    st2 = tg.Stack(g2, k2, max_batch=wl2.batch)
    x = syn.normal((2, wl.hidden), 1.0, wl2.cfg_id, syn.X_LAYER, 0, "cuda").half()
    _reset(k2, wl2.past, wl2.batch)
    ref = st2.decode(x, workspace=st2.workspace(2))
    st2.check()
    _reset(k2, wl2.past, wl2.batch)
    y = torch.empty_like(x)
    st2.decode_static(x, y)
    st2.check()
    assert torch.equal(y, ref)
    st.close()
    st2.close()


def test_static_scratch_rejects_a_step_beyond_its_size():
    """A stack whose step needs more workspace than the static array is refused before any launch."""
    wl = dataclasses.replace(syn.WORKLOADS["c1"], hidden=2048, heads=32, head_dim=64, ffn=2048, weight_dtype="f16",
                             act_dtype="f16", batch=4, past=0, cfg_id=303)
    gl, _ = gpu_layer_and_oracle_weights(wl, 0)
    # a long cache makes the attention partials large: 4 x 32 heads x 256 chunks x 66 x 8 B = 17.3 MB
    kv = tg.KVCache(4, wl.heads, 16384, wl.head_dim, torch.float16, "cuda")
    with tg.Stack([gl], [kv], max_batch=4) as st:
        need = st.workspace_bytes(4)
        assert need > (16 << 20)
        y = torch.empty((4, wl.hidden), dtype=torch.float16, device="cuda")
        x = torch.zeros_like(y)
        with pytest.raises(ValueError, match="static scratch"):
            st.decode_static(x, y)
        assert kv.lengths() == [0] * 4
