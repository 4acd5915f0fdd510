"""Decode throughput of the fused GPT-layer stack on one MI355X (and, with --config c5, prefill).

One step = one decode token for every sequence of the batch through all L layers of the stack
(LN1+QKV, attention over the KV cache, output projection, LN2+FF1+GeLU, FF2), starting from the
same cache lengths each step. Weights and caches are seeded synthetic tensors resident in HBM
(distinct per layer, so weights stream from HBM rather than the 256 MB last-level cache).

Prints one JSON line: decode tokens/s and the achieved HBM GB/s per layer step (against the
8 TB/s peak), the roofline entry of the dominant kernel, and the CPU oracle's throughput on a
bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0

# HBM traffic of a kernel as counted by rocprofv3 (FETCH_SIZE and WRITE_SIZE, each scaled by what
# the same counter reads for a copy of known size) is recorded in a profile summary together with
# the SHA-256 of the kernel's source file; the figure is reported only while that source is
# unchanged.
TRAFFIC_RECORDS = {
    "stack_decode_kernel": ("profiles/stack_decode_kernel_c2_f16_b1.md",
                            ("transformer_gpt_layer_amd/csrc/kernels_stack.hip", "transformer_gpt_layer_amd/csrc/ds_stack.hpp")),
}


def measured_traffic(kernel: str, workload: str):
    import hashlib
    import re

    if kernel not in TRAFFIC_RECORDS:
        return None
    summary, sources = TRAFFIC_RECORDS[kernel]
    summary = os.path.join(ROOT, summary)
    sources = [os.path.join(ROOT, p) for p in sources]
    if not (os.path.exists(summary) and all(os.path.exists(p) for p in sources)):
        return None
    # the record holds for exactly these kernel sources (the files concatenated, in this order)
    digest = hashlib.sha256(b"".join(open(p, "rb").read() for p in sources)).hexdigest()
    for line in open(summary):
        m = re.match(r"traffic-record: (\{.*\})\s*$", line.strip())
        if m:
            rec = json.loads(m.group(1))
            if rec.get("workload") == workload and rec.get("source_sha256") == digest:
                return int(rec["hbm_bytes_per_launch"])
    return None


def read_probe_gbs(torch, tg, gib=2, reps=5):
    """HBM read bandwidth this device reaches: the library's streaming read of a 2 GiB buffer,
    best of a few launches timed with events on the current stream."""
    buf = torch.empty(gib << 30, dtype=torch.uint8, device="cuda")
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    tg.read_probe(buf, out)
    torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        tg.read_probe(buf, out)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    del buf
    return (gib << 30) / (best * 1e-3) / 1e9


def step_stats(times_ms):
    """Median, p10 and p90 of per-step times (ms)."""
    t = sorted(times_ms)
    pick = lambda q: t[min(len(t) - 1, max(0, int(round(q * (len(t) - 1)))))]
    return {"median": round(pick(0.5), 4), "p10": round(pick(0.1), 4), "p90": round(pick(0.9), 4)}


def copy_calibration(torch, gib: int = 1):
    """Three plain device-to-device copies of `gib` GiB (torch's copy kernel): the reference whose
    FETCH_SIZE / WRITE_SIZE counters scale the kernels' counters to bytes."""
    n = (gib << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read_per_copy": n * 4, "bytes_written_per_copy": n * 4, "copies": 3}))


def algorithmic_bytes_per_layer(wl) -> dict:
    """Bytes one layer step must move at least once (weights and scales, biases and LayerNorm
    vectors, the past K/V rows read, the new K/V rows written, x read and y written)."""
    H, F, B, P, T = wl.hidden, wl.ffn, wl.batch, wl.past, wl.seq
    a = 4 if wl.act_dtype == "f32" else 2
    nw = 3 * H * H + H * H + 2 * H * F
    if wl.weight_dtype == "i8":
        wbytes = nw + (nw // wl.group) * 2
    else:
        wbytes = nw * (4 if wl.weight_dtype == "f32" else 2)
    small = (3 * H + H + F + H + 4 * H) * a
    kv_read = 2 * B * P * H * a
    kv_write = 2 * B * T * H * a
    xy = 2 * B * T * H * a
    return {"weights": wbytes, "small": small, "kv_read": kv_read, "kv_write": kv_write, "xy": xy,
            "total": wbytes + small + kv_read + kv_write + xy}


def build_stack(wl, torch, tg, syn, layers):
    """Device weights, caches (P seeded rows each) and one shared workspace."""
    dev = "cuda"
    act = torch.float32 if wl.act_dtype == "f32" else torch.float16
    cfg = tg.make_config(hidden=wl.hidden, heads=wl.heads, ffn=wl.ffn,
                         dtype={"f32": "fp32", "f16": "fp16", "i8": "int8"}[wl.weight_dtype],
                         quant_group=wl.group if wl.weight_dtype == "i8" else None)
    stack, kvs = [], []
    lens = torch.zeros((layers, wl.batch), dtype=torch.int32, device=dev)
    for l in range(layers):
        w32 = syn.layer_weights_f32(wl, l, dev)
        gw = {}
        for name, t in w32.items():
            if name.startswith("w_") and wl.weight_dtype == "i8":
                q, s = tg.quantize_i8(t.contiguous(), wl.group)
                gw[name], gw["s" + name[1:]] = q, s
            else:
                gw[name] = t.to(act).contiguous()
        del w32
        layer = tg.Layer(cfg, gw)
        kv = tg.KVCache(wl.batch, wl.heads, wl.capacity, wl.head_dim, act, dev, track_host=False)
        kv.d_len = lens[l]  # one [L, B] tensor so one fill resets every layer
        if wl.past:
            kp, vp = syn.past_kv_f32(wl, l, dev)
            to_rows = lambda t: t.permute(0, 2, 1, 3).reshape(wl.batch, wl.past, wl.hidden).to(act).contiguous()
            layer.kv_append(kv, to_rows(kp), to_rows(vp))
            del kp, vp
        stack.append(layer)
        kvs.append(kv)
    torch.cuda.synchronize()
    ws = stack[0].workspace(wl.batch, 1, wl.capacity)
    return stack, kvs, lens, ws, act


PEAK_F16_TFLOPS = 2500.0


def prefill_flops_per_layer(wl) -> dict:
    """Algorithmic FLOPs of one prefill layer step: the four weight GEMMs (2 M N K each, M = B S)
    and causal attention (QK^T and PV over the visible keys only: S (S+1) / 2 per sequence and
    head, 2 d FLOPs each for the two products)."""
    H, F, B, S, nh, d = wl.hidden, wl.ffn, wl.batch, wl.seq, wl.heads, wl.head_dim
    M = B * S
    g = {"qkv": 2 * M * 3 * H * H, "o": 2 * M * H * H, "ff1": 2 * M * F * H, "ff2": 2 * M * H * F}
    attn = 2 * 2 * d * nh * B * (S * (S + 1) // 2)
    return {**g, "attention": attn, "gemm_total": sum(g.values()), "total": sum(g.values()) + attn}


def _oracle_weights(layer, wl):
    import numpy as np
    import torch

    import oracle

    w = {}
    for n in ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_o", "b_o", "ln2_g", "ln2_b", "w_ff1", "b_ff1", "w_ff2", "b_ff2"):
        t = layer._weights[n]
        if n.startswith("w_") and wl.weight_dtype == "i8":
            s = layer._weights["s" + n[1:]]
            w[n] = oracle.dequantize_i8(t.cpu().numpy(), s.cpu().view(torch.int16).numpy().view(np.uint16), wl.group)
        else:
            w[n] = t.double().cpu().numpy()
    return w


def cpu_baseline_prefill(wl, stack, target_rows: int = 256):
    """The oracle (plain C, double, one thread) on a bounded sample: the first target_rows prompt
    rows of one sequence through layer 0, scaled to prompt tokens/s of the full L-layer stack."""
    import numpy as np

    import oracle

    desc = oracle.Desc(wl.hidden, wl.heads, wl.head_dim, wl.ffn)
    w = _oracle_weights(stack[0], wl)
    S = min(target_rows, wl.seq)
    x = np.random.default_rng(0).standard_normal((1, S, wl.hidden))
    k = np.zeros((1, wl.heads, wl.capacity, wl.head_dim))
    v = np.zeros_like(k)
    lens = np.zeros(1, dtype=np.int32)
    t0 = time.perf_counter()
    oracle.layer_forward(desc, w, k, v, lens, x)
    spent = time.perf_counter() - t0
    return {"value": S / (spent * wl.layers), "unit": "prompt tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"the first {S} prompt rows of one sequence of {wl.name} through one layer in {spent:.1f} s "
                      f"on one host thread, scaled to the {wl.layers}-layer stack"}


def run_prefill(args, wl, torch, tg, syn):
    """C5-style workload: one step = the B x S prompt through all L layers (cache lengths reset to
    0 each step), captured once in a HIP graph and replayed."""
    layers = args.layers or wl.layers
    stack, kvs, lens, _, act = build_stack(wl, torch, tg, syn, layers)
    ws = stack[0].workspace(wl.batch, wl.seq, wl.capacity)
    x0 = syn.normal((wl.batch, wl.seq, wl.hidden), 1.0, wl.cfg_id, syn.X_LAYER, 0, "cuda").to(act)
    bufs = [torch.empty_like(x0), torch.empty_like(x0)]

    def step():
        lens.zero_()
        for l in range(layers):
            stack[l].prefill(kvs[l], x0 if l == 0 else bufs[l % 2], bufs[(l + 1) % 2], ws)

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    with torch.cuda.stream(stream):
        for _ in range(max(1, args.warmup)):
            g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    with torch.cuda.stream(stream):
        e0.record(stream)
        for i in range(args.steps):
            g.replay()
            marks[i].record(stream)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    per_step = [(e0 if i == 0 else marks[i - 1]).elapsed_time(marks[i]) for i in range(args.steps)]
    out = bufs[layers % 2]
    assert torch.isfinite(out.float()).all(), "non-finite prefill output"
    fl = prefill_flops_per_layer(wl)
    tflops = fl["total"] * layers / (ms * 1e-3) / 1e12
    gemm_tflops = fl["gemm_total"] * layers / (ms * 1e-3) / 1e12
    result = {
        "metric": "prefill prompt tokens/s + MFMA utilization (weight-GEMM FLOPs / step time / 2.5 PF)",
        "value": round(wl.batch * wl.seq / (ms * 1e-3), 1),
        "unit": "prompt tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) prompt rows)",
        "config": {"workload": wl.name, "layers": layers, "batch": wl.batch, "seq": wl.seq,
                   "hidden": wl.hidden, "heads": wl.heads, "ffn": wl.ffn,
                   "launch": "per-layer kernels (LN, 4 MFMA GEMMs, flash attention), hip-graph"},
        "flops_per_layer": fl,
        "step_ms": step_stats(per_step),
        "roofline": {"bound": "mfma", "kernel": "whole prefill step (weight GEMMs + attention)",
                     "achieved": round(tflops, 1), "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_F16_TFLOPS, 4), "traffic": None,
                     "gemm_flops_over_step_tflops": round(gemm_tflops, 1)},
    }
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline_prefill(wl, stack)
    print(json.dumps(result))


def cpu_baseline(wl, stack, kvs, target_s: float):
    """The oracle (plain C, double, one thread) on a bounded sample: whole decode layer steps of
    this workload, every layer once and then the last layer's weights again, until about target_s
    seconds of oracle time have run; scaled to tokens/s of the full L-layer stack."""
    import numpy as np
    import torch

    import oracle

    desc = oracle.Desc(wl.hidden, wl.heads, wl.head_dim, wl.ffn)
    x = np.random.default_rng(0).standard_normal((wl.batch, 1, wl.hidden))
    done, spent, w, k, v = 0, 0.0, None, None, None
    lens = np.full(wl.batch, wl.past, dtype=np.int32)
    while spent < target_s:
        if done < len(stack):
            layer, kv = stack[done], kvs[done]
            w = _oracle_weights(layer, wl)
            k = np.zeros((wl.batch, wl.heads, wl.capacity, wl.head_dim))
            v = np.zeros_like(k)
            k[:, :, :wl.past] = kv.k[:, :, :wl.past].double().cpu().numpy()
            v[:, :, :wl.past] = kv.v[:, :, :wl.past].double().cpu().numpy()
        t0 = time.perf_counter()
        # the cache and the lengths are advanced in place: every step starts from the same past
        x = oracle.layer_forward(desc, w, k.copy(), v.copy(), lens.copy(), x)
        spent += time.perf_counter() - t0
        done += 1
    per_layer = spent / done
    return {"value": wl.batch / (per_layer * wl.layers), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} decode layer steps of {wl.name} (batch {wl.batch}, {wl.past} past rows; each of the "
                      f"{min(done, len(stack))} layers once, then the last layer's weights again) in {spent:.1f} s "
                      f"on one host thread, scaled to the {wl.layers}-layer stack"}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c2", help="workload key in synthetic.WORKLOADS (c5: prefill)")
    ap.add_argument("--layers", type=int, default=0, help="override the layer count (0: the workload's)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle sample budget (0 disables)")
    ap.add_argument("--mode", choices=["auto", "stack", "layers"], default="auto",
                    help="stack: one persistent launch per step; layers: six kernels per layer")
    ap.add_argument("--no-graph", action="store_true", help="layers mode: launch eagerly instead of a HIP graph")
    ap.add_argument("--no-read-probe", dest="read_probe", action="store_false",
                    help="skip the streaming-read measurement of the HBM bandwidth this device reaches")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run three 1 GiB device copies (the reference for HBM traffic counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import synthetic as syn
    import transformer_gpt_layer_amd as tg

    if args.copy_calibration:
        torch.cuda.set_device(0)
        return copy_calibration(torch)
    wl = syn.WORKLOADS[args.config]
    torch.cuda.set_device(0)
    if wl.seq != 1:
        return run_prefill(args, wl, torch, tg, syn)
    layers = args.layers or wl.layers
    torch.cuda.set_device(0)
    stack, kvs, lens, ws, act = build_stack(wl, torch, tg, syn, layers)
    x0 = syn.normal((wl.batch, wl.hidden), 1.0, wl.cfg_id, syn.X_LAYER, 0, "cuda").to(act)
    bufs = [torch.empty_like(x0), torch.empty_like(x0)]

    def step():
        lens.fill_(wl.past)
        for l in range(layers):
            stack[l].decode(kvs[l], x0 if l == 0 else bufs[l % 2], bufs[(l + 1) % 2], ws)

    stream = torch.cuda.Stream()
    use_stack = args.mode == "stack" or (args.mode == "auto" and wl.batch <= 4)
    kernel_ms = None
    if use_stack:
        st = tg.Stack(stack, kvs, max_batch=wl.batch)
        sws = st.workspace(wl.batch)
        out = torch.empty_like(x0)

        def launch():
            st.decode(x0, out, sws)

        with torch.cuda.stream(stream):
            for _ in range(max(1, args.warmup)):
                lens.fill_(wl.past)
                launch()
        st.check()
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            for i in range(args.steps):
                lens.fill_(wl.past)
                starts[i].record(stream)
                launch()
                ends[i].record(stream)
            e1.record(stream)
        torch.cuda.synchronize()
        st.check()
        groups = st.groups
        st.close()  # release the handle now, not during interpreter shutdown
        ms = e0.elapsed_time(e1) / args.steps
        per_step = [a.elapsed_time(b) for a, b in zip(starts, ends)]
        kernel_ms = sum(per_step) / args.steps
        launch_desc = f"persistent stack kernel, {groups} workgroups"
    else:
        def step():
            lens.fill_(wl.past)
            for l in range(layers):
                stack[l].decode(kvs[l], x0 if l == 0 else bufs[l % 2], bufs[(l + 1) % 2], ws)

        with torch.cuda.stream(stream):
            step()
        torch.cuda.synchronize()
        if args.no_graph:
            run = step
        else:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                step()
            run = g.replay
        with torch.cuda.stream(stream):
            for _ in range(args.warmup):
                run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        with torch.cuda.stream(stream):
            e0.record(stream)
            for i in range(args.steps):
                run()
                marks[i].record(stream)
            e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        per_step = [(e0 if i == 0 else marks[i - 1]).elapsed_time(marks[i]) for i in range(args.steps)]
        out = bufs[layers % 2]
        launch_desc = "per-layer kernels, " + ("eager" if args.no_graph else "hip-graph")
    assert torch.isfinite(out.float()).all(), "non-finite decode output"

    per = algorithmic_bytes_per_layer(wl)
    step_bytes = per["total"] * layers
    gbs = step_bytes / (ms * 1e-3) / 1e9
    tok_s = wl.batch / (ms * 1e-3)
    if kernel_ms is not None:
        kgbs = step_bytes / (kernel_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "kernel": "stack_decode_kernel (all layers of one step)",
                    "achieved": round(kgbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(kgbs / PEAK_HBM_GBS, 4),
                    "traffic": measured_traffic("stack_decode_kernel", wl.name) if layers == wl.layers else None,
                    "kernel_ms": round(kernel_ms, 4), "bytes_per_launch": step_bytes}
    else:
        roofline = {"bound": "hbm", "kernel": "whole decode step (per-layer kernels)",
                    "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None}
    result = {
        "metric": "decode tokens/s at batch 1/8 + achieved HBM GB/s (% of peak) per layer step",
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "f16": "f16", "i8": "i8w-f16"}[wl.weight_dtype],
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) inputs and past K/V)",
        "config": {"workload": wl.name, "layers": layers, "batch": wl.batch, "past_kv": wl.past,
                   "hidden": wl.hidden, "heads": wl.heads, "ffn": wl.ffn,
                   "launch": launch_desc},
        "hbm_gbs_per_layer_step": round(gbs, 1),
        "hbm_frac_of_peak": round(gbs / PEAK_HBM_GBS, 4),
        "bytes_per_layer_step": per,
        "step_ms": step_stats(per_step),
        "roofline": roofline,
    }
    if args.read_probe:
        probe = read_probe_gbs(torch, tg)
        result["read_probe_gbs"] = round(probe, 1)
        # the roofline kernel's achieved rate over what a plain streaming read reaches here
        result["hbm_frac_of_read_probe"] = round(roofline["achieved"] / probe, 4)
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(wl, stack, kvs, args.cpu_seconds)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
