"""Decode throughput of the fused GPT-layer stack on one MI355X, with nested records for the other
workloads of the metric (batch 8 fp16 and int8, int8 batch 1, the generation step with the LM head,
the headline step in bf16 and with an int8 KV cache, prefill, and the MoE expert FF).

One decode step = one new token for every sequence of the batch through all L layers of the stack
(LN1+QKV, attention over the KV cache, output projection, LN2+FF1+GeLU, FF2), starting from the
same cache lengths each step. Weights and caches are seeded synthetic tensors resident in HBM
(distinct per layer, so weights stream from HBM rather than the 256 MB last-level cache).

Prints one JSON line. Its top level is the headline workload (GPT-Neo-2.7B shapes, fp16, batch 1,
512 past rows, 32 layers): decode tokens/s, achieved HBM GB/s per layer step, the roofline entry of
the dominant kernel (timed with HIP events on the stream it runs on), and the oracle's throughput on
a bounded sample of the same workload, on one host thread and on all host cores. `records` holds the
same fields for the other workloads.
"""
import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_F16_TFLOPS = 2500.0
METRIC = "decode tokens/s at batch 1/8 + achieved HBM GB/s (% of peak) per layer step"

# HBM traffic of a kernel as counted by rocprofv3 (FETCH_SIZE and WRITE_SIZE, each scaled by what
# the same counter reads for a copy of known size) is recorded in a profile summary together with
# the SHA-256 of the kernel's source files; the figure is reported only while they are unchanged.
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


# ------------------------------------------------------------------ algorithmic work
def _sizes(wl):
    a = 4 if wl.act_dtype == "f32" else 2

    def wbytes(n, k, mlp=False):
        if wl.weight_dtype == "i8":
            g = wl.group_mlp if mlp and wl.group_mlp else wl.group
            return n * k + (n * k // g) * 2
        return n * k * (4 if wl.weight_dtype == "f32" else 2)
    return a, wbytes


def kv_row_bytes(wl) -> int:
    """Bytes of one cached position's K (or V) over all heads: the activation type, or an int8 cache's
    codes with one fp16 scale per head."""
    a, _ = _sizes(wl)
    return wl.hidden + 2 * wl.heads if wl.extra.get("kv_dtype") == "int8" else wl.hidden * a


def part_bytes(wl) -> dict:
    """Bytes each kernel of one decode layer step must move at least once: its weights (and scales),
    biases and LayerNorm vectors, the past K/V rows it reads, the new K/V rows it writes, x read by
    the first and y written by the last. Intermediates between kernels are not counted."""
    H, F, B, P, T = wl.hidden, wl.ffn, wl.batch, wl.past, wl.seq
    a, wb = _sizes(wl)
    kr = kv_row_bytes(wl)
    return {"ln1": B * T * H * a + 2 * H * a, "qkv": wb(3 * H, H) + 3 * H * a + 2 * B * T * kr,
            "attn": 2 * B * P * kr, "o": wb(H, H) + H * a, "ln2": 2 * H * a, "ff1": wb(F, H, True) + F * a,
            "ff2": wb(H, F, True) + H * a + B * T * H * a, "len": 0}


def algorithmic_bytes_per_layer(wl) -> dict:
    """Bytes one layer step must move at least once (the sum over its kernels of part_bytes)."""
    H, F, B, P, T = wl.hidden, wl.ffn, wl.batch, wl.past, wl.seq
    a, wb = _sizes(wl)
    weights = wb(3 * H, H) + wb(H, H) + wb(F, H, True) + wb(H, F, True)
    small = (3 * H + H + F + H + 4 * H) * a
    kr = kv_row_bytes(wl)
    kv_read, kv_write, xy = 2 * B * P * kr, 2 * B * T * kr, 2 * B * T * H * a
    total = weights + small + kv_read + kv_write + xy
    assert total == sum(part_bytes(wl).values())
    return {"weights": weights, "small": small, "kv_read": kv_read, "kv_write": kv_write, "xy": xy, "total": total}


def head_bytes(wl, vocab) -> int:
    """The LM head's bytes per generation step: its weight (and scales), the final LayerNorm
    vectors, the last layer's output read and the fp32 logits written."""
    a, wb = _sizes(wl)
    return wb(vocab, wl.hidden) + 2 * wl.hidden * a + wl.batch * wl.hidden * a + wl.batch * vocab * 4


def prefill_flops(wl) -> dict:
    """Algorithmic FLOPs of one prefill layer step: the four weight GEMMs (2 M N K each, M = B S)
    and causal attention (QK^T and PV over the visible keys only: S (S+1) / 2 per sequence and
    head, 2 d FLOPs each for the two products)."""
    H, F, B, S, nh, d = wl.hidden, wl.ffn, wl.batch, wl.seq, wl.heads, wl.head_dim
    M = B * S
    g = {"qkv": 2 * M * 3 * H * H, "o": 2 * M * H * H, "ff1": 2 * M * F * H, "ff2": 2 * M * H * F}
    attn = 2 * 2 * d * nh * B * (S * (S + 1) // 2)
    return {**g, "attn": attn, "gemm_total": sum(g.values()), "total": sum(g.values()) + attn}


# ------------------------------------------------------------------ building a stack
def dtype_label(wl) -> str:
    """The arithmetic types of a workload: weights (int8 with fp16 activations), cache, MLP groups."""
    dtype = {"f32": "f32", "f16": "f16", "i8": "i8w-f16", "bf16": "bf16"}[wl.weight_dtype]
    if wl.extra.get("kv_dtype") == "int8":
        dtype += "-kv8"
    if wl.weight_dtype == "i8" and wl.group_mlp:
        dtype += f"-mlpg{wl.group_mlp}"
    return dtype


def build_stack(wl, torch, tg, syn, layers):
    """Device weights and caches (P seeded rows each) for every layer, one [L, B] length tensor."""
    dev = "cuda"
    act = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[wl.act_dtype]
    kv8 = wl.extra.get("kv_dtype") == "int8"
    cfg = tg.make_config(hidden=wl.hidden, heads=wl.heads, ffn=wl.ffn,
                         dtype={"f32": "fp32", "f16": "fp16", "i8": "int8", "bf16": "bf16"}[wl.weight_dtype],
                         quant_group=wl.group if wl.weight_dtype == "i8" else None,
                         quant_group_mlp=wl.group_mlp if wl.weight_dtype == "i8" and wl.group_mlp else None,
                         **({"kv_dtype": "int8"} if kv8 else {}))
    stack, kvs = [], []
    lens = torch.zeros((layers, wl.batch), dtype=torch.int32, device=dev)
    for l in range(layers):
        w32 = syn.layer_weights_f32(wl, l, dev)
        gw = {}
        for name, t in w32.items():
            if name.startswith("w_") and wl.weight_dtype == "i8":
                g = wl.group_mlp if wl.group_mlp and name in ("w_ff1", "w_ff2") else wl.group
                q, s = tg.quantize_i8(t.contiguous(), g)
                gw[name], gw["s" + name[1:]] = q, s
            else:
                gw[name] = t.to(act).contiguous()
        del w32
        layer = tg.Layer(cfg, gw)
        kv = tg.KVCache(wl.batch, wl.heads, wl.capacity, wl.head_dim, torch.int8 if kv8 else act, dev, track_host=False)
        kv.d_len = lens[l]  # one [L, B] tensor so one fill resets every layer
        if wl.past:
            kp, vp = syn.past_kv_f32(wl, l, dev)
            to_rows = lambda t: t.permute(0, 2, 1, 3).reshape(wl.batch, wl.past, wl.hidden).to(act).contiguous()
            layer.kv_append(kv, to_rows(kp), to_rows(vp))
            del kp, vp
        stack.append(layer)
        kvs.append(kv)
    torch.cuda.synchronize()
    return stack, kvs, lens, act


def gpu_head(wl, vocab, torch, tg, syn):
    act = torch.float32 if wl.act_dtype == "f32" else torch.float16
    h32 = syn.lm_head_f32(wl, vocab, "cuda")
    head = {"ln_g": h32["ln_g"].to(act).contiguous(), "ln_b": h32["ln_b"].to(act).contiguous()}
    if wl.weight_dtype == "i8":
        head["w"], head["s"] = tg.quantize_i8(h32["w"].contiguous(), wl.group)
    else:
        head["w"] = h32["w"].to(act).contiguous()
    return head


# ------------------------------------------------------------------ timing
def time_launches(torch, stream, launch, reset, steps, warmup):
    """Run launch() warmup + steps times on `stream` (reset() before each), with an event pair
    around every launch: (mean ms over the timed region, per-launch ms)."""
    with torch.cuda.stream(stream):
        for _ in range(max(1, warmup)):
            reset()
            launch()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for i in range(steps):
            reset()
            starts[i].record(stream)
            launch()
            ends[i].record(stream)
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, [a.elapsed_time(b) for a, b in zip(starts, ends)]


def time_graph(torch, stream, step, steps, warmup):
    """Capture step() in a HIP graph and replay it: (mean ms over the timed region, per-step ms)."""
    with torch.cuda.stream(stream):
        step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    with torch.cuda.stream(stream):
        for _ in range(max(1, warmup)):
            g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    with torch.cuda.stream(stream):
        e0.record(stream)
        for i in range(steps):
            g.replay()
            marks[i].record(stream)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return ms, [(e0 if i == 0 else marks[i - 1]).elapsed_time(marks[i]) for i in range(steps)]


def kernel_times(torch, stream, stack, kvs, lens, wl, x, reset, ws=None, reps=3):
    """Per-kernel durations of the per-layer path: one layer step at a time with events between its
    kernel launches (the library's ds_layer_time_kernels, on `stream`), on three layers spread over
    the stack, `reps` times each; the median per kernel kind, in ms."""
    L = len(stack)
    got = {}
    with torch.cuda.stream(stream):
        for _ in range(reps):
            for l in sorted({0, L // 2, L - 1}):
                reset()
                for part, ms in stack[l].time_kernels(kvs[l], x, workspace=ws, stream=stream):
                    got.setdefault(part, []).append(ms)
    torch.cuda.synchronize()
    return {k: statistics.median(v) for k, v in got.items()}


# ------------------------------------------------------------------ the oracle on the host
def _cpu_share():
    """Host threads this run may use: the OMP_NUM_THREADS the box sets, else the CPU count (at
    most 16, the share of one GPU)."""
    n = int(os.environ.get("OMP_NUM_THREADS") or 0) or (os.cpu_count() or 1)
    return max(1, min(16, n))


def _oracle_worker(job):
    """One host process's share of the CPU baseline: oracle layer steps on the arrays in job (files
    under /dev/shm, memory-mapped read-only) until target_s seconds of oracle time have run."""
    import numpy as np

    import oracle

    w = {n: np.load(p, mmap_mode="r") for n, p in job["weights"].items()}
    k = np.array(np.load(job["k"], mmap_mode="r"))
    v = np.array(np.load(job["v"], mmap_mode="r"))
    desc = oracle.Desc(*job["desc"])
    rng = np.random.default_rng(job["seed"])
    x = rng.standard_normal(tuple(job["x_shape"]))
    done, spent = 0, 0.0
    while spent < job["target_s"]:
        lens = np.full(x.shape[0], job["past"], dtype=np.int32)
        t0 = time.perf_counter()
        # the layer overwrites rows past.. and advances a fresh copy of the lengths, so every step
        # starts from the same cache
        oracle.layer_forward(desc, w, k, v, lens, x)
        spent += time.perf_counter() - t0
        done += 1
    return done, spent


def cpu_baselines(wl, layer, kv, target_s: float, rows=None):
    """The oracle (plain C, double, single-threaded) timed on a bounded sample of this workload:
    whole layer steps of layer 0's weights and cache (decode: one new row per sequence; prefill:
    `rows` prompt rows of one sequence), on one host thread and on every host thread of this run
    (one process each, same sample), scaled to the full L-layer stack."""
    import multiprocessing as mp

    import numpy as np
    import torch

    import oracle

    tag = f"/dev/shm/ds_bench_{os.getpid()}"
    paths = {"weights": {}}
    try:
        for n in ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_o", "b_o", "ln2_g", "ln2_b", "w_ff1", "b_ff1", "w_ff2", "b_ff2"):
            t = layer._weights[n]
            if n.startswith("w_") and wl.weight_dtype == "i8":
                s = layer._weights["s" + n[1:]].cpu().view(torch.int16).numpy().view(np.uint16)
                arr = oracle.dequantize_i8(t.cpu().numpy(), s, wl.group)
            else:
                arr = t.double().cpu().numpy()
            paths["weights"][n] = f"{tag}_{n}.npy"
            np.save(paths["weights"][n], arr)
            del arr
        prefill = rows is not None
        B = 1 if prefill else wl.batch
        past = 0 if prefill else wl.past
        shape = (B, wl.heads, wl.capacity, wl.head_dim)
        k = np.zeros(shape)
        v = np.zeros(shape)
        if past:
            k[:, :, :past] = kv.k[:B, :, :past].double().cpu().numpy()
            v[:, :, :past] = kv.v[:B, :, :past].double().cpu().numpy()
        paths["k"], paths["v"] = f"{tag}_k.npy", f"{tag}_v.npy"
        np.save(paths["k"], k)
        np.save(paths["v"], v)
        del k, v
        job = dict(paths, desc=(wl.hidden, wl.heads, wl.head_dim, wl.ffn), past=past, target_s=target_s,
                   x_shape=(B, rows if prefill else 1, wl.hidden), seed=0)
        done1, spent1 = _oracle_worker(job)
        n = _cpu_share()
        t0 = time.perf_counter()
        with mp.get_context("spawn").Pool(n) as pool:
            res = pool.map(_oracle_worker, [dict(job, seed=i) for i in range(n)])
        wall = time.perf_counter() - t0
    finally:
        for p in list(paths["weights"].values()) + [paths.get("k"), paths.get("v")]:
            if p and os.path.exists(p):
                os.remove(p)
    per_step_tokens = rows if prefill else wl.batch
    unit = "prompt tokens/s" if prefill else "tokens/s"
    what = (f"{rows} prompt rows of one sequence" if prefill else
            f"one decode step of {wl.batch} sequences against {wl.past} past rows")
    one = per_step_tokens * done1 / (spent1 * wl.layers)
    steps_all = sum(d for d, _ in res)
    longest = max(s for _, s in res)
    allc = per_step_tokens * steps_all / (longest * wl.layers)
    return ({"value": round(one, 4), "unit": unit, "cores": 1, "kind": "oracle",
             "sample": f"{done1} oracle layer steps ({what}, layer 0 of {wl.name}) in {spent1:.1f} s on one host "
                       f"thread, scaled to the {wl.layers}-layer stack"},
            {"value": round(allc, 4), "unit": unit, "cores": n, "kind": "oracle",
             "sample": f"{steps_all} oracle layer steps of the same sample in {n} single-threaded processes "
                       f"({wall:.1f} s wall), scaled to the {wl.layers}-layer stack"})


# ------------------------------------------------------------------ records
def _base(wl, layers, ms, steps, warmup, value, unit, dtype, launch):
    return {"metric": METRIC, "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": steps, "warmup": warmup,
            "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": dtype, "data": "synthetic (seeded N(0,0.02) weights, N(0,1) inputs and past K/V)",
            "config": {"workload": wl.name, "layers": layers, "batch": wl.batch, "past_kv": wl.past,
                       "hidden": wl.hidden, "heads": wl.heads, "ffn": wl.ffn, "launch": launch}}


def decode_record(args, wl, torch, tg, syn, layers, mode="auto", cpu_s=0.0, vocab=0):
    """One decode workload. The persistent stack (one launch per step) serves batches up to 4; larger
    batches run the per-layer kernels under a HIP graph. With vocab > 0 the step is a whole
    generation step: the stack runs the LM head and the greedy choice after the last layer."""
    stack, kvs, lens, act = build_stack(wl, torch, tg, syn, layers)
    x0 = syn.normal((wl.batch, wl.hidden), 1.0, wl.cfg_id, syn.X_LAYER, 0, "cuda").to(act)
    stream = torch.cuda.Stream()
    per = algorithmic_bytes_per_layer(wl)
    step_bytes = per["total"] * layers
    use_stack = mode == "stack" or (mode == "auto" and wl.batch <= 4)
    dtype = dtype_label(wl)
    reset = lambda: lens.fill_(wl.past)
    extra = {}
    if use_stack:
        head = gpu_head(wl, vocab, torch, tg, syn) if vocab else None
        st = tg.Stack(stack, kvs, max_batch=wl.batch, head=head)
        sws = st.workspace(wl.batch)
        out = torch.empty_like(x0)
        if vocab:
            logits = torch.empty((wl.batch, vocab), dtype=torch.float32, device="cuda")
            tokens = torch.empty(4, dtype=torch.int32, device="cuda")
            launch = lambda: st.generate(x0, out, logits, tokens, sws, stream=stream)
            step_bytes += head_bytes(wl, vocab)
        else:
            launch = lambda: st.decode(x0, out, sws, stream=stream)
        ms, per_step = time_launches(torch, stream, launch, reset, args.steps, args.warmup)
        st.check()
        groups = st.groups
        st.close()
        kernel_ms = statistics.mean(per_step)
        kgbs = step_bytes / (kernel_ms * 1e-3) / 1e9
        name = "stack_decode_kernel (all layers" + (" and the LM head" if vocab else "") + " of one step)"
        roofline = {"bound": "hbm", "kernel": name, "achieved": round(kgbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(kgbs / PEAK_HBM_GBS, 4),
                    "traffic": measured_traffic("stack_decode_kernel", wl.name)
                    if (layers == wl.layers and not vocab) else None,
                    "kernel_ms": round(kernel_ms, 4), "bytes_per_launch": step_bytes}
        launch_desc = f"persistent stack kernel, {groups} workgroups" + (f", LM head over {vocab} rows" if vocab else "")
        if vocab:
            extra = {"vocab": vocab, "head_bytes": head_bytes(wl, vocab), "tokens": tokens[:wl.batch].tolist()}
    else:
        ws = stack[0].workspace(wl.batch, 1, wl.capacity)
        bufs = [torch.empty_like(x0), torch.empty_like(x0)]

        def step():
            lens.fill_(wl.past)
            for l in range(layers):
                stack[l].decode(kvs[l], x0 if l == 0 else bufs[l % 2], bufs[(l + 1) % 2], ws)

        ms, per_step = time_graph(torch, stream, step, args.steps, args.warmup)
        out = bufs[layers % 2]
        kt = kernel_times(torch, stream, stack, kvs, lens, wl, x0, reset, ws)
        pb = part_bytes(wl)
        kernels = {p: {"ms": round(t, 4), "bytes": pb[p], "gbs": round(pb[p] / (t * 1e-3) / 1e9, 1)}
                   for p, t in kt.items()}
        dom = max(kt, key=kt.get)
        gbs_dom = pb[dom] / (kt[dom] * 1e-3) / 1e9
        roofline = {"bound": "hbm", "kernel": f"{dom} (per-layer kernel; the longest of the layer step)",
                    "achieved": round(gbs_dom, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(gbs_dom / PEAK_HBM_GBS, 4), "traffic": None, "kernel_ms": round(kt[dom], 4),
                    "bytes_per_launch": pb[dom], "kernels": kernels}
        launch_desc = "per-layer kernels under a HIP graph (LN, skinny GEMMs, chunked attention)"
    assert torch.isfinite(out.float()).all(), "non-finite decode output"
    gbs = step_bytes / (ms * 1e-3) / 1e9
    rec = _base(wl, layers, ms, args.steps, args.warmup, wl.batch / (ms * 1e-3), "tokens/s", dtype, launch_desc)
    rec.update({"hbm_gbs_per_layer_step": round(gbs, 1), "hbm_frac_of_peak": round(gbs / PEAK_HBM_GBS, 4),
                "bytes_per_layer_step": per, "step_ms": step_stats(per_step), "roofline": roofline, **extra})
    if cpu_s > 0:
        rec["cpu_baseline"], rec["cpu_baseline_all_cores"] = cpu_baselines(wl, stack[0], kvs[0], cpu_s)
    return rec


def prefill_record(args, wl, torch, tg, syn, layers, cpu_s=0.0):
    """Prefill: one step = the B x S prompt through all L layers (lengths reset to 0 each step),
    captured once in a HIP graph and replayed. The roofline entry is the longest MFMA GEMM of the
    layer step, timed per kernel."""
    stack, kvs, lens, act = build_stack(wl, torch, tg, syn, layers)
    ws = stack[0].workspace(wl.batch, wl.seq, wl.capacity)
    x0 = syn.normal((wl.batch, wl.seq, wl.hidden), 1.0, wl.cfg_id, syn.X_LAYER, 0, "cuda").to(act)
    bufs = [torch.empty_like(x0), torch.empty_like(x0)]

    def step():
        lens.zero_()
        for l in range(layers):
            stack[l].prefill(kvs[l], x0 if l == 0 else bufs[l % 2], bufs[(l + 1) % 2], ws)

    stream = torch.cuda.Stream()
    ms, per_step = time_graph(torch, stream, step, args.steps, args.warmup)
    out = bufs[layers % 2]
    assert torch.isfinite(out.float()).all(), "non-finite prefill output"
    fl = prefill_flops(wl)
    kt = kernel_times(torch, stream, stack, kvs, lens, wl, x0, lambda: lens.zero_(), ws)
    kernels = {p: {"ms": round(t, 4), **({"tflops": round(fl[p] / (t * 1e-3) / 1e12, 1)} if p in fl else {})}
               for p, t in kt.items()}
    gemms = [p for p in ("qkv", "o", "ff1", "ff2") if p in kt]
    dom = max(gemms, key=kt.get)
    tf_dom = fl[dom] / (kt[dom] * 1e-3) / 1e12
    tflops = fl["total"] * layers / (ms * 1e-3) / 1e12
    rec = _base(wl, layers, ms, args.steps, args.warmup, wl.batch * wl.seq / (ms * 1e-3), "prompt tokens/s", dtype_label(wl),
                "per-layer kernels (LN, 4 MFMA GEMMs, flash attention) under a HIP graph")
    rec["metric"] = "prefill prompt tokens/s + MFMA utilization of the prefill GEMMs"
    rec["config"].update({"seq": wl.seq})
    rec.update({"flops_per_layer": fl, "step_ms": step_stats(per_step),
                "step_tflops": round(tflops, 1), "step_frac_of_peak": round(tflops / PEAK_F16_TFLOPS, 4),
                "roofline": {"bound": "mfma", "kernel": f"{dom} GEMM (the longest GEMM of the layer step)",
                             "achieved": round(tf_dom, 1), "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(tf_dom / PEAK_F16_TFLOPS, 4), "traffic": None,
                             "kernel_ms": round(kt[dom], 4), "flops_per_launch": fl[dom], "kernels": kernels}})
    if cpu_s > 0:
        rec["cpu_baseline"], rec["cpu_baseline_all_cores"] = cpu_baselines(wl, stack[0], kvs[0], cpu_s, rows=32)
    return rec


def moe_record(args, mw, torch, tg, syn, cpu_s=0.0):
    """The MoE expert FF block of the MoE page's 1.3B + MoE-128 model: one step = the tokens through
    the gate, the routing, the chosen experts' two products and the combination, captured in a HIP
    graph. Algorithmic bytes: the LayerNorm and gate weights, each chosen expert's weights and
    biases once, x2 read and y written. The roofline entry is the longer of the two expert
    products, timed per kernel (ds_moe_time_kernels), over the bytes of the experts it streams."""
    import numpy as np

    import oracle

    H, F, E, T, k = mw.hidden, mw.ffn, mw.experts, mw.tokens, mw.top_k
    w32 = syn.moe_weights_f32(mw, "cuda")
    gw = {n: t.half().contiguous() for n, t in w32.items()}
    del w32
    _free(torch)
    moe = tg.MoE(H, F, E, k, gw, dtype="fp16")
    x = syn.moe_input_f32(mw, "cuda").half()
    y = torch.empty_like(x)
    ws = moe.workspace(T)
    _, sel, _ = moe.forward(x, routing=True)
    torch.cuda.synchronize()
    used = sorted(set(int(e) for e in sel.cpu().numpy().ravel()))
    U = len(used)
    stream = torch.cuda.Stream()
    ms, per_step = time_graph(torch, stream, lambda: moe.forward(x, y, ws, stream=stream), args.steps, args.warmup)
    assert torch.isfinite(y.float()).all(), "non-finite MoE output"
    reps = [moe.time_kernels(x, y, ws, stream=stream) for _ in range(5)]
    kt = {p: statistics.median(r[p] for r in reps) for p in reps[0]}
    b_ff1 = U * (F * H * 2 + F * 2)
    b_ff2 = U * (H * F * 2 + H * 2)
    b_gate = E * H * 2 + 2 * H * 2
    step_bytes = b_gate + b_ff1 + b_ff2 + 2 * T * H * 2
    pb = {"gate": b_gate, "ff1": b_ff1, "ff2": b_ff2}
    kernels = {p: {"ms": round(t, 4), **({"bytes": pb[p], "gbs": round(pb[p] / (t * 1e-3) / 1e9, 1)} if p in pb else {})}
               for p, t in kt.items()}
    dom = "ff1" if kt["ff1"] >= kt["ff2"] else "ff2"
    gbs_dom = pb[dom] / (kt[dom] * 1e-3) / 1e9
    gbs = step_bytes / (ms * 1e-3) / 1e9
    rec = {"metric": "MoE expert-FF tokens/s (gate, top-k routing, chosen experts, combination) + HBM roofline",
           "value": round(T / (ms * 1e-3), 2), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f16",
           "data": "synthetic (seeded N(0,0.02) expert weights, N(0,1/H) gate, N(0,1) inputs)",
           "config": {"workload": mw.name, "hidden": H, "ffn": F, "experts": E, "top_k": k, "tokens": T,
                      "experts_chosen": U, "launch": "5 kernels (gate, routing, grouped FF1, grouped FF2, "
                                                     "combination) under a HIP graph"},
           "hbm_gbs": round(gbs, 1), "hbm_frac_of_peak": round(gbs / PEAK_HBM_GBS, 4), "bytes_per_step": step_bytes,
           "step_ms": step_stats(per_step),
           "roofline": {"bound": "hbm", "kernel": f"moe {dom} (grouped expert GEMV)", "achieved": round(gbs_dom, 1),
                        "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs_dom / PEAK_HBM_GBS, 4),
                        "traffic": None, "kernel_ms": round(kt[dom], 4), "bytes_per_launch": pb[dom],
                        "kernels": kernels}}
    if cpu_s > 0:
        # the oracle on the chosen experts only (a compact copy: the full 128 experts would not fit
        # the host as float64), one token at a time, on one host thread
        idx = torch.tensor(used, device="cuda")
        ow = {"ln_g": gw["ln_g"].double().cpu().numpy(), "ln_b": gw["ln_b"].double().cpu().numpy(),
              "w_gate": gw["w_gate"].index_select(0, idx).double().cpu().numpy()}
        for n in ("w1", "b1", "w2", "b2"):
            ow[n] = gw[n].index_select(0, idx).double().cpu().numpy()
        xd = x.double().cpu().numpy()
        local = np.searchsorted(np.array(used), sel.cpu().numpy())
        t0, done = time.perf_counter(), 0
        while done < T and (done == 0 or time.perf_counter() - t0 < cpu_s):
            oracle.moe_forward(ow, xd[done:done + 1], top_k=k, force_sel=local[done:done + 1])
            done += 1
        el = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": round(done / el, 4), "unit": "tokens/s", "cores": 1, "kind": "oracle",
                               "sample": f"{done} tokens through the oracle's MoE block on the chosen experts in "
                                         f"{el:.1f} s on one host thread"}
    moe.close()
    del gw
    return rec


def _free(torch):
    import gc
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c2", help="headline workload key in synthetic.WORKLOADS (c5: prefill)")
    ap.add_argument("--layers", type=int, default=0, help="override the headline's layer count (0: the workload's)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="oracle sample per leg (one thread, all threads) for the headline (0 disables)")
    ap.add_argument("--record-cpu-seconds", type=float, default=4.0, help="the same for each nested record")
    ap.add_argument("--records", default="c2gen,c2bf16,c2kv8,c3,c4b8,c4b1,c4b1m32,c5,c5bf16,c5kv8,c5i8,moe,moe1",
                    help="nested records after the c2 headline (comma list; empty for none): c2gen (the "
                         "generation step with the LM head), c2bf16 (bf16 weights and activations), c2kv8 "
                         "(an int8 KV cache), c3, c4b8, c4b1, c4b1m32 (int8 with groups of 32 in the MLP matrices), c5, c5bf16 "
                         "(C5 in bf16), c5kv8 (C5 with an int8 KV cache), c5i8 (C5 with int8 weights), moe (the MoE expert FF of the 1.3B + "
                         "MoE-128 model, 8 tokens), moe1 (the same, 1 token)")
    ap.add_argument("--mode", choices=["auto", "stack", "layers"], default="auto",
                    help="stack: one persistent launch per step; layers: the per-layer kernels")
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

    torch.cuda.set_device(0)
    if args.copy_calibration:
        return copy_calibration(torch)
    wl = syn.WORKLOADS[args.config]
    layers = args.layers or wl.layers
    if wl.seq != 1:
        result = prefill_record(args, wl, torch, tg, syn, layers, args.cpu_seconds)
    else:
        result = decode_record(args, wl, torch, tg, syn, layers, args.mode, args.cpu_seconds)
    _free(torch)
    if args.read_probe:
        probe = read_probe_gbs(torch, tg)
        result["read_probe_gbs"] = round(probe, 1)
        if result["roofline"]["unit"] == "GB/s":
            # the roofline kernel's achieved rate over what a plain streaming read reaches here
            result["hbm_frac_of_read_probe"] = round(result["roofline"]["achieved"] / probe, 4)
    names = [r for r in args.records.split(",") if r] if args.config == "c2" else []
    if names:
        result["records"] = {}
    for name in names:
        print(f"[bench] record {name}", file=sys.stderr, flush=True)
        cs = args.record_cpu_seconds
        if name in ("moe", "moe1"):
            mw = syn.MOE_WORKLOADS["moe-1.3b-e128" if name == "moe" else "moe-1.3b-e128-t1"]
            rec = moe_record(args, mw, torch, tg, syn, cs)
        elif name == "c2gen":
            w2 = syn.WORKLOADS["c2"]
            rec = decode_record(args, w2, torch, tg, syn, w2.layers, "stack", 0.0, vocab=syn.GPT_NEO_VOCAB)
            rec["metric"] = "generation-step tokens/s (32 layers + final LayerNorm + LM head + greedy choice)"
        elif syn.WORKLOADS[name].seq != 1:
            cs_rec = 0.0 if name in ("c5bf16", "c5kv8", "c5i8") else cs  # the C5 record's baseline covers the shapes
            rec = prefill_record(args, syn.WORKLOADS[name], torch, tg, syn, syn.WORKLOADS[name].layers, cs_rec)
        else:
            # the C2 precision variants carry no CPU baseline of their own (the headline's covers C2)
            cs_rec = 0.0 if name in ("c2bf16", "c2kv8", "c4b1m32") else cs
            rec = decode_record(args, syn.WORKLOADS[name], torch, tg, syn, syn.WORKLOADS[name].layers, "auto", cs_rec)
        result["records"][name] = rec
        _free(torch)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
