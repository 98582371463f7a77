#!/usr/bin/env python3
"""Decode-step benchmark of the attention layer on one MI355X.

A step is one pass of the whole layer stack of the chosen workload (every
layer: RMSNorm, Q8_0 quantization, Q/K/V projections, RoPE, KV append,
split-K GQA attention, O projection + residual) over one token per sequence,
with every input already resident in HBM. The step is captured once in a HIP
graph (through torch's CUDA-graph API on the current stream) and replayed; K
steps are timed with HIP events on that stream. Replicas of the whole stack
are rotated when one step's bytes would fit the 256 MB last-level cache.

Prints one JSON line: value = achieved GB/s over the algorithmic bytes
(quantized weight blocks + K and V of every attended token, in the cache's
element type; under a sliding window only the last W tokens) of the step.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-layer µs/token + achieved HBM GB/s (weights+KV bytes) vs peak"
PEAK_GBS = 8000.0
MALL_BYTES = 256 * 2 ** 20

DESCRIBE = {
    "c1": "tiny decode layer: D=256 H=4 KV=2 hd=64, 17 attended tokens, 1 layer",
    "c2": "Qwen2-0.5B-shaped decode layer: D=896 H=14 KV=2 hd=64, 1025 attended tokens, 24 layers",
    "c3": "7B-shaped decode layer: D=3584 H=28 KV=4 hd=128, 4097 attended tokens, 28 layers",
    "c4": "long-context decode layer: D=4096 H=32 KV=8 hd=128, 32769 attended tokens, 1 layer",
    "c5": "batched paged decode: D=4096 H=32 KV=8 hd=128, m=8, L_s~U[512,8192], pages of 16, 1 layer",
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c3", choices=sorted(DESCRIBE))
    ap.add_argument("--variant", default="fused",
                    choices=["fused", "chain", "persistent", "two_launch"])
    ap.add_argument("--kv", default="f32", choices=["f32", "bf16", "fp8"],
                    help="KV-cache element type (fp8: E4M3 with one scale per tensor)")
    ap.add_argument("--window", type=int, default=0,
                    help="sliding window: attend only the last W positions (0 = all)")
    ap.add_argument("--ring", action="store_true",
                    help="keep the cache as a ring of `window` slots (contiguous workloads)")
    ap.add_argument("--topk", type=int, default=0,
                    help="sparse attention: each sequence attends a selection of this many "
                         "entries (its last 128 tokens, then uniform picks, then -1), with "
                         "per-head sinks")
    ap.add_argument("--attn-chunk", type=int, default=0,
                    help="tokens per attention split (0 = sized to fill the GPU)")
    ap.add_argument("--eager", action="store_true", help="launch from Python, no graph replay")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="budget of the oracle CPU-baseline sample")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU baseline")
    ap.add_argument("--kernel-reps", type=int, default=50)
    ap.add_argument("--no-extras", action="store_true",
                    help="default workload only: skip the other variants, the long-context "
                         "record and the streaming probe")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy 5 times (the known-size "
                         "reference for the FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.window < 0 or (args.ring and args.window < 1):
        ap.error("--ring needs --window W with W >= 1")
    if args.ring and args.config == "c5":
        ap.error("a ring cache is contiguous; c5 is paged")
    if args.variant == "persistent" and (args.window or args.topk):
        ap.error("the persistent variant takes no window, ring or selection")
    if args.topk < 0 or (args.topk and args.window):
        ap.error("--topk takes a positive count and no window")
    return args


def workload_key(args) -> str:
    """Short name of the timed workload: the configuration, plus the cache's
    element type, window, ring, selection and layer variant when they differ
    from the defaults."""
    key = args.config if args.kv == "f32" else f"{args.config}-{args.kv}"
    if args.window:
        key += f"-w{args.window}" + ("-ring" if args.ring else "")
    if args.topk:
        key += f"-top{args.topk}"
    if getattr(args, "variant", "fused") != "fused":
        key += f"-{args.variant}"
    return key


def workload_text(args) -> str:
    text = f"{args.config}: {DESCRIBE[args.config]}"
    if args.kv != "f32":
        text += f", {args.kv} KV cache"
    if args.window:
        text += f", sliding window of {args.window} tokens"
        if args.ring:
            text += f" in a ring of {args.window} slots"
    if args.topk:
        text += (f", sparse attention over selections of {args.topk} entries (the last 128 "
                 f"tokens, then uniform picks) with per-head sinks")
    return text


def copy_calibration():
    """A plain copy of known size: 256 MiB read and 256 MiB written per
    dispatch (torch's device-to-device copy kernel)."""
    import torch

    n = 256 * 2 ** 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "dispatches": 5}), flush=True)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


VARIANTS = ("chain", "fused", "persistent", "two_launch")


def variant_code(ck, name):
    return {"fused": ck.CK_VARIANT_FUSED, "chain": ck.CK_VARIANT_CHAIN,
            "persistent": ck.CK_VARIANT_PERSISTENT,
            "two_launch": ck.CK_VARIANT_TWO_LAUNCH}[name]


def build_stacks(cfg, kv_dtype, keep_host, window=0, ring=False, topk=0):
    """The workload on the GPU, plus replicas when one step's bytes would fit
    three times in the last-level cache (rotated so that each step reads from
    HBM)."""
    from decode_step_attention_layer_amd import synth
    from decode_step_attention_layer_amd.workload import DeviceStack

    t0 = time.time()
    stack = DeviceStack(cfg, "cuda:0", keep_host=keep_host, kv_dtype=kv_dtype, window=window,
                        ring=ring, topk=topk)
    log(f"[bench] {cfg.name}: {stack.nlayers} layers on device in {time.time() - t0:.1f}s")
    nbytes = synth.algorithmic_bytes(cfg, stack.lens, kv_dtype, window, topk)
    step_bytes = nbytes["total"] * stack.nlayers
    replicas = 1
    if step_bytes < 3 * MALL_BYTES:
        replicas = min(8, math.ceil(3 * MALL_BYTES / step_bytes))
    stacks = [stack] + [stack.clone() for _ in range(replicas - 1)]
    return stacks, nbytes, step_bytes


def time_steps(stacks, desc, steps, warmup, eager=False):
    """Decode steps of the stacks (rotated) with the given layer descriptor:
    eager warm-up, one HIP graph per replica (checked equal to the eager
    step), then `steps` replays timed with one pair of HIP events on the
    launch stream around them (the headline: an event between consecutive
    replays puts a barrier between them, measured at about 4 us per step),
    then a second pass of `steps` replays with an event between consecutive
    steps for the distribution. Returns (mean ms per step, per-step ms of the
    second pass, workspaces)."""
    import torch

    from decode_step_attention_layer_amd import ck

    stack = stacks[0]
    cfg = stack.cfg
    replicas = len(stacks)
    stream = torch.cuda.current_stream()
    if desc.variant == ck.CK_VARIANT_PERSISTENT:
        # every layer of the step in one persistent kernel (ck_decode_step)
        wss = [s.step_workspace(desc) for s in stacks]
        outs = [torch.empty((cfg.m, cfg.D), dtype=torch.float32, device="cuda:0")
                for _ in stacks]

        def one_step(j):
            return stacks[j].decode_step(desc, wss[j], out=outs[j])
    else:
        # one ck_decode_layer call per layer
        wss = [s.workspace(desc) for s in stacks]
        outs = [s.bufs[(stack.nlayers - 1) % 2] for s in stacks]

        def one_step(j):
            return stacks[j].step(desc, wss[j])

    for _ in range(max(1, warmup)):
        for j in range(replicas):
            one_step(j)
    torch.cuda.synchronize()
    ref = outs[0].clone()
    graphs = []
    if not eager:
        for j in range(replicas):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                one_step(j)
            graphs.append(g)
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(outs[0], ref), "graph replay differs from the eager step"

    def run_step(i):
        if graphs:
            graphs[i % replicas].replay()
        else:
            one_step(i % replicas)

    for i in range(warmup):
        run_step(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(steps):
        run_step(i)
    b.record(stream)
    torch.cuda.synchronize()
    mean = a.elapsed_time(b) / steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        run_step(i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    assert torch.isfinite(outs[0]).all(), "non-finite layer output"
    if desc.variant == ck.CK_VARIANT_PERSISTENT:
        for s, ws in zip(stacks, wss):
            assert s.step_status(desc, ws) == 0, "a persistent step timed out"
    if desc.variant == ck.CK_VARIANT_TWO_LAUNCH:
        off = ck.ck_decode_layer_ws_offset(desc, stack.max_ctx, "status")
        for ws in wss:
            assert int(ws[off:off + 4].view(torch.int32).item()) == 0, "a wait timed out"
    return mean, ms, wss


def pct(v, q):
    import numpy as np

    return float(np.percentile(np.asarray(v, float), q))


def stream_probe():
    """The box's achievable streaming-read bandwidth: libck's plain read
    kernel (ck_read_probe: 16-byte non-temporal loads, four workgroups per
    compute unit) over 2 GiB, timed with HIP events on the launch stream;
    the best of 6 launches."""
    import torch

    from decode_step_attention_layer_amd import ck

    n = 2 << 30
    x = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    sink = torch.zeros(8192, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream()
    best = None
    for _ in range(6):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        ck.ck_read_probe(x, n, sink)
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        best = ms if best is None else min(best, ms)
    del x
    torch.cuda.empty_cache()
    return {"GBs": round(n / (best * 1e-3) / 1e9, 1), "bytes": n,
            "frac_of_peak": round(n / (best * 1e-3) / 1e9 / PEAK_GBS, 4),
            "kind": "ck_read_probe over 2 GiB (plain streaming read), best of 6"}


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the layer is built and timed on a single MI355X "
              "(sharding the layer across GPUs is not implemented).", file=sys.stderr)
        sys.exit(2)

    import torch

    from decode_step_attention_layer_amd import ck, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    ck.load()
    cfg = synth.CONFIGS[args.config]
    kv_dtype = {"f32": synth.KV_F32, "bf16": synth.KV_BF16, "fp8": synth.KV_FP8}[args.kv]
    stacks, nbytes, step_bytes = build_stacks(cfg, kv_dtype, not args.no_cpu, args.window,
                                              args.ring, args.topk)
    stack = stacks[0]
    desc = stack.desc(variant_code(ck, args.variant), args.attn_chunk)
    ms_step, ms, wss = time_steps(stacks, desc, args.steps, args.warmup, args.eager)
    us_layer = ms_step * 1e3 / stack.nlayers
    value = step_bytes / (ms_step * 1e-3) / 1e9
    log(f"[bench] step {ms_step * 1e3:.2f} us, {us_layer:.2f} us/layer, {value:.0f} GB/s")

    if desc.variant == ck.CK_VARIANT_PERSISTENT:
        # the step is one kernel (k_step, after a counter-clearing kernel of
        # about a microsecond): its launches are the timed region itself
        roof = {"bound": "hbm", "achieved": round(value, 1), "peak": PEAK_GBS, "unit": "GB/s",
                "frac": round(value / PEAK_GBS, 4), "traffic": None, "kernel": "k_step",
                "us_per_launch": round(ms_step * 1e3, 3), "bytes_per_launch": step_bytes}
    else:
        roof = roofline(args, stacks, desc, wss[0], nbytes)
    extras = {}
    default_run = (args.config == "c3" and args.kv == "f32" and not args.window and not args.topk
                   and not args.eager and not args.no_extras)
    if default_run:
        extras = extra_records(args, stacks, step_bytes, args.variant, us_layer)
    del wss
    cpu = None if args.no_cpu else cpu_baseline(args, stack, nbytes)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8-dot/f32",
        "data": "synthetic (seeded; quantized N(0,0.02) weights, N(0,1) activations and cache)",
        "config": {
            "workload": workload_text(args),
            "kv_cache": args.kv,
            "window": args.window,
            "ring": args.ring,
            "topk": args.topk,
            "variant": args.variant,
            "attn_chunk": args.attn_chunk,
            "launch": "eager" if args.eager else "hip-graph",
            "layers": stack.nlayers,
            "tokens_per_step": cfg.m,
            "replicas": len(stacks),
        },
        "us_per_layer": round(us_layer, 3),
        "us_per_token": round(ms_step * 1e3 / cfg.m, 3),
        "step_us": {"mean": round(ms_step * 1e3, 2),
                    "evented": {"median": round(pct(ms, 50) * 1e3, 2),
                                "p10": round(pct(ms, 10) * 1e3, 2),
                                "p90": round(pct(ms, 90) * 1e3, 2),
                                "note": "a second pass of the same steps with an event between "
                                        "consecutive ones: each adds a barrier between graph "
                                        "replays (about 4 us per step)"}},
        "bytes_per_step": step_bytes,
        "frac_of_peak": round(value / PEAK_GBS, 4),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    line.update(extras)
    print(json.dumps(line), flush=True)


def extra_records(args, stacks, step_bytes, variant, us_layer):
    """Beside the default workload's line: the same stack in every variant
    (the fused layer against the unfused chain, the persistent step and the
    two-launch layer), the long-context layer (the second target workload)
    with its attention kernel's roofline, and the streaming-read probe."""
    import torch

    from decode_step_attention_layer_amd import ck, synth

    steps, warm = max(10, min(args.steps, 30)), max(2, min(args.warmup, 5))
    stack = stacks[0]
    var = {}
    for v in VARIANTS:
        if v == variant:
            var[v] = {"us_per_layer": round(us_layer, 3)}
            continue
        d = stack.desc(variant_code(ck, v), args.attn_chunk)
        m, ms, wss = time_steps(stacks, d, steps, warm)
        del wss
        var[v] = {"us_per_layer": round(m * 1e3 / stack.nlayers, 3),
                  "median_us_per_layer_evented": round(pct(ms, 50) * 1e3 / stack.nlayers, 3),
                  "GBs": round(step_bytes / (m * 1e-3) / 1e9, 1)}
        log(f"[bench] c3 {v}: {var[v]['us_per_layer']:.2f} us/layer")
    torch.cuda.synchronize()
    del stacks[1:]
    torch.cuda.empty_cache()

    # the long-context layer
    cfg4 = synth.CONFIGS["c4"]
    st4, nb4, sb4 = build_stacks(cfg4, synth.KV_F32, False)
    d4 = st4[0].desc(variant_code(ck, variant), 0)
    m4, ms4, ws4 = time_steps(st4, d4, max(20, steps), warm)
    g4 = sb4 / (m4 * 1e-3) / 1e9
    class A:   # the roofline's view of the arguments for this workload
        kernel_reps = args.kernel_reps
        config, kv, window, ring, topk = "c4", "f32", 0, False, 0
    r4 = roofline(A, st4, d4, ws4[0], nb4) if d4.variant != ck.CK_VARIANT_PERSISTENT else None
    secondary = {"workload": workload_text(A),
                 "variant": variant,
                 "us_per_layer": round(m4 * 1e3, 3),
                 "evented_steps_us": {"median": round(pct(ms4, 50) * 1e3, 2),
                                      "p10": round(pct(ms4, 10) * 1e3, 2),
                                      "p90": round(pct(ms4, 90) * 1e3, 2)},
                 "GBs": round(g4, 1), "frac_of_peak": round(g4 / PEAK_GBS, 4),
                 "bytes_per_layer": sb4,
                 "attention": None if r4 is None else {
                     "kernel": r4["kernel"], "us_per_launch": r4["us_per_launch"],
                     "GBs": r4["achieved"], "frac": r4["frac"], "traffic": r4["traffic"]}}
    log(f"[bench] c4: {m4 * 1e3:.2f} us/layer, {g4:.0f} GB/s")
    del st4, ws4
    torch.cuda.empty_cache()
    return {"variants_c3": var, "secondary": secondary, "stream_probe": stream_probe()}


def _time_launches(fn, reps, passes=5):
    """Time of one fn() launch: `reps` launches captured in one HIP graph
    (torch's graph API on the current stream), so that the host's launch rate
    does not pace short kernels, replayed `passes` times, each replay timed
    with events on that stream; the median replay's average per launch."""
    import torch

    stream = torch.cuda.current_stream()
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(passes):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        per.append(a.elapsed_time(b) * 1e3 / reps)     # us per launch
    return pct(per, 50)


def roofline(args, stacks, desc, ws, nbytes):
    """Per-launch timing, with HIP events on the launch stream, of the layer's
    large kernels through their C-ABI entry points, in the launch
    configuration the layer uses: the split-K attention pass (ck_attn_partial,
    one kernel: k_attn) and the O-projection GEMV (ck_gemv_q5_0_q8_0, one
    kernel: k_gemv). Successive launches cycle over every layer of every
    replica, as the decode steps do, so that a launch does not find its cache
    or weights left in the last-level cache by the one before; they are
    replayed from one HIP graph. The kernel that takes longer is reported,
    against the algorithmic bytes it reads."""
    import torch

    from decode_step_attention_layer_amd import ck, synth

    stack = stacks[0]
    cfg = stack.cfg
    units = [L for s in stacks for L in s.layers]
    turn = [0, 0]

    def nxt(k):
        turn[k] += 1
        return units[turn[k] % len(units)]
    m, D, H, KV, hd = cfg.m, cfg.D, cfg.H, cfg.KV, cfg.hd
    off = lambda n: ck.ck_decode_layer_ws_offset(desc, stack.max_ctx, n)
    base = ws.data_ptr()
    q, aq = base + off("q"), base + off("aq")
    # the split the layer plans for these positions, passed explicitly
    chunk, _ = ck.ck_decode_layer_attn_plan(desc, units[0].cache, stack.pos, stack.topk)
    nws = ck.ck_attn_workspace_size(m, H, KV, hd, stack.max_ctx, chunk)
    part = torch.empty(nws, dtype=torch.uint8, device=ws.device)
    out = torch.empty((m, D), dtype=torch.float32, device=ws.device)
    scale = 1.0 / math.sqrt(hd)

    if stack.topk:
        # the sparse attention has no separate partial entry point: the pair
        # of kernels (partial and merge) is timed
        nws = ck.ck_attn_workspace_size(m, H, KV, hd, stack.topk, chunk)
        part = torch.empty(nws, dtype=torch.uint8, device=ws.device)
        att_out = torch.empty((m, H * hd), dtype=torch.float32, device=ws.device)

        def sparse_attn():
            L = nxt(0)
            ck.ck_attn_sparse(q, L.cache, stack.pos, L.tensors["sel"], stack.topk,
                              L.tensors["sink"], att_out, m, H, scale, chunk, part, nws)
        attn_us = _time_launches(sparse_attn, args.kernel_reps)
        attn_name = "k_attn+k_attn_merge"
    else:
        attn_us = _time_launches(lambda: ck.ck_attn_partial(
            q, nxt(0).cache, stack.pos, m, H, scale, chunk, part, nws),
            args.kernel_reps)
        # query groups over 4 heads attending an fp32 cache, and one sequence
        # attending a bf16 or fp8 cache, run on the matrix cores (kernels of
        # their own names)
        if args.kv == "f32":
            attn_name = "k_attn_mfma" if H // KV > 4 else "k_attn"
        else:
            attn_name = "k_attn_mfma16" if m == 1 else "k_attn"

    def o_gemv():
        L = nxt(1)
        ck.ck_gemv_q5_0_q8_0(L.tensors["wo"], aq, L.tensors["bo"], stack.x0, out, D, H * hd, m)
    wo_us = _time_launches(o_gemv, args.kernel_reps)
    kv_bytes = nbytes["kv"]
    wo_bytes = D * (H * hd // 32) * synth.Q5_0_BYTES
    att_gbs = kv_bytes / (attn_us * 1e-6) / 1e9
    wo_gbs = wo_bytes / (wo_us * 1e-6) / 1e9
    log(f"[bench] k_attn {attn_us:.2f} us ({att_gbs:.0f} GB/s), O GEMV {wo_us:.2f} us "
        f"({wo_gbs:.0f} GB/s)")
    if attn_us >= wo_us:
        name, gbs, us, b = attn_name, att_gbs, attn_us, kv_bytes
    else:
        name, gbs, us, b = "k_gemv", wo_gbs, wo_us, wo_bytes
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_GBS, 4),
            "traffic": recorded_traffic(name, workload_key(args)),
            "traffic_unit": "bytes per launch",
            "kernel": name,
            "us_per_launch": round(us, 3), "bytes_per_launch": b,
            "other": {"attn_chunk": chunk, "k_attn_us": round(attn_us, 3),
                      "k_attn_GBs": round(att_gbs, 1),
                      "o_gemv_us": round(wo_us, 3), "o_gemv_GBs": round(wo_gbs, 1)}}


def recorded_traffic(kernel: str, workload: str, launches_bytes=None):
    """HBM bytes per dispatch of `kernel` on `workload` from the FETCH_SIZE /
    WRITE_SIZE counter runs recorded in profiles/hbm_traffic_counters.md
    (each counter scaled by its reading for a copy of known size), or None if
    there is no record or the kernel's source changed since it was taken.
    A name joined by '+' sums the records of its kernels."""
    if "+" in kernel:
        parts = [recorded_traffic(k, workload) for k in kernel.split("+")]
        return None if any(p is None for p in parts) else sum(parts)
    import hashlib
    import re

    path = os.path.join(ROOT, "profiles", "hbm_traffic_counters.md")
    try:
        text = open(path).read()
    except OSError:
        return None
    mt = re.search(r"```json\n(.*?)```", text, re.S)
    if not mt:
        return None
    rec = json.loads(mt.group(1))
    csrc = os.path.join(ROOT, "decode_step_attention_layer_amd", "csrc")
    h = hashlib.sha256()
    src_file = {"k_attn_merge": "k_attn", "k_attn_mfma": "k_attn",
                "k_attn_mfma16": "k_attn16"}.get(kernel, kernel) + ".hip"
    # the merge runs as k_attn_merge1 (one wavefront) when a sequence has at
    # most 32 chunks: either record stands for it
    names = ("k_attn_merge", "k_attn_merge1") if kernel == "k_attn_merge" else (kernel,)
    for f in (src_file, "ck_device.hpp", "ck_internal.hpp", "ck_gemv_common.hpp",
              "ck_attn_common.hpp"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    src = h.hexdigest()[:16]
    for r in rec["records"]:
        if r["kernel"] in names and r["workload"] == workload and r["src"] == src:
            return round(r["fetch_kib"] * 1024 * rec["fetch_scale"] +
                         r["write_kib"] * 1024 * rec["write_scale"])
    return None


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(args, stack, nbytes):
    """The oracle (plain single-threaded C) on the host cores, on a bounded
    sample of the same workload: whole layers, cycling over the stack's layers
    with the first layer's input, until the time budget is spent. The process
    is pinned to one core while the sample runs."""
    import numpy as np

    import oracle
    from decode_step_attention_layer_amd import synth

    allowed = sorted(os.sched_getaffinity(0))
    core = allowed[-1]
    os.sched_setaffinity(0, {core})
    try:
        res = _cpu_sample(args, stack, nbytes, oracle, synth)
    finally:
        os.sched_setaffinity(0, set(allowed))
    res.update({"pinned_core": core, "nproc": os.cpu_count(), "cores_allowed": len(allowed),
                "cpu_model": cpu_model()})
    return res


def _cpu_sample(args, stack, nbytes, oracle, synth):

    cfg = stack.cfg
    cos, sin = synth.rope_for(cfg)
    dims = dict(D=cfg.D, H=cfg.H, KV=cfg.KV, hd=cfg.hd, m=cfg.m, eps=cfg.eps)
    x = stack.x0_host
    done, t_spent, li = 0, 0.0, 0
    while t_spent < args.cpu_seconds:
        L = stack.layers[li % stack.nlayers]
        h = L.host
        kvd = dict(dtype=stack.kv_dtype, k_scale=stack.k_scale, v_scale=stack.v_scale,
                   window=stack.window, ring=stack.ring)
        if cfg.page_size:
            c = oracle.Cache(h["k"], h["v"], cfg.KV, cfg.hd, page_size=cfg.page_size,
                             page_table=h["table"], max_pages_per_seq=cfg.max_pages_per_seq,
                             num_pages=h["k"].shape[0], **kvd)
        else:
            c = oracle.Cache(h["k"], h["v"], cfg.KV, cfg.hd, capacity=stack.capacity, **kvd)
        w = dict(h, rope_cos=cos, rope_sin=sin)
        t = time.perf_counter()
        if stack.topk:
            oracle.decode_layer(dims, w, c, x, x, stack.pos, sel=h["sel"], sink=h["sink"])
        else:
            oracle.decode_layer(dims, w, c, x, x, stack.pos)
        t_spent += time.perf_counter() - t
        done += 1
        li += 1
    gbs = nbytes["total"] * done / t_spent / 1e9
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "us_per_layer": round(t_spent * 1e6 / done, 1),
            "sample": f"{done} whole-layer calls of the {workload_key(args)} workload "
                      f"(layers cycled, first-layer input), {t_spent:.1f} s single-threaded "
                      f"on one pinned core"}


if __name__ == "__main__":
    main()
