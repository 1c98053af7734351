#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE layer on one MI355X.

Workload (default): GLM-5.2-shaped decode layer — hidden 6144, expert inter
2048, 256 routed experts top-8 + 1 shared, int4 per-row-scaled experts
(18.9 MB each), Q8_0 activations, random fp32 router gate — with 12 layers
resident in HBM (about 58 GB).  A step is one token through one layer:
coli_moe_layer (router, Q8_0, 8 routed experts + shared, combine); step s
uses layer s mod 12 and its own hidden state, so expert reads do not hit in
the 256 MB last-level cache.  Steps are captured in a HIP graph and
replayed.

--workload prefill times the batch-union prefill instead: the same layer
shape with all 257 experts resident, a step being one batch of 2048 tokens
whose routing has a Zipf(1.1) skew over expert popularity (the grouped
int8 matrix-core kernels); its roofline is the gate/up kernel's int8
TOPS against the MI355X dense int8 peak.

--workload verify times the speculative-verify batch: 4 tokens per step
routed jointly through int8 layers (12 resident, about 116 GB), the tokens
sharing about 40% of their experts.

--workload tiered streams GLM-5.2-shaped layers (75 by default, int4 or,
with --tier-bits 2, int2) through a 48 GB HBM expert cache split into
per-layer LRUs, the other experts staged from pinned host memory by
hipMemcpyAsync on a side stream while the resident experts compute; one
token per step through every layer, routed by a seeded trace in which each
of the 8 slots reuses the previous step's expert with probability 0.6.

--copy-calibration MB runs only a device-to-device copy of MB megabytes
(torch copy_) ten times: the reference for scaling rocprofv3's
FETCH_SIZE / WRITE_SIZE counters to bytes.

Prints one JSON line: MoE-layer tokens/s, the roofline of the dominant
kernel (HIP-event kernel durations measured in this run), whole-layer HBM
GB/s, and the CPU oracle timed on this host as a baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + achieved HBM GB/s (decode), int8 TOPS (prefill)"
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload", choices=("decode", "verify", "prefill", "tiered"), default="decode")
    ap.add_argument("--tier-bits", type=int, choices=(4, 2), default=4, help="tiered: expert width")
    ap.add_argument("--group-size", type=int, choices=(0, 64), default=0,
                    help="decode / prefill: 64 = group-scaled int4 experts (one scale per 64 codes of a row)")
    ap.add_argument("--wformat", choices=("int", "mxfp4"), default="int",
                    help="decode, prefill: mxfp4 = MXFP4 experts (E2M1 codes, one E8M0 scale per 32 codes of a row)")
    ap.add_argument("--tier-layers", type=int, default=75, help="tiered: layers streamed")
    ap.add_argument("--host-layers", type=int, default=8,
                    help="tiered: distinct layers of expert bytes in pinned host memory (reused cyclically)")
    ap.add_argument("--cache-gb", type=float, default=48.0, help="tiered: HBM expert cache, split over the layers")
    ap.add_argument("--lookahead", action="store_true",
                    help="tiered: while a layer computes, stage the experts the next layer's router predicts from "
                         "this layer's state (seeded trace with about 71.6%% one-layer-ahead recall) into the next "
                         "layer's slots")
    ap.add_argument("--steps", type=int, default=None, help="timed steps (decode 2400, prefill 200)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (decode 240, prefill 20)")
    ap.add_argument("--tokens", type=int, default=2048, help="tokens per prefill step")
    ap.add_argument("--layers", type=int, default=12, help="resident GLM-shaped layers")
    ap.add_argument("--graph-steps", type=int, default=240, help="steps per captured HIP graph")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU-oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill-record", action="store_true",
                    help="decode: skip the prefill record the default run adds to its line")
    ap.add_argument("--prefill-steps", type=int, default=50, help="decode: timed steps of the added prefill record")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="only run a device copy of MB megabytes ten times (counter calibration)")
    ap.add_argument("--path", choices=("layer", "split"), default="layer",
                    help="layer: one coli_moe_layer launch per step; split: coli_moe_route + coli_moe_forward")
    ap.add_argument("--kernels", choices=("auto", "multi", "persistent", "grouped"), default="auto",
                    help="kernel set: the library's choice, the multi-launch decode kernels, the persistent "
                         "one or the grouped matrix-core kernels")
    a = ap.parse_args()
    if a.steps is None:
        a.steps = {"decode": 2400, "verify": 1200, "prefill": 200, "tiered": 64}[a.workload]
    if a.warmup is None:
        a.warmup = {"decode": 240, "verify": 120, "prefill": 20, "tiered": 8}[a.workload]
    return a


PATHS = {"auto": 0, "multi": 1, "persistent": 2, "grouped": 3}
INT8_PEAK_TOPS = 5000.0   # MI355X dense int8 matrix-core peak
FP8_PEAK_TOPS = 5000.0    # MI355X dense FP8 matrix-core peak (TFLOP/s)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} requested, but this layer build runs on exactly one GPU "
              "(no collectives or sharding); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if args.copy_calibration:
        n = args.copy_calibration * 1000 * 1000
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 10}), flush=True)
        return

    hipbuild = _hipbuild()
    if not os.path.exists(hipbuild.LIB):
        hipbuild.build()
    import quantized_expert_ffn_amd as q
    import synth

    torch.cuda.set_device(0)
    q.coli_moe_debug_force_path(PATHS[args.kernels])
    if args.workload == "prefill":
        run_prefill(args, q, synth)
        return
    if args.workload == "tiered":
        run_tiered(args, q, synth)
        return
    verify = args.workload == "verify"
    spec = synth.GLM_INT8 if verify else synth.GLM
    if args.group_size:
        if verify:
            raise SystemExit("--group-size applies to int4 experts (decode, prefill)")
        spec = synth.GLM_GS64
    if args.wformat == "mxfp4":
        if verify or args.group_size:
            raise SystemExit("--wformat mxfp4 applies to the decode workload without --group-size")
        spec = synth.GLM_MX
    S = 4 if verify else 1  # tokens per step
    dims = q.make_dims(spec)
    H, E = spec.hidden, spec.n_experts
    L = args.layers
    bb = spec.blob_bytes
    nblob = E + 1  # routed + shared, contiguous per layer

    # ---- resident layers: generated on the host (pinned staging), copied to HBM
    t0 = time.time()
    layers = []
    staging = [torch.empty(nblob * bb, dtype=torch.uint8, pin_memory=True) for _ in range(2)]
    copy_stream = torch.cuda.Stream()
    done = [None, None]
    for l in range(L):
        buf = staging[l % 2]
        if done[l % 2] is not None:
            done[l % 2].synchronize()
        base = buf.data_ptr()
        for e in range(nblob):
            if spec.fmt == 1:
                synth.mx_cdf_expert_into(base + e * bb, args.seed, l, e, spec)
            else:
                synth.cdf_expert_into(base + e * bb, args.seed, l, e, spec)
        dev = torch.empty(nblob * bb, dtype=torch.uint8, device="cuda")
        with torch.cuda.stream(copy_stream):
            dev.copy_(buf, non_blocking=True)
            ev = torch.cuda.Event()
            ev.record(copy_stream)
        done[l % 2] = ev
        d = synth.layer_inputs(args.seed, l, spec, 1)
        table = torch.tensor([dev.data_ptr() + e * bb for e in range(E)], dtype=torch.int64, device="cuda")
        layers.append({"blobs": dev, "table": table, "shared": dev.data_ptr() + E * bb,
                       "router_w": torch.from_numpy(d["router_w"]).cuda(), "router_w_host": d["router_w"],
                       "bias": torch.from_numpy(d["bias"]).cuda()})
        log(f"layer {l}: {nblob} experts generated and staged ({time.time() - t0:.1f} s)")
    torch.cuda.synchronize()
    del staging
    G, reps, reps_w, warm_eager = graph_plan(args.steps, args.warmup, args.graph_steps)
    if verify:
        # step s: 4 tokens of layer s mod L sharing experts (independent draws per step)
        xs_host = np.concatenate([synth.verify_hidden_states(args.seed, s % L, spec, S, batch=1 + s // L,
                                                             W=layers[s % L]["router_w_host"])
                                  for s in range(G)])
    else:
        xs_host = synth.hidden_states(args.seed, 1000, G, H)
    xs = torch.from_numpy(xs_host).cuda()
    ws = torch.zeros(q.coli_moe_workspace_bytes(dims, S), dtype=torch.uint8, device="cuda")
    idx = torch.empty((G * S, spec.top_k), dtype=torch.int32, device="cuda")
    wts = torch.empty((G * S, spec.top_k), dtype=torch.float32, device="cuda")
    out = torch.empty((G * S, H), dtype=torch.float32, device="cuda")
    log(f"setup done in {time.time() - t0:.1f} s; {torch.cuda.memory_allocated() / 1e9:.1f} GB allocated")

    def step(s):
        lay = layers[s % L]
        r = slice(s * S, (s + 1) * S)
        x = xs[r]
        if args.path == "layer":
            q.coli_moe_layer(dims, x, lay["router_w"], lay["bias"], lay["table"], lay["shared"],
                             idx[r], wts[r], out[r], ws)
        else:
            q.coli_moe_route(dims, x, lay["router_w"], lay["bias"], idx[r], wts[r], ws)
            q.coli_moe_forward(dims, x, idx[r], wts[r], lay["table"], lay["shared"], out[r], ws)

    # eager pass: correctness of the status word, kernel timing with HIP events
    for s in range(G):
        step(s)
    rc = q.coli_moe_status(ws)
    if rc != 0:
        raise RuntimeError(f"device status {rc}: {q.coli_moe_last_error()}")
    routed = idx.cpu().numpy()

    # per-kernel durations: every launch of an eager pass carries a HIP event
    # pair recorded at the kernel's own start and end
    kernel_us, launches = kernel_times(q, lambda: [step(s) for s in range(G)])

    # captured steps
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        for s in range(G):
            step(s)
    torch.cuda.synchronize()
    for _ in range(reps_w):
        graph.replay()
    for s in range(warm_eager):
        step(s)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    rep_ev = replay_timed(graph, reps)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t1
    steps = reps * G
    rc = q.coli_moe_status(ws)
    if rc != 0:
        raise RuntimeError(f"device status after replay {rc}: {q.coli_moe_last_error()}")
    ms_per_step = 1e3 * elapsed / steps
    tokens_per_s = steps * S / elapsed
    step_spread = replay_spread(rep_ev, G)

    # algorithmic bytes: each step reads W_r and each unique expert of its
    # tokens (8 routed + shared for one token) once
    uniq = [len(set(routed[s * S:(s + 1) * S].ravel().tolist())) for s in range(G)]
    n_units = float(np.mean(uniq)) + spec.n_shared
    lay_bytes = E * H * 4 + E * 4 + n_units * bb
    if "layer" in kernel_us:
        dom, dom_kernel = "layer", "k_layer<%d,%d,1,24>" % (spec.wbits, S)
        dom_bytes = lay_bytes
    elif "forward_persistent" in kernel_us:
        dom, dom_kernel = "forward_persistent", "k_layer<%d,%d,0,24>" % (spec.wbits, S)
        dom_bytes = n_units * bb
    else:
        # for up to 2 tokens with at most 128 KiB of shared gate/up rows per
        # 16-row half tile, the layer call runs the shared expert's gate/up in
        # its router launch; the gate/up launch then reads the routed experts
        # only
        in_router = args.path == "layer" and S <= 2 and 32 * H * spec.wbits // 8 <= 128 * 1024
        gu_units = n_units - (spec.n_shared if in_router else 0)
        dom, dom_kernel = "gateup", "k_gateup<%d,%d%s>" % (spec.wbits, min(S, 4),
                                                            ",gs64" if spec.group else (",mxfp4" if spec.fmt else ""))
        n_scales = H // spec.group if spec.group else 1   # per gate / up row
        scale_bytes = 2 * spec.inter * (H // 32) if spec.fmt == 1 else 2 * spec.inter * 4 * n_scales
        dom_bytes = gu_units * (2 * spec.inter * H * spec.wbits // 8 + scale_bytes)
    dom_us = kernel_us[dom]
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    layer_gbs = lay_bytes / (ms_per_step * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8xi8->i32,f32" if verify else ("i8xe2m1->i32,f32" if spec.fmt == 1 else "i8xi4->i32,f32"),
        "data": "synthetic (seeded; GLM-5.2-shaped random-code experts)",
        "config": {
            "workload": ("GLM-5.2-shaped speculative-verify batch, 4 tokens/step routed jointly (about 40% "
                         "shared experts): hidden 6144, expert inter 2048, 256 routed experts top-8 + 1 shared, "
                         "int8 per-row-scaled weights (37.8 MB/expert), Q8_0 activations, fp32 router gate; "
                         f"{L} layers resident in HBM, step s uses layer s mod {L}") if verify else
                        ("GLM-5.2-shaped MoE decode layer, 1 token/step: hidden 6144, expert inter 2048, "
                         "256 routed experts top-8 + 1 shared, "
                         + ("int4 weights with one scale per 64 codes of a row (21.2 MB/expert), " if spec.group
                            else "MXFP4 weights: E2M1 codes, one E8M0 scale per 32 codes of a row (20.05 MB/expert), "
                            if spec.fmt == 1 else "int4 per-row-scaled weights (18.9 MB/expert), ")
                         + f"Q8_0 activations, fp32 router gate; {L} layers resident in HBM, step s uses layer "
                         f"s mod {L}"),
            "layers_resident": L, "resident_gb": round(L * nblob * bb / 1e9, 1),
            "tokens_per_step": S, "graph_steps": G, "graph_replays": reps, "entry": args.path,
            "kernels": args.kernels,
        },
        "roofline": {
            "bound": "hbm", "kernel": dom_kernel,
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": counted_traffic(dom_kernel),
            "algorithmic_bytes_per_launch": dom_bytes, "avg_launch_us": round(dom_us, 3),
        },
        "layer_hbm_gbs": round(layer_gbs, 1),
        "layer_hbm_frac": round(layer_gbs / HBM_PEAK_GBS, 4),
        "kernel_avg_us": {k: round(v, 3) for k, v in kernel_us.items()},
        "experts_read_per_step": n_units,
        "ms_per_step_p10_p50_p90": step_spread,
    }

    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(args, spec, xs_host, layers, L, S)
    add_measured_roof(res, q, "hbm")
    if args.workload == "decode" and not args.group_size and args.wformat == "int" and not args.no_prefill_record:
        # the prefill half of the metric, on the same GPU in the same run
        del layers, graph, xs, ws, idx, wts, out
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        pa = argparse.Namespace(**vars(args))
        pa.steps, pa.warmup, pa.tokens, pa.kernels = args.prefill_steps, 10, 2048, "auto"
        q.coli_moe_debug_force_path(0)
        res["prefill"] = run_prefill(pa, q, synth, embedded=True)
    print(json.dumps(res), flush=True)


def graph_plan(steps, warmup, graph_steps):
    """Steps per captured graph G and replays: G divides the timed steps K
    exactly (K = reps * G), leaves at least five replays when K allows (so
    the per-replay spread has several samples) and is at most the warmup W
    when W > 0 (so that the graph has been replayed once before the timed
    replays).  Warmup: exactly W steps, as whole replays of the graph while
    they fit, then single eager steps."""
    cap = max(1, min(graph_steps, steps // 5 if steps >= 5 else steps, warmup if warmup > 0 else steps))
    G = max(g for g in range(1, cap + 1) if steps % g == 0)
    return G, steps // G, warmup // G, warmup % G


KINDS = (("router_logits", 0), ("router_select", 1), ("quant_x", 7), ("group", 8), ("gateup", 2), ("down", 3),
         ("combine", 4), ("layer", 5), ("forward_persistent", 6))


def replay_timed(graph, reps):
    """Replays the captured graph reps times, with an event pair around each
    replay; returns the pairs (read after the caller's synchronize)."""
    import torch
    evs = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        graph.replay()
        b.record()
        evs.append((a, b))
    return evs


def replay_spread(evs, steps_per_replay):
    """10th, 50th and 90th percentile over the replays of ms per step."""
    import numpy as np
    v = np.array([a.elapsed_time(b) / steps_per_replay for a, b in evs])
    return [round(float(x), 5) for x in np.percentile(v, [10, 50, 90])]


def add_measured_roof(res, q, kind):
    """Adds to res["roofline"] the ceiling of the same kind measured on this
    GPU in this run, and the dominant kernel's fraction of it:
      hbm   a streaming read of 4 GiB (coli_moe_roof_stream_read), GB/s;
      mfma  the int8 matrix cores alone (coli_moe_roof_mfma_i8), TOPS.
    Median of five timed repetitions after one untimed one."""
    import torch
    sink = torch.empty(q.coli_moe_roof_sink_words(), dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()

    def timed(fn, stream):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        return sorted(ts)[2]

    if kind == "hbm":
        n = 4 << 30
        buf = torch.empty(n, dtype=torch.uint8, device="cuda")
        t = timed(lambda: q.coli_moe_roof_stream_read(buf, sink, st), st)
        val, unit, how = n / t / 1e9, "GB/s", "streaming read of 4 GiB, 16-byte loads"
        del buf
    elif kind == "mfma":
        iters = 200
        t = timed(lambda: q.coli_moe_roof_mfma_i8(iters, sink, st), st)
        ops = 2048 * 4 * iters * 4 * 2 * 32 * 32 * 32
        val, unit, how = ops / t / 1e12, "TOPS", "v_mfma_i32_32x32x32_i8 loop, 8192 wavefronts, register operands"
    else:
        raise ValueError(kind)
    r = res["roofline"]
    r["measured_peak"] = {"value": round(val, 1), "unit": unit, "how": how}
    if r.get("unit") == unit and val > 0:
        r["frac_of_measured"] = round(r["achieved"] / val, 4)


def kernel_times(q, run):
    """Average duration (us) and launch count per kernel kind over one eager
    call of run(), every launch bracketed by HIP events recorded at the
    kernel's own start and end."""
    import torch
    q.coli_moe_timing_enable(True)
    run()
    torch.cuda.synchronize()
    q.coli_moe_timing_enable(False)
    us, n_l = {}, {}
    for name, k in KINDS:
        ms, n = q.coli_moe_timing_read(k)
        if n:
            us[name] = 1e3 * ms / n
            n_l[name] = n
    return us, n_l


def run_prefill(args, q, synth, embedded=False):
    """Batch-union prefill: GLM-5.2-shaped layer, all experts resident, one
    step = coli_moe_layer over a batch of args.tokens Zipf-routed tokens
    (two batches alternate).  embedded: return the record (for the default
    run's line) instead of printing it."""
    import numpy as np
    import torch

    mx = args.wformat == "mxfp4"
    if mx and args.group_size:
        raise SystemExit("--wformat mxfp4 takes no --group-size")
    spec = synth.GLM_MX if mx else (synth.GLM_GS64 if args.group_size else synth.GLM)
    pf_kernel = "k_pf_gateup_mx" if mx else ("k_pf_gateup<4,gs64>" if spec.group else "k_pf_gateup<4>")
    # the peak of the products' own format: int8, or FP8 for the MXFP4
    # kernels' E2M1 x E4M3 products (the FP8 rate; the split of each Q8_0
    # code into two E4M3 parts doubles their matrix-core work)
    peak = FP8_PEAK_TOPS if mx else INT8_PEAK_TOPS
    dims = q.make_dims(spec)
    S, H, I, E, K = args.tokens, spec.hidden, spec.inter, spec.n_experts, spec.top_k
    bb = spec.blob_bytes
    t0 = time.time()
    host = torch.empty((E + 1) * bb, dtype=torch.uint8, pin_memory=True)
    fill = synth.mx_cdf_expert_into if mx else synth.cdf_expert_into
    for e in range(E + 1):
        fill(host.data_ptr() + e * bb, args.seed, 0, e, spec)
    dev = host.cuda()
    table = torch.tensor([dev.data_ptr() + e * bb for e in range(E)], dtype=torch.int64, device="cuda")
    shared = dev.data_ptr() + E * bb
    d = synth.layer_inputs(args.seed, 0, spec, 1)
    W = torch.from_numpy(d["router_w"]).cuda()
    bias = torch.zeros(E, dtype=torch.float32, device="cuda")
    xs_host = [synth.prefill_hidden_states(args.seed, 0, spec, S, batch=b) for b in range(2)]
    xs = [torch.from_numpy(x).cuda() for x in xs_host]
    ws = torch.zeros(q.coli_moe_workspace_bytes(dims, S), dtype=torch.uint8, device="cuda")
    idx = [torch.empty((S, K), dtype=torch.int32, device="cuda") for _ in range(2)]
    wts = [torch.empty((S, K), dtype=torch.float32, device="cuda") for _ in range(2)]
    out = [torch.empty((S, H), dtype=torch.float32, device="cuda") for _ in range(2)]
    log(f"prefill setup: {E + 1} experts resident, 2 batches of {S} tokens ({time.time() - t0:.1f} s)")

    def step(s):
        b = s % 2
        q.coli_moe_layer(dims, xs[b], W, bias, table, shared, idx[b], wts[b], out[b], ws)

    step(0)
    step(1)
    rc = q.coli_moe_status(ws)
    if rc != 0:
        raise RuntimeError(f"device status {rc}: {q.coli_moe_last_error()}")
    routed = [i.cpu().numpy() for i in idx]
    counts = np.bincount(routed[0].ravel(), minlength=E)
    kernel_us, launches = kernel_times(q, lambda: [step(s) for s in range(2)])

    G, reps, reps_w, warm_eager = graph_plan(args.steps, args.warmup, 10)
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        for s in range(G):
            step(s)
    torch.cuda.synchronize()
    for _ in range(reps_w):
        graph.replay()
    for s in range(warm_eager):
        step(s)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    rep_ev = replay_timed(graph, reps)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t1
    steps = reps * G
    rc = q.coli_moe_status(ws)
    if rc != 0:
        raise RuntimeError(f"device status after replay {rc}: {q.coli_moe_last_error()}")
    ms_per_step = 1e3 * elapsed / steps

    # algorithmic work: every (token, expert) pair of the batch, shared expert
    # included, costs 2 H I MACs in gate/up and H I in down (2 ops a MAC)
    pairs = S * K + S * spec.n_shared
    ops_gateup = 2 * 2 * H * I * pairs
    ops_layer = 3 * 2 * H * I * pairs
    g_us = kernel_us["gateup"]
    achieved = ops_gateup / (g_us * 1e-6) / 1e12
    layer_tops = ops_layer / (ms_per_step * 1e-3) / 1e12
    hbm_bytes = (E + 1) * bb + E * H * 4
    res = {
        "metric": METRIC,
        "value": round(S / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e2m1xe4m3->f32" if mx else "i8xi4->i32,f32",
        "data": "synthetic (seeded; GLM-5.2-shaped random-code experts, Zipf(1.1)-routed tokens)",
        "config": {
            "workload": f"GLM-5.2-shaped MoE prefill layer, {S} tokens/step: hidden 6144, expert inter 2048, "
                        "256 routed experts top-8 + 1 shared, "
                        + ("MXFP4 weights (E2M1 codes, one E8M0 scale per 32 codes of a row) on the FP4 "
                           "matrix cores, " if mx else "int4 weights with one scale per 64 codes of a row, "
                           if spec.group else "int4 per-row-scaled weights, ") + "Q8_0 activations, "
                        "fp32 router gate, zero bias; Zipf(1.1) expert popularity; all 257 experts resident",
            "tokens_per_step": S, "graph_steps": G, "graph_replays": reps, "kernels": args.kernels,
            "routing": {"unique": int((counts > 0).sum()), "min": int(counts[counts > 0].min()),
                        "median": float(np.median(counts[counts > 0])), "max": int(counts.max())},
        },
        "roofline": {
            "bound": "mfma", "kernel": pf_kernel,
            "achieved": round(achieved, 1), "peak": peak, "unit": "TOPS",
            "frac": round(achieved / peak, 4), "traffic": counted_traffic(pf_kernel),
            "algorithmic_ops_per_launch": ops_gateup, "avg_launch_us": round(g_us, 3),
        },
        "layer_tops": round(layer_tops, 1),
        "layer_frac": round(layer_tops / peak, 4),
        # the attainable roofline of the whole layer: min(peak, its
        # arithmetic intensity (ops per algorithmic HBM byte) x HBM peak)
        "layer_ops_per_byte": round(ops_layer / hbm_bytes, 1),
        "layer_attainable_tops": round(min(peak, ops_layer / hbm_bytes * HBM_PEAK_GBS / 1e3), 1),
        "layer_frac_of_attainable": round(layer_tops / min(peak, ops_layer / hbm_bytes * HBM_PEAK_GBS / 1e3), 4),
        "layer_hbm_gbs": round(hbm_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "ms_per_step_p10_p50_p90": replay_spread(rep_ev, G),
        "kernel_avg_us": {k: round(v, 3) for k, v in kernel_us.items()},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_prefill(args, spec, xs_host[0], d, host.numpy(), routed[0])
    add_measured_roof(res, q, "mfma")
    if embedded:
        for k in ("metric", "n_gpus", "higher_is_better", "scaling", "vs_baseline"):
            res.pop(k)
        res["tokens_per_s"] = res.pop("value")
        res.pop("unit")
        del graph, dev, host, xs, ws, idx, wts, out
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        return res
    print(json.dumps(res), flush=True)


PCIE_PEAK_GBS = 64.0  # PCIe Gen5 x16, one direction


def run_tiered(args, q, synth):
    """Tiered streaming decode: every step routes one token through all
    layers; each layer's experts beyond its HBM slots come from pinned host
    memory through coli_moe_stage_experts, the forward running the resident
    experts first (pending mask) and the copied ones after the copy event."""
    import numpy as np
    import torch

    from quantized_expert_ffn_amd.tier import ExpertTier

    spec = synth.GLM if args.tier_bits == 4 else synth.GLM_INT2
    dims = q.make_dims(spec)
    L, HL = args.tier_layers, min(args.host_layers, args.tier_layers)
    H, E, K = spec.hidden, spec.n_experts, spec.top_k
    bb = spec.blob_bytes
    spl = int(args.cache_gb * 1e9 // bb) // L
    if spl < K:
        raise SystemExit(f"{spl} cache slots per layer is fewer than top-{K}")
    n_steps = args.warmup + args.steps
    t0 = time.time()
    host = torch.empty(HL * E * bb, dtype=torch.uint8, pin_memory=True)
    hp = host.data_ptr()
    for hl in range(HL):
        for e in range(E):
            synth.cdf_expert_into(hp + (hl * E + e) * bb, args.seed, hl, e, spec)
    log(f"tiered: {HL} layers x {E} experts in pinned host memory ({HL * E * bb / 1e9:.1f} GB, "
        f"{time.time() - t0:.1f} s)")
    tmp = torch.empty(bb, dtype=torch.uint8, pin_memory=True)
    shared = torch.empty(L * bb, dtype=torch.uint8, device="cuda")
    for l in range(L):
        synth.cdf_expert_into(tmp.data_ptr(), args.seed, l % HL, E, spec)
        shared[l * bb:(l + 1) * bb].copy_(tmp)
    cache = torch.empty(L * spl * bb, dtype=torch.uint8, device="cuda")
    Ws, biases, xs = [], [], []
    Wh = [synth.router_weights(args.seed, l, spec) for l in range(L)]
    traces = [synth.reuse_trace(args.seed, l, spec, n_steps) for l in range(L)]
    for l in range(L):
        W = Wh[l]
        t_here = synth.trace_target_logits(args.seed, l, spec, traces[l])
        if args.lookahead and l + 1 < L:
            # layer l's state also carries the next layer's predicted set
            pred = synth.predicted_sets(args.seed, l + 1, spec, traces[l + 1])
            t_next = synth.trace_target_logits(args.seed, l + 1, spec, pred)
            x = synth.lookahead_hidden_states(W, Wh[l + 1], t_here, t_next, args.seed, l, stream=11)
        else:
            x = synth.shaped_hidden_states(W, t_here, args.seed, l, stream=11)
        Ws.append(torch.from_numpy(W).cuda())
        biases.append(torch.from_numpy(synth.router_bias(args.seed, l, spec)).cuda())
        xs.append(torch.from_numpy(x).cuda())
    del Wh
    torch.cuda.synchronize()
    log(f"tiered setup: {L} layers, {spl} HBM slots each ({L * spl * bb / 1e9:.1f} GB cache), "
        f"{time.time() - t0:.1f} s")

    cp = cache.data_ptr()
    tier = ExpertTier(L, E, spl, bb, slot_addr=lambda l, s: cp + (l * spl + s) * bb,
                      host_addr=lambda l, e: hp + ((l % HL) * E + e) * bb)
    ws = torch.zeros(q.coli_moe_workspace_bytes(dims, 1), dtype=torch.uint8, device="cuda")
    idx = torch.empty((1, K), dtype=torch.int32, device="cuda")
    wts = torch.empty((1, K), dtype=torch.float32, device="cuda")
    out = torch.empty((1, H), dtype=torch.float32, device="cuda")
    idx_host = torch.empty((1, K), dtype=torch.int32, pin_memory=True)
    idx_pred = torch.empty((1, K), dtype=torch.int32, device="cuda")
    wts_pred = torch.empty((1, K), dtype=torch.float32, device="cuda")
    pred_host = torch.empty((1, K), dtype=torch.int32, pin_memory=True)
    last_pred = [None] * L   # the prediction made for each layer, for the measured recall
    R = 16
    ring = torch.empty((R, E), dtype=torch.int64, pin_memory=True)
    ring_ev = [None] * R
    dev_tab = torch.zeros((L, E), dtype=torch.int64, device="cuda")
    copy = torch.cuda.Stream()
    comp = torch.cuda.current_stream()
    got = torch.cuda.Event()
    copies_timed = []
    state = {"r": 0, "bytes": 0, "copies": 0, "layer_steps": 0, "pref_bytes": 0, "pref_copies": 0,
             "recall_hits": 0, "recall_n": 0, "early": 0}

    def stage(copies, ev, timed, kind):
        """Copies on the copy stream, bracketed by timing events; ev (may be
        None) recorded after them.  Demand copies also wait for the compute
        stream's work so far; look-ahead copies do not (they fill the next
        layer's slots, whose last reader finished before the host read this
        layer's routing), so they run while this layer computes."""
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if kind == "demand":
            copy.wait_stream(comp)
        c0.record(copy)
        q.coli_moe_stage_experts([c[1] for c in copies], [c[2] for c in copies], bb, copy, ev)
        c1.record(copy)
        if timed:
            copies_timed.append((c0, c1, len(copies)))
            state["bytes" if kind == "demand" else "pref_bytes"] += len(copies) * bb
            state["copies" if kind == "demand" else "pref_copies"] += len(copies)

    def layer_step(s, l, timed):
        q.coli_moe_route(dims, xs[l][s:s + 1], Ws[l], biases[l], idx, wts, ws)
        ahead = args.lookahead and l + 1 < L
        if ahead:
            # the next layer's router on this layer's state: its predicted set
            q.coli_moe_route(dims, xs[l][s:s + 1], Ws[l + 1], biases[l + 1], idx_pred, wts_pred, ws)
            pred_host.copy_(idx_pred, non_blocking=True)
        idx_host.copy_(idx, non_blocking=True)
        got.record(comp)
        got.synchronize()
        chosen = idx_host[0].tolist()
        if timed and last_pred[l] is not None:
            state["recall_hits"] += len(set(chosen) & set(last_pred[l]))
            state["recall_n"] += K
        table, copies, early = tier.plan_with_ahead(l, chosen)
        ev = None
        mask = None
        if copies or early:
            # experts copied now, and experts a look-ahead copied earlier whose
            # copies may still be running, wait for everything staged so far
            ev = torch.cuda.Event()
            if copies:
                stage(copies, ev, timed, "demand")
            else:
                ev.record(copy)
            mask = np.zeros(E, np.uint8)
            mask[[c[0] for c in copies] + list(early)] = 1
            if timed:
                state["early"] += len(early)
        r = state["r"]
        state["r"] = (r + 1) % R
        if ring_ev[r] is not None:
            ring_ev[r].synchronize()
        ring[r].copy_(torch.tensor(table, dtype=torch.int64))
        dev_tab[l].copy_(ring[r], non_blocking=True)
        ring_ev[r] = torch.cuda.Event()
        ring_ev[r].record(comp)
        q.coli_moe_forward(dims, xs[l][s:s + 1], idx, wts, dev_tab[l], shared.data_ptr() + l * bb, out, ws,
                           pending_mask=mask, pending_ready=ev)
        if ahead:
            # stage the next layer's predicted misses into its slots while this
            # layer computes (behind this layer's own copies on the copy stream)
            pred = pred_host[0].tolist()
            last_pred[l + 1] = pred
            pcopies = tier.prefetch(l + 1, pred)
            if pcopies:
                stage(pcopies, None, timed, "prefetch")
        if timed:
            state["layer_steps"] += 1

    for s in range(args.warmup):
        for l in range(L):
            layer_step(s, l, False)
    torch.cuda.synchronize()
    rc = q.coli_moe_status(ws)
    if rc != 0:
        raise RuntimeError(f"device status {rc}: {q.coli_moe_last_error()}")
    h0, m0 = tier.hits, tier.misses
    t1 = time.perf_counter()
    for s in range(args.warmup, n_steps):
        for l in range(L):
            layer_step(s, l, True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t1
    rc = q.coli_moe_status(ws)
    if rc != 0:
        raise RuntimeError(f"device status after the timed steps {rc}: {q.coli_moe_last_error()}")
    hits, misses = tier.hits - h0, tier.misses - m0
    roof = pcie_copy_roof(q, tier, L, bb, copy)
    copy_ms = sum(a.elapsed_time(b) for a, b, _ in copies_timed)
    staged = state["bytes"] + state["pref_bytes"]
    copy_gbs = staged / (copy_ms * 1e-3) / 1e9 if copy_ms > 0 else 0.0
    steps = args.steps
    res = {
        "metric": METRIC,
        "value": round(steps / elapsed, 3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * elapsed / steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8xi%d->i32,f32" % spec.wbits,
        "data": "synthetic (seeded; GLM-5.2-shaped random-code experts, 60%-reuse routing trace)",
        "config": {
            "workload": f"tiered streaming decode: {L} GLM-5.2-shaped layers (int{spec.wbits}, "
                        f"{bb / 1e6:.2f} MB/expert, {L * (E + 1) * bb / 1e9:.0f} GB in all), 1 token/step through "
                        f"every layer, {args.cache_gb:g} GB HBM cache as {spl} LRU slots per layer, other experts "
                        "in pinned host memory staged by hipMemcpyAsync on a side stream, shared experts resident",
            "layers": L, "slots_per_layer": spl, "host_layers_distinct": HL, "lookahead": bool(args.lookahead),
        },
        "roofline": {
            "bound": "pcie", "kernel": "coli_moe_stage_experts (hipMemcpyAsync host to device)",
            "achieved": round(copy_gbs, 2), "peak": PCIE_PEAK_GBS, "unit": "GB/s",
            "frac": round(copy_gbs / PCIE_PEAK_GBS, 4), "traffic": None,
            "bytes_per_copy_batch": round(staged / max(1, len(copies_timed))),
            "copy_batches": len(copies_timed), "copy_busy_ms": round(copy_ms, 3),
            "measured_peak": roof,
            "frac_of_measured": round(copy_gbs / roof["value"], 4) if roof else None,
        },
        "staged_gb_per_token": round(staged / steps / 1e9, 3),
        "pcie_gbs_wall": round(staged / elapsed / 1e9, 2),
        "copy_busy_frac_of_wall": round(copy_ms * 1e-3 / elapsed, 4),
        "hit_rate": round(hits / max(1, hits + misses), 4),
        "misses_per_layer_step": round(misses / max(1, state["layer_steps"]), 3),
        "layer_step_ms": round(1e3 * elapsed / max(1, state["layer_steps"]), 4),
    }
    if args.lookahead:
        ls = max(1, state["layer_steps"])
        res["lookahead"] = {
            "recall_measured": round(state["recall_hits"] / max(1, state["recall_n"]), 4),
            "prefetched_per_layer_step": round(state["pref_copies"] / ls, 3),
            "prefetched_then_used_per_layer_step": round(state["early"] / ls, 3),
            "demand_copies_per_layer_step": round(state["copies"] / ls, 3),
            "prefetch_gb_per_token": round(state["pref_bytes"] / steps / 1e9, 3),
        }
    print(json.dumps(res), flush=True)


def _oracle_threads():
    import oracle
    return oracle.threads()


def pcie_copy_roof(q, tier, L, bb, copy):
    """The pinned-host-to-HBM copy ceiling on this machine: 16 blob copies in one
    coli_moe_stage_experts call, timed with events on the copy stream (median
    of five).  Each copy rewrites a resident slot with the bytes it already
    holds (the slot's expert from the pinned host set), so the tier is left
    as it was; the sources are the run's pinned buffer, alive until the
    synchronisation at the end."""
    import torch
    pairs = []
    for l in range(L):
        for e, slot in tier.lru[l].resident().items():
            pairs.append((tier.host_addr(l, e), tier.slot_addr(l, slot)))
            if len(pairs) == 16:
                break
        if len(pairs) == 16:
            break
    if len(pairs) < 16:
        return None
    src, dst = [p[0] for p in pairs], [p[1] for p in pairs]
    torch.cuda.synchronize()
    ts = []
    for rep in range(6):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(copy)
        q.coli_moe_stage_experts(src, dst, bb, copy, None)
        b.record(copy)
        b.synchronize()
        if rep:
            ts.append(a.elapsed_time(b) * 1e-3)
    torch.cuda.synchronize()
    t = sorted(ts)[2]
    return {"value": round(16 * bb / t / 1e9, 2), "unit": "GB/s",
            "how": f"16 pinned-host-to-HBM copies of {bb} bytes in one stage call on the copy stream, median of 5"}


def cpu_baseline_prefill(args, spec, x, d, host, routed):
    """The CPU oracle on the first tokens of the prefill batch (each token's
    output depends on that token only): the multi-threaded build over
    tokens on all of this host's threads, as many tokens as fit the time
    budget at its rate, and the single-threaded build on a few tokens."""
    import numpy as np

    import oracle
    E, bb = spec.n_experts, spec.blob_bytes
    blobs = [host[e * bb:(e + 1) * bb] for e in range(E)]
    shared = host[E * bb:(E + 1) * bb]
    bias = np.zeros(E, np.float32)
    n1, spent1 = 0, 0.0
    while spent1 < args.cpu_seconds / 4 and n1 < x.shape[0]:
        t = time.perf_counter()
        oracle.layer(spec, x[n1:n1 + 1], d["router_w"], bias, blobs, shared)
        spent1 += time.perf_counter() - t
        n1 += 1
    rate1 = n1 / spent1
    thr = _oracle_threads()
    n = int(min(x.shape[0], max(thr, int(round(rate1 * thr * args.cpu_seconds / thr)) * thr)))
    t = time.perf_counter()
    oracle.layer(spec, x[:n], d["router_w"], bias, blobs, shared, parallel=True)
    spent = time.perf_counter() - t
    return {"value": round(n / spent, 4), "unit": "tokens/s", "cores": thr, "kind": "oracle",
            "sample": f"first {n} tokens of the 2048-token batch (route + 9 experts + combine each) through the "
                      f"oracle's OpenMP build, tokens spread over {thr} threads, {spent:.1f} s",
            "single_core": {"value": round(rate1, 4), "unit": "tokens/s", "cores": 1,
                            "sample": f"first {n1} tokens one at a time, single-threaded build, {spent1:.1f} s"}}


def _hipbuild():
    """The library's build module, loaded by path: importing the package
    itself needs the built library."""
    import importlib.util
    path = os.path.join(ROOT, "quantized_expert_ffn_amd", "build.py")
    spec = importlib.util.spec_from_file_location("coli_moe_hip_build", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def counted_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by a device copy), or None when
    there is none or the kernel's sources changed since it was taken."""
    import glob
    import hashlib
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path) as f:
            for line in f:
                if not line.startswith("traffic_json: "):
                    continue
                rec = json.loads(line[len("traffic_json: "):])
                if rec.get("kernel") != kernel:
                    continue
                h = hashlib.sha256()
                for src in rec["sources"]:
                    with open(os.path.join(ROOT, src), "rb") as s:
                        h.update(s.read())
                if h.hexdigest() == rec["sha256"]:
                    return int(rec["read_bytes"]) + int(rec["write_bytes"])
    return None


def cpu_baseline(args, spec, xs_host, layers, L, S=1):
    """The CPU oracle on a bounded sample of the same workload: whole
    token-layer steps (route + the token's experts + shared + combine).  The
    single-threaded build runs the benchmark's own steps (their layers) one
    at a time; the multi-threaded build (the same source, its loop over
    independent tokens on all of this host's threads) runs a batch of
    hidden states of layer 0 drawn the same way, as many as fit the time
    budget at that rate.  Expert generation is excluded from both."""
    import numpy as np

    import oracle
    import synth
    n1, spent1 = 0, 0.0
    while spent1 < args.cpu_seconds / 3 and n1 < xs_host.shape[0]:
        l = (n1 // S) % L
        d = synth.layer_inputs(args.seed, l, spec, 1)
        x = xs_host[n1:n1 + 1]
        idx, w, _, _ = oracle.route(spec, x, d["router_w"], d["bias"])
        blobs = [None] * spec.n_experts
        for e in idx[0]:
            blobs[int(e)] = synth.cdf_expert(args.seed, l, int(e), spec)
        shared = synth.cdf_expert(args.seed, l, spec.n_experts, spec)
        t = time.perf_counter()
        oracle.layer(spec, x, d["router_w"], d["bias"], blobs, shared)
        spent1 += time.perf_counter() - t
        n1 += 1
    rate1 = n1 / spent1
    thr = _oracle_threads()
    # as many tokens as the budget allows at the single-threaded rate on
    # every thread, a whole number of tokens per thread
    n = int(round(rate1 * thr * args.cpu_seconds / thr)) * thr
    n = int(max(thr, min(n, 16 * thr)))
    d = synth.layer_inputs(args.seed, 0, spec, 1)
    x = synth.hidden_states(args.seed, 2000, n, spec.hidden)
    idx, w, _, _ = oracle.route(spec, x, d["router_w"], d["bias"], parallel=True)
    used = sorted(set(idx.ravel().tolist()))
    blobs = [None] * spec.n_experts
    for e in used:
        blobs[e] = synth.cdf_expert(args.seed, 0, e, spec)
    shared = synth.cdf_expert(args.seed, 0, spec.n_experts, spec)
    t = time.perf_counter()
    oracle.layer(spec, x, d["router_w"], d["bias"], blobs, shared, parallel=True)
    spent = time.perf_counter() - t
    del blobs
    return {"value": round(n / spent, 4), "unit": "tokens/s", "cores": thr, "kind": "oracle",
            "sample": f"{n} token-layer steps of the same workload (layer 0, N(0,1) hidden states; route + 9 "
                      f"experts + combine each) through the oracle's OpenMP build, tokens spread over {thr} "
                      f"threads, {spent:.1f} s; expert generation excluded",
            "single_core": {"value": round(rate1, 4), "unit": "tokens/s", "cores": 1,
                            "sample": f"{n1} of the benchmark's token-layer steps one at a time, single-threaded "
                                      f"build, {spent1:.1f} s"}}


if __name__ == "__main__":
    main()
