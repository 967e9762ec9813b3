#!/usr/bin/env python3
"""Throughput of the routed MoE FFN over Q4_K / Q8_0 experts on one MI355X.

A step is one pass of the whole hot path (route -> [quantize] -> expert FFN ->
combine) through every layer of a stack of distinct seeded synthetic layers
resident in HBM, for one batch of fresh router logits and activations per
layer.  Default workload: Sage-A1.5-like decode (1 token, hidden 2048, 256
experts, top-8, intermediate 512, Q4_K gate/up/down, 40 layers).

Prints ONE JSON line on stdout: MoE-layer tokens/s (whole job), the roofline of
the dominant kernel call measured with HIP events on its own stream, and the CPU
oracle timed on a bounded sample of the same workload.  Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0         # MI355X dense int8 MFMA


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def traffic_from_profiles(config: str):
    """HBM bytes per launch of the dominant call from committed rocprofv3 counter runs, or None
    when they were taken on other kernel sources."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p)).get(config)
    except (ValueError, OSError):
        return None
    from quantized_moe_ffn_amd.profiling import kernel_source_hash
    if not rec or rec.get("kernel_hash") != kernel_source_hash(config):
        return None
    return rec.get("bytes_per_launch")


def main() -> int:
    from quantized_moe_ffn_amd import synth
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="sage_decode", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--layers", type=int, default=None, help="override the number of distinct layers")
    ap.add_argument("--replays", type=int, default=8, help="distinct input sets cycled over the steps")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", choices=["on", "off"], default="on", help="replay each step as a HIP graph")
    ap.add_argument("--router", action="store_true",
                    help="compute each layer's logits on the GPU from x and a seeded fp32 [E][H] router "
                         "matrix (moe_router_logits) inside the timed step")
    ap.add_argument("--tokens", type=int, default=None,
                    help="override the tokens per layer call (a decode batch or verify window of the "
                         "same layer shape)")
    ap.add_argument("--experts", type=int, default=None,
                    help="override the routed experts per layer (e.g. one GPU's share under expert parallelism)")
    ap.add_argument("--top-k", type=int, default=None, help="override the routed experts per token")
    ap.add_argument("--path", choices=["auto", "decode", "int8"], default=None,
                    help="FFN path (default: the workload's own; auto takes the decode path up to 8 tokens)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: the MoE FFN path here is built and measured on a "
              "single MI355X (--gpus %d requested; multi-GPU sharding is a design note, not built)"
              % args.gpus, file=sys.stderr)
        return 2

    import torch
    import quantized_moe_ffn_amd as qm
    from quantized_moe_ffn_amd import layers as qlayers

    if not os.path.exists(qm.LIB_PATH):
        from quantized_moe_ffn_amd import build as hb
        hb.build()
    qm.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    w = synth.WORKLOADS[args.config]
    if args.tokens is not None:
        if args.tokens < 1:
            print("--tokens must be at least 1", file=sys.stderr)
            return 2
        if args.tokens != w.tokens:
            w = dataclasses.replace(w, name="%s_t%d" % (w.name, args.tokens), tokens=args.tokens)
    if args.experts is not None or args.top_k is not None:
        E2 = args.experts if args.experts is not None else w.n_experts
        k2 = args.top_k if args.top_k is not None else w.top_k
        if not (1 <= k2 <= min(E2, 16)):
            print("need 1 <= top-k <= min(experts, 16)", file=sys.stderr)
            return 2
        w = dataclasses.replace(w, name="%s_e%d_k%d" % (w.name, E2, k2), n_experts=E2, top_k=k2)
    L = args.layers or w.layers
    R = max(1, args.replays)
    T, H, E, k, I = w.tokens, w.hidden, w.n_experts, w.top_k, w.inter
    flags = qm.MOE_FFN_INT8 if w.int8_path else qm.MOE_FFN_DECODE
    if args.path is not None:
        flags = {"auto": qm.MOE_FFN_AUTO, "decode": qm.MOE_FFN_DECODE, "int8": qm.MOE_FFN_INT8}[args.path]
        int8 = flags == qm.MOE_FFN_INT8 or (flags == qm.MOE_FFN_AUTO and T > qm.AUTO_DECODE_MAX_T)
        if int8 != w.int8_path:
            # the roofline, the dtype and the oracle's quantisation points follow the path taken
            w = dataclasses.replace(w, name="%s_%s" % (w.name, "int8" if int8 else "decode"), int8_path=int8)

    log("[bench] building %d layers of %s (%.2f GB of expert weights)"
        % (L, w.name, L * (E * w.expert_bytes() + (w.expert_bytes() if w.shared else 0)) / 1e9))
    t0 = time.time()
    stack = [qlayers.make_layer(w, seed=0, index=l, device=dev) for l in range(L)]
    torch.cuda.synchronize()
    log("[bench] layers ready in %.1f s" % (time.time() - t0))

    inputs = []
    for r in range(R):
        row = []
        for l in range(L):
            lg, x = qlayers.inputs_np(w, seed=0, index=l, replay=r)
            row.append((torch.from_numpy(lg).to(dev), torch.from_numpy(x).to(dev)))
        inputs.append(row)
    bufs = qm.LayerBuffers(stack[0].layer, T, k, flags, device=dev)
    routers = None
    if args.router:
        # seeded N(0, 1/H) fp32 router rows, one matrix per layer; the logits of
        # every layer call then come from the GPU router stage
        routers = [torch.from_numpy((np.random.default_rng((0, l, 0x52)).standard_normal((E, H))
                                     / np.sqrt(H)).astype(np.float32)).to(dev) for l in range(L)]
        lgbuf = torch.empty((T, E), dtype=torch.float32, device=dev)
        for r in range(R):
            for l in range(L):
                qm.moe_router_logits(inputs[r][l][1], routers[l], lgbuf)
                inputs[r][l] = (lgbuf.clone(), inputs[r][l][1])

    def run_replay(r, stream):
        row = inputs[r]
        for l in range(L):
            lg, x = row[l]
            if routers is not None:
                qm.moe_router_logits(x, routers[l], lgbuf, stream)
                lg = lgbuf
            qm.forward(stack[l].layer, lg, x, k, bufs, flags=flags, stream=stream)

    # unique experts per (replay, layer): algorithmic bytes of each layer call
    stream = torch.cuda.current_stream()
    uniq = np.zeros((R, L), np.int64)
    for r in range(R):
        for l in range(L):
            lg, _ = inputs[r][l]
            qm.moe_route_topk(lg, k, bufs.routing, True, bufs.route_ws, stream)
            uniq[r, l] = int(bufs.routing.n_active.item())
    qm.moe_check_device_errors()
    per_expert = w.expert_bytes()
    shared_bytes = w.expert_bytes() if w.shared else 0
    bytes_rl = uniq * per_expert + shared_bytes           # expert weight bytes each layer call streams
    if routers is not None:
        bytes_rl = bytes_rl + E * H * 4                   # and the router matrix

    graphs = None
    if args.graph == "on":
        log("[bench] capturing %d graphs of %d layer calls" % (R, L))
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        graphs = []
        with torch.cuda.stream(cap):
            run_replay(0, cap)           # warm the allocator/library on the capture stream
            for r in range(R):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cap):
                    run_replay(r, cap)
                graphs.append(g)
        stream.wait_stream(cap)
        torch.cuda.synchronize()

    def step(s):
        if graphs is not None:
            graphs[s % R].replay()
        else:
            run_replay(s % R, stream)

    log("[bench] warmup %d steps" % args.warmup)
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    qm.moe_check_device_errors()

    log("[bench] timing %d steps x %d layers (graphs %s)" % (args.steps, L, args.graph))
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record(stream)
    step_ev = []
    for s in range(args.steps):
        step(args.warmup + s)
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        step_ev.append(e)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = ev0.elapsed_time(ev1)
    # per-step spread of the layer call (each step is L calls)
    step_us = np.array([(ev0 if s == 0 else step_ev[s - 1]).elapsed_time(step_ev[s]) * 1e3 / L
                        for s in range(args.steps)])
    pct = {q: round(float(np.percentile(step_us, q)), 3) for q in (10, 50, 90)}
    qm.moe_check_device_errors()
    ms_per_step = ms_total / args.steps
    tokens = T * L * args.steps
    value = tokens / (ms_total / 1e3)
    n_launch = L * args.steps
    avg_us = ms_total * 1e3 / n_launch
    dom_bytes = sum(int(bytes_rl[(args.warmup + s) % R].sum()) for s in range(args.steps))
    log("[bench] %.3f ms/step (wall %.3f ms/step), %.0f layer-tokens/s, %.2f us per layer call"
        % (ms_per_step, wall * 1e3 / args.steps, value, avg_us))

    # dominant call: the layer call (moe_forward), whose average duration is the
    # timed region divided by the number of calls in it
    if w.int8_path:
        ops = 2.0 * T * k * 3 * H * I + (2.0 * T * 3 * H * I if w.shared else 0.0)
        achieved = ops / (avg_us / 1e6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": INT8_PEAK_TOPS, "unit": "TFLOP/s",
                "frac": round(achieved / INT8_PEAK_TOPS, 4), "traffic": traffic_from_profiles(w.name),
                "kernel": ("moe_router_logits + " if routers is not None else "") +
                          "moe_forward (int8 path: route, quantize, gate/up, requantize, down, combine)",
                "ops_per_launch": ops, "avg_launch_us": round(avg_us, 3)}
    else:
        achieved = dom_bytes / (ms_total / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic_from_profiles(w.name),
                "kernel": ("moe_router_logits + " if routers is not None else "") +
                          "moe_forward (decode: route+gate/up+SiLU kernel, down+combine kernel)",
                "bytes_per_launch": round(dom_bytes / n_launch), "avg_launch_us": round(avg_us, 3)}
    log("[bench] layer call: %.2f us, %s %s" % (avg_us, roof["achieved"], roof["unit"]))

    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        # with --router the oracle takes the logits the GPU router produced
        # (untimed, above) as its input
        cpu, parity = cpu_baseline(w, stack, inputs, bufs, flags, k, args.cpu_seconds)

    rec = {
        "metric": "MoE-layer tokens/s + achieved HBM GB/s (decode), int8 TOPS (prefill)",
        "value": round(value, 1),
        "unit": "layer-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8" if w.int8_path else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": T, "hidden": H, "experts": E, "top_k": k, "inter": I,
                   "shared_expert": w.shared, "layers": L, "replays": R,
                   "formats": {"gate": fmt(w.qt_gate), "up": fmt(w.qt_up), "down": fmt(w.qt_down)},
                   "parallelism": "single GPU", "graphs": args.graph,
                   "router": "fp32 [E][H], moe_router_logits in the timed step" if routers is not None else None},
        "hbm_GBps_end_to_end": round(dom_bytes / (ms_total / 1e3) / 1e9, 1),
        "layer_call_us_p10_p50_p90": [pct[10], pct[50], pct[90]],
        "hbm_copy_GBps_measured": copy_bandwidth(torch, dev),
        "roofline": roof,
        "cpu_baseline": cpu,
        "parity_max_normwise_err": parity,
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
    }
    print(json.dumps(rec), flush=True)
    return 0


def copy_bandwidth(torch, dev) -> float:
    """Measured device-to-device copy rate of 1 GiB (bytes read + written per second, GB/s):
    the practical streaming ceiling the decode roofline is read against."""
    n = 1 << 28
    x = torch.ones(n, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    y.copy_(x)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record()
    for _ in range(reps):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    rate = 2.0 * 4 * n * reps / (e0.elapsed_time(e1) / 1e3) / 1e9
    del x, y
    torch.cuda.empty_cache()
    return round(rate, 1)


def fmt(qt):
    return {7: "Q5_1", 8: "Q8_0", 12: "Q4_K", 13: "Q5_K"}[qt]


def cpu_baseline(w, stack, inputs, bufs, flags, k, budget_s):
    """The oracle (as it stands) on a bounded sample of the same workload, on this host's
    cores; also checks the GPU outputs of the sampled tokens against it."""
    import torch
    import oracle
    import quantized_moe_ffn_amd as qm
    T = w.tokens
    tok_sample = np.arange(T) if T <= 64 else np.linspace(0, T - 1, 16).round().astype(np.int64)
    mode = 1 if w.int8_path else 0
    spent, tokens_done, layers_done, errs = 0.0, 0, 0, []
    qt = (w.qt_gate, w.qt_up, w.qt_down)
    cache = []          # host copies of the first items, reused once every item has been seen
    kCache = 32

    def run_oracle(lg, x, hb, remap, shared):
        idx, wts = oracle.route_topk(lg, k)
        oracle.bucket(idx, w.n_experts)
        pe = remap[idx.reshape(-1)]
        bad = bool(np.any(pe < 0))      # the oracle chose an expert the GPU did not: parity failure
        pe = np.maximum(pe, 0)
        pt = np.repeat(np.arange(len(tok_sample)), k)
        y = oracle.expert_ffn(hb["gate"], hb["up"], hb["down"], qt, w.hidden, w.inter, pe, pt, x, mode)
        ys = None
        if shared is not None:
            ys = oracle.expert_ffn(*shared, qt, w.hidden, w.inter, np.zeros(len(tok_sample), np.int32),
                                   np.arange(len(tok_sample), dtype=np.int32), x, mode)
        return oracle.combine(y, wts, ys), bad

    # first pass: every (replay, layer) input once, checked against the GPU output
    items = [(r, l) for r in range(len(inputs)) for l in range(len(stack))]
    for r, l in items:
        if spent >= budget_s:
            break
        dl = stack[l]
        lg_t, x_t = inputs[r][l]
        qm.forward(dl.layer, lg_t, x_t, k, bufs, flags=flags)
        torch.cuda.synchronize()
        gpu_out = bufs.out.cpu().numpy()[tok_sample]
        lg = lg_t.cpu().numpy()[tok_sample]
        x = x_t.cpu().numpy()[tok_sample]
        # copy back only the experts this sample touches (not timed)
        idx_gpu = bufs.routing.idx.cpu().numpy()[tok_sample]
        uniq = np.unique(idx_gpu)
        sel = torch.as_tensor(uniq, device=dl.banks["gate"].device)
        hb = {n: dl.banks[n].index_select(0, sel).cpu().numpy() for n in ("gate", "up", "down")}
        remap = np.full(w.n_experts, -1, np.int64)
        remap[uniq] = np.arange(len(uniq))
        shared = tuple(dl.banks[n].cpu().numpy() for n in ("sh_gate", "sh_up", "sh_down")) if w.shared else None
        t0 = time.perf_counter()
        out, bad = run_oracle(lg, x, hb, remap, shared)
        spent += time.perf_counter() - t0
        tokens_done += len(tok_sample)
        layers_done += 1
        den = np.abs(out).max(axis=1)
        errs.append(float("inf") if bad else float((np.abs(gpu_out - out).max(axis=1) / den).max()))
        if len(cache) < kCache:
            cache.append((lg, x, hb, remap, shared))
        if layers_done % 20 == 0:
            log("[bench] cpu oracle: %d layer calls done, %.1f s spent" % (layers_done, spent))
    # then the cached items again until the budget is spent (no GPU work, no copies)
    i = 0
    while spent < budget_s and cache:
        t0 = time.perf_counter()
        run_oracle(*cache[i % len(cache)])
        spent += time.perf_counter() - t0
        tokens_done += len(tok_sample)
        layers_done += 1
        i += 1
        if layers_done % 500 == 0:
            log("[bench] cpu oracle: %d layer calls done, %.1f s spent" % (layers_done, spent))
    cpu = {"value": round(tokens_done / spent, 3), "unit": "layer-tokens/s", "cores": oracle.threads(),
           "kind": "oracle",
           "sample": "%d layer call(s) x %d token(s) of %s, route+bucket+FFN+combine in fp64 (%.1f s)"
                     % (layers_done, len(tok_sample), w.name, spent)}
    return cpu, (max(errs) if errs else None)


if __name__ == "__main__":
    sys.exit(main())
