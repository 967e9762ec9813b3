#!/usr/bin/env python3
"""Throughput of the routed MoE FFN over Q4_K / Q8_0 experts on one MI355X.

A step is one pass of the whole hot path (route -> [quantize] -> expert FFN ->
combine) through every layer of a stack of distinct seeded synthetic layers
resident in HBM, for one batch of fresh router logits and activations per
layer.

Default run (no --config): the prompt chunk (4,096 tokens, hidden 2048, 256
experts, top-8, intermediate 512, Q4_K, Zipf-loaded routing, int8 path) is the
line's workload, with its int8 TOPS against the MFMA peak (for the layer call,
and for the expert FFN call alone as gemm_tops) and the CPU oracle timed and
checked on one whole layer; the Sage-like decode layer (1 token, 40 layers) and
the Flash-Next-like decode layer (1 token, 10 routed + 1 shared, 48 layers) are
sub-records decode_c1 and decode_c3, each with its own HBM roofline, CPU oracle
baseline (all host threads and one thread) and parity.  The sub-record
prefill_chunk_pair_bf16 is the prompt chunk again with MOE_FFN_PAIR_BF16 (the
per-pair outputs handed to the combine as bf16 in the workspace), checked
against the oracle on one whole layer.  --config runs one workload alone
(--pair-bf16 sets the flag).

Prints ONE JSON line on stdout.  Progress goes to stderr.
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


METRIC = "MoE-layer tokens/s + achieved HBM GB/s (decode), int8 TOPS (prefill)"

# the default run: the prompt chunk as the line's workload, the two decode layers as sub-records
DEFAULT_MAIN = "prefill_chunk"
DEFAULT_SUBS = (("decode_c1", "sage_decode"), ("decode_c3", "flash_next_decode"))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def pair_bf16(w, flags, qm):
    """Workload w run with MOE_FFN_PAIR_BF16 (its records and traffic kept under its own name)."""
    from quantized_moe_ffn_amd.profiling import PAIR_BF16_SUFFIX
    return dataclasses.replace(w, name=w.name + PAIR_BF16_SUFFIX), flags | qm.MOE_FFN_PAIR_BF16


def resolve_workload(args, synth, qm, name):
    """The workload named `name` with the command line's overrides; None + message on error."""
    w = synth.WORKLOADS[name]
    if args.tokens is not None:
        if args.tokens < 1:
            return None, "--tokens must be at least 1"
        if args.tokens != w.tokens:
            w = dataclasses.replace(w, name="%s_t%d" % (w.name, args.tokens), tokens=args.tokens)
    if args.experts is not None or args.top_k is not None:
        E2 = args.experts if args.experts is not None else w.n_experts
        k2 = args.top_k if args.top_k is not None else w.top_k
        if not (1 <= k2 <= min(E2, 16)):
            return None, "need 1 <= top-k <= min(experts, 16)"
        w = dataclasses.replace(w, name="%s_e%d_k%d" % (w.name, E2, k2), n_experts=E2, top_k=k2)
    flags = qm.MOE_FFN_INT8 if w.int8_path else qm.MOE_FFN_DECODE
    if args.path is not None:
        flags = {"auto": qm.MOE_FFN_AUTO, "decode": qm.MOE_FFN_DECODE, "int8": qm.MOE_FFN_INT8}[args.path]
        int8 = flags == qm.MOE_FFN_INT8 or (flags == qm.MOE_FFN_AUTO and w.tokens > qm.AUTO_DECODE_MAX_T)
        if int8 != w.int8_path:
            # the roofline, the dtype and the oracle's quantisation points follow the path taken
            w = dataclasses.replace(w, name="%s_%s" % (w.name, "int8" if int8 else "decode"), int8_path=int8)
    return (w, flags), None


def run_workload(args, w, flags, torch, qm, dev, full_layer_oracle=False, single_thread=False) -> dict:
    """Builds the layer stack of workload w, times `steps` steps of it (graph replays) and
    returns its record: throughput, roofline of the layer call, CPU oracle baseline, parity."""
    from quantized_moe_ffn_amd import layers as qlayers
    L = args.layers or w.layers
    R = max(1, args.replays)
    T, H, E, k, I = w.tokens, w.hidden, w.n_experts, w.top_k, w.inter
    log("[bench] %s: building %d layers (%.2f GB of expert weights)"
        % (w.name, L, L * (E * w.expert_bytes() + (w.expert_bytes() if w.shared else 0)) / 1e9))
    t0 = time.time()
    stack = [qlayers.make_layer(w, seed=0, index=l, device=dev) for l in range(L)]
    torch.cuda.synchronize()
    log("[bench] %s: layers ready in %.1f s" % (w.name, time.time() - t0))

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
                # the layer from x and the router matrix: router kernel, then the layer
                qm.moe_forward_router(stack[l].layer, x, routers[l], lgbuf, k, bufs.routing, bufs.y_pair, bufs.out,
                                      bufs.fwd_ws, bufs.y_shared, flags=flags, stream=stream)
            else:
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
        log("[bench] %s: capturing %d graphs of %d layer calls" % (w.name, R, L))
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

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    qm.moe_check_device_errors()

    log("[bench] %s: timing %d steps x %d layers (graphs %s)" % (w.name, args.steps, L, args.graph))
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
    log("[bench] %s: %.3f ms/step, %.0f layer-tokens/s, %.2f us per layer call"
        % (w.name, ms_per_step, value, avg_us))

    # dominant call: the layer call (moe_forward), whose average duration is the
    # timed region divided by the number of calls in it
    if w.int8_path:
        ops = 2.0 * T * k * 3 * H * I + (2.0 * T * 3 * H * I if w.shared else 0.0)
        achieved = ops / (avg_us / 1e6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": INT8_PEAK_TOPS, "unit": "TFLOP/s",
                "frac": round(achieved / INT8_PEAK_TOPS, 4),
                "traffic": traffic_from_profiles(w.name) if routers is None else None,
                "kernel": ("moe_forward_router (router kernel, then " if routers is not None else "moe_forward (") +
                          "int8 path: route, quantize, gate/up, requantize, down, combine)",
                "ops_per_launch": ops, "avg_launch_us": round(avg_us, 3)}
        if routers is None and not flags & qm.MOE_FFN_PAIR_BF16:
            # (the separate FFN call has no bf16 hand-off: it times the unflagged GEMMs)
            roof.update(gemm_time(w, stack, inputs, bufs, flags, k, ops, args.steps, L, R, torch, qm))
    else:
        achieved = dom_bytes / (ms_total / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic_from_profiles(w.name) if routers is None else None,
                "kernel": ("moe_forward_router (router kernel, then " if routers is not None else "moe_forward (") +
                          "decode: route+gate/up+SiLU kernel, down+combine kernel)",
                "bytes_per_launch": round(dom_bytes / n_launch), "avg_launch_us": round(avg_us, 3)}
    log("[bench] %s: layer call %.2f us, %s %s" % (w.name, avg_us, roof["achieved"], roof["unit"]))

    cpu = None
    parity = None
    extra = {}
    if not args.no_cpu_baseline:
        # with --router the oracle takes the logits the GPU router produced
        # (untimed, above) as its input
        if full_layer_oracle:
            cpu, parity, extra = cpu_full_layer(w, stack, inputs, bufs, flags, k)
        else:
            cpu, parity = cpu_baseline(w, stack, inputs, bufs, flags, k, args.cpu_seconds)
            if single_thread:
                cpu["single_thread"] = cpu_single_thread(w, stack, inputs, bufs, flags, k, args.cpu_seconds / 4)
        cpu["cpu_model"] = cpu_model()

    rec = {
        "value": round(value, 1),
        "unit": "layer-tokens/s",
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "dtype": "i8" if w.int8_path else "f32",
        "config": {"workload": w.name, "tokens": T, "hidden": H, "experts": E, "top_k": k, "inter": I,
                   "shared_expert": w.shared, "layers": L, "replays": R,
                   "formats": {"gate": fmt(w.qt_gate), "up": fmt(w.qt_up), "down": fmt(w.qt_down)},
                   "parallelism": "single GPU", "graphs": args.graph,
                   "pair_outputs": ("workspace, bf16 on the MFMA GEMMs (MOE_FFN_PAIR_BF16)"
                                    if flags & qm.MOE_FFN_PAIR_BF16 else "fp32 y_pair"),
                   "router": "fp32 [E][H], moe_forward_router in the timed step" if routers is not None else None},
        "hbm_GBps_end_to_end": round(dom_bytes / (ms_total / 1e3) / 1e9, 1),
        "layer_call_us_p10_p50_p90": [pct[10], pct[50], pct[90]],
        "roofline": roof,
        "cpu_baseline": cpu,
        "parity_max_normwise_err": parity,
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
    }
    rec.update(extra)
    del graphs, stack, inputs, bufs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def gemm_time(w, stack, inputs, bufs, flags, k, ops, steps, L, R, torch, qm) -> dict:
    """The expert FFN call alone (moe_expert_ffn_q on the int8 path: the tile list, the code
    sums and the two grouped MFMA GEMMs), timed with events on its stream around each call of
    an eager pass of the separate calls over the same layers and inputs."""
    stream = torch.cuda.current_stream()
    times = []
    for s in range(steps):
        row = inputs[s % R]
        for l in range(L):
            lg, x = row[l]
            qm.moe_route_topk(lg, k, bufs.routing, True, bufs.route_ws, stream)
            qm.moe_quantize_act(x, bufs.xq, bufs.xd, stream)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            qm.moe_expert_ffn_q(stack[l].layer, bufs.routing, w.tokens, k, bufs.y_pair, xq=bufs.xq, xd=bufs.xd,
                                flags=flags & ~qm.MOE_FFN_PAIR_BF16, y_shared=bufs.y_shared,
                                workspace=bufs.ffn_ws, stream=stream)
            e1.record(stream)
            times.append((e0, e1))
    torch.cuda.synchronize()
    qm.moe_check_device_errors()
    us = float(np.mean([a.elapsed_time(b) * 1e3 for a, b in times]))
    tops = ops / (us / 1e6) / 1e12
    return {"gemm_tops": round(tops, 2), "gemm_frac": round(tops / INT8_PEAK_TOPS, 4),
            "gemm_call_us": round(us, 3),
            "gemm_kernel": "moe_expert_ffn_q (tile list, code sums, gate/up and down grouped int8 MFMA GEMMs)"}


def main() -> int:
    from quantized_moe_ffn_amd import synth
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default=None, choices=sorted(synth.WORKLOADS),
                    help="run one workload alone (default: the prompt chunk with the two decode layers as "
                         "sub-records)")
    ap.add_argument("--layers", type=int, default=None, help="override the number of distinct layers")
    ap.add_argument("--replays", type=int, default=8, help="distinct input sets cycled over the steps")
    ap.add_argument("--cpu-seconds", type=float, default=8.0, help="budget of each sampled CPU oracle run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", choices=["on", "off"], default="on", help="replay each step as a HIP graph")
    ap.add_argument("--router", action="store_true",
                    help="run each layer from x and a seeded fp32 [E][H] router matrix (moe_forward_router: the "
                         "router projection on the GPU inside the timed step)")
    ap.add_argument("--tokens", type=int, default=None,
                    help="override the tokens per layer call (a decode batch or verify window of the "
                         "same layer shape)")
    ap.add_argument("--experts", type=int, default=None,
                    help="override the routed experts per layer (e.g. one GPU's share under expert parallelism)")
    ap.add_argument("--top-k", type=int, default=None, help="override the routed experts per token")
    ap.add_argument("--path", choices=["auto", "decode", "int8"], default=None,
                    help="FFN path (default: the workload's own; auto takes the decode path up to 8 tokens)")
    ap.add_argument("--pair-bf16", action="store_true",
                    help="layer calls with MOE_FFN_PAIR_BF16: the per-pair outputs reach the combine through "
                         "the workspace, as bf16 on the int8 MFMA GEMMs")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: the MoE FFN path here is built and measured on a "
              "single MI355X (--gpus %d requested; multi-GPU sharding is a design note, not built)"
              % args.gpus, file=sys.stderr)
        return 2
    if args.config is None and (args.tokens is not None or args.experts is not None or args.top_k is not None
                                or args.path is not None or args.layers is not None or args.router
                                or args.pair_bf16):
        print("--tokens, --experts, --top-k, --path, --layers, --router and --pair-bf16 need --config",
              file=sys.stderr)
        return 2

    import torch
    import quantized_moe_ffn_amd as qm

    if not os.path.exists(qm.LIB_PATH):
        from quantized_moe_ffn_amd import build as hb
        hb.build()
    qm.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    main_name = args.config or DEFAULT_MAIN
    wf, err = resolve_workload(args, synth, qm, main_name)
    if err:
        print(err, file=sys.stderr)
        return 2
    w, flags = wf
    if args.pair_bf16:
        w, flags = pair_bf16(w, flags, qm)
    full = args.config is None
    rec_main = run_workload(args, w, flags, torch, qm, dev, full_layer_oracle=full and w.int8_path,
                            single_thread=not w.int8_path)
    rec = {
        "metric": METRIC,
        "value": rec_main.pop("value"),
        "unit": rec_main.pop("unit"),
        "n_gpus": 1,
        "steps": rec_main.pop("steps"),
        "warmup": rec_main.pop("warmup"),
        "ms_per_step": rec_main.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": rec_main.pop("dtype"),
        "data": "synthetic",
        "config": rec_main.pop("config"),
    }
    rec.update(rec_main)
    rec["hbm_copy_GBps_measured"] = copy_bandwidth(torch, dev)
    if full:
        for key, name in DEFAULT_SUBS:
            (ws, fs), _ = resolve_workload(args, synth, qm, name)
            sub = run_workload(args, ws, fs, torch, qm, dev, single_thread=True)
            rec[key] = sub
        # the same prompt chunk with the per-pair outputs handed to the combine as bf16
        wb, fb = pair_bf16(w, flags, qm)
        rec["prefill_chunk_pair_bf16"] = run_workload(args, wb, fb, torch, qm, dev, full_layer_oracle=True)
        if not args.no_cpu_baseline:
            rec["cpu_single_thread_tiny"] = cpu_tiny_single_thread(torch, qm, dev)
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


def cpu_full_layer(w, stack, inputs, bufs, flags, k):
    """The oracle on one whole layer call of the workload (every token and pair), timed on
    this host's cores, and the GPU's output of the same call checked against it.  On the
    int8 path a pair or token over the bound must match the oracle with some choice of the
    neighbouring h code at the positions where the code is a float-rounding decision
    (oracle.int8_pair_candidates); those rows are counted."""
    import torch
    import oracle
    import quantized_moe_ffn_amd as qm
    dl = stack[0]
    lg_t, x_t = inputs[0][0]
    if flags & qm.MOE_FFN_PAIR_BF16:
        # the flagged call returns no y_pair: the pairs are checked from the same call without
        # the flag (its fp32 y is what the bf16 hand-off rounds), out from the flagged call
        qm.forward(dl.layer, lg_t, x_t, k, bufs, flags=flags & ~qm.MOE_FFN_PAIR_BF16)
        torch.cuda.synchronize()
        gpu_y = bufs.y_pair.cpu().numpy()
    qm.forward(dl.layer, lg_t, x_t, k, bufs, flags=flags)
    torch.cuda.synchronize()
    qm.moe_check_device_errors()
    gpu_out = bufs.out.cpu().numpy()
    if not flags & qm.MOE_FFN_PAIR_BF16:
        gpu_y = bufs.y_pair.cpu().numpy()
    idx_gpu = bufs.routing.idx.cpu().numpy()
    lg = lg_t.cpu().numpy()
    x = x_t.cpu().numpy()
    T = x.shape[0]
    uniq = np.unique(idx_gpu)
    sel = torch.as_tensor(uniq, device=dl.banks["gate"].device)
    hb = {n: dl.banks[n].index_select(0, sel).cpu().numpy() for n in ("gate", "up", "down")}
    remap = np.full(w.n_experts, -1, np.int64)
    remap[uniq] = np.arange(len(uniq))
    qt = (w.qt_gate, w.qt_up, w.qt_down)
    mode = 1 if w.int8_path else 0
    log("[bench] %s: CPU oracle over the whole layer call (%d tokens, %d pairs, %d experts)"
        % (w.name, T, T * k, len(uniq)))
    t0 = time.perf_counter()
    idx, wts = oracle.route_topk(lg, k)
    oracle.bucket(idx, w.n_experts)
    pe = remap[idx.reshape(-1)]
    same_routing = bool(np.array_equal(idx, idx_gpu))
    pe = np.maximum(pe, 0)
    pt = np.repeat(np.arange(T), k)
    y = oracle.expert_ffn(hb["gate"], hb["up"], hb["down"], qt, w.hidden, w.inter, pe, pt, x, mode)
    out = oracle.combine(y, wts)
    spent = time.perf_counter() - t0
    tol = 5e-3 if w.int8_path else 2e-3

    def nerr(a, b):
        den = np.abs(b).max(axis=1)
        den[den == 0] = 1.0
        return np.abs(a - b).max(axis=1) / den
    ey, eo = nerr(gpu_y, y), nerr(gpu_out, out)
    raw = float(max(ey.max(), eo.max()))
    tie_rows = 0
    if not same_routing:
        parity = float("inf")
    elif raw <= tol or not w.int8_path:
        parity = raw
    else:
        mats, cand = {}, {}

        def pair(p):
            if p not in cand:
                e = int(pe[p])
                if e not in mats:
                    mats[e] = [oracle.dequant(hb[n][e], q).reshape(r, c) for n, q, r, c in
                               (("gate", qt[0], w.inter, w.hidden), ("up", qt[1], w.inter, w.hidden),
                                ("down", qt[2], w.hidden, w.inter))]
                cand[p] = oracle.int8_pair_candidates(*mats[e], x[p // k])
            return cand[p]
        worst = 0.0
        for p in np.nonzero(ey > tol)[0]:
            yc, d = pair(p)
            worst = max(worst, oracle.best_candidate_err(gpu_y[p], yc, d))
            tie_rows += 1
        for t in np.nonzero(eo > tol)[0]:
            ps = [t * k + j for j in range(k)]
            base = sum(wts[t, j] * pair(q)[0] for j, q in enumerate(ps))
            d = [wts[t, j] * dl_ for j, q in enumerate(ps) for dl_ in pair(q)[1]]
            worst = max(worst, oracle.best_candidate_err(gpu_out[t], base, d))
            tie_rows += 1
        ok_y = ey[ey <= tol].max() if np.any(ey <= tol) else 0.0
        ok_o = eo[eo <= tol].max() if np.any(eo <= tol) else 0.0
        parity = float(max(worst, ok_y, ok_o))
    cpu = {"value": round(T / spent, 3), "unit": "layer-tokens/s", "cores": oracle.threads(), "kind": "oracle",
           "sample": "1 whole layer call of %s (%d tokens, %d pairs): route+bucket+FFN+combine in fp64 (%.1f s)"
                     % (w.name, T, T * k, spent)}
    extra = {"parity_raw_max_normwise_err": raw, "parity_rows_decided_by_h_ties": tie_rows,
             "parity_scope": "every pair and token of one layer call"}
    return cpu, parity, extra


def cpu_single_thread(w, stack, inputs, bufs, flags, k, budget_s) -> dict:
    """The same sampled oracle run on one thread."""
    import oracle
    n0 = oracle.threads()
    oracle.set_threads(1)
    try:
        cpu, _ = cpu_baseline(w, stack, inputs, bufs, flags, k, budget_s)
    finally:
        oracle.set_threads(n0)
    return {"value": cpu["value"], "unit": cpu["unit"], "cores": 1, "sample": cpu["sample"]}


def cpu_tiny_single_thread(torch, qm, dev) -> dict:
    """The tiny layer (hidden 256, 8 experts, top-2, intermediate 256, 4 tokens) through the
    oracle on one thread, with its parity against the GPU's layer call."""
    import oracle
    from quantized_moe_ffn_amd import layers as qlayers, synth
    w = synth.WORKLOADS["tiny"]
    dl = qlayers.make_layer(w, seed=0, index=0, device=dev)
    logits, x = qlayers.inputs_np(w, seed=0)
    bufs = qm.forward(dl.layer, torch.from_numpy(logits).to(dev), torch.from_numpy(x).to(dev), w.top_k,
                      flags=qm.MOE_FFN_DECODE)
    torch.cuda.synchronize()
    got = bufs.out.cpu().numpy()
    banks = {n: t.cpu().numpy() for n, t in dl.banks.items()}
    n0 = oracle.threads()
    oracle.set_threads(1)
    try:
        calls, t0 = 0, time.perf_counter()
        while True:
            ref = oracle.moe_layer(logits, x, banks["gate"], banks["up"], banks["down"],
                                   (w.qt_gate, w.qt_up, w.qt_down), w.top_k)
            calls += 1
            spent = time.perf_counter() - t0
            if spent > 1.0:
                break
    finally:
        oracle.set_threads(n0)
    den = np.abs(ref["out"]).max(axis=1)
    err = float((np.abs(got - ref["out"]).max(axis=1) / den).max())
    return {"value": round(calls * w.tokens / spent, 2), "unit": "layer-tokens/s", "cores": 1, "kind": "oracle",
            "sample": "%d calls of the tiny layer (%d tokens), route+bucket+FFN+combine in fp64 (%.1f s)"
                      % (calls, w.tokens, spent),
            "parity_max_normwise_err": err}


if __name__ == "__main__":
    sys.exit(main())
