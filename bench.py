#!/usr/bin/env python3
"""Benchmark of the fused MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--mode mega|separate]

A step is one full layer forward (router, top-k, permutation, gate|up GEMM +
SwiGLU + FP8 requant, down GEMM, weighted combine) over one batch of
synthetic tokens whose inputs are already resident in HBM.  Prints one JSON
line: tokens/s, effective TFLOP/s, the roofline of the dominant kernel (the
persistent layer kernel in mega mode) and the oracle's throughput on a
bounded sample of the same workload timed on the host cores.
"""

import argparse
import dataclasses
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
PROFILES = os.path.join(ROOT, "profiles")


def source_digest() -> str:
    """sha256 over the HIP sources, the C header and the build flags: a
    traffic figure taken from hardware counters is valid only for the kernel
    built from exactly these."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "moe_layer_router_amd", "csrc")
    files = sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith((".h", ".hip")))
    files += [os.path.join(ROOT, "include", "moe_layer.h"), os.path.join(ROOT, "moe_layer_router_amd", "build.py")]
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    counter summary (FETCH_SIZE and WRITE_SIZE, calibrated against a copy of
    known size), or None when there is none or it was taken on other
    sources."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None
    d = json.loads(m.group(1))
    if d.get("source_sha256") != source_digest():
        return None
    return d.get("traffic_bytes")

# MI355X published peaks
PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"fp8": 5000.0, "fp4": 10100.0, "bf16": 2500.0}


def algorithmic_cost(cfg, inputs, counts):
    """Algorithmic FLOPs and HBM bytes of one layer forward.

    FLOPs: 6*T*k*H*I for the two expert GEMMs (2 flop per multiply-add,
    gate|up is 2I wide) plus 2*T*H*E for the router.  Bytes: weights and
    scales of every expert that receives a token (each read once), plus
    x, its scales, the router weights and bias, y, top-k ids and weights."""
    T, H, E, k, I = cfg.T, cfg.H, cfg.E, cfg.k, cfg.I
    f_exp = 6.0 * T * k * H * I
    f_router = 2.0 * T * H * E
    active = int((counts > 0).sum())

    def per_expert(name):
        t = inputs[name]
        return 0 if t is None else t[0].numel() * t.element_size()
    w_bytes = active * sum(per_expert(n) for n in ("w_gate_up", "w_gate_up_scales", "w_down", "w_down_scales"))
    io = 0
    for n in ("x", "x_scales", "router_w", "router_bias"):
        t = inputs[n]
        io += 0 if t is None else t.numel() * t.element_size()
    io += T * H * 2 + T * k * 4 * 2
    return f_exp, f_router, w_bytes + io, active


def roofline(cfg, f_exp, f_router, nbytes, t_s):
    exp_fmt = cfg.weight if cfg.weight == "bf16" else "fp8"     # FP8 x FP4 issues at the FP8 rate
    t_mfma = f_exp / (PEAK_TFLOPS[exp_fmt] * 1e12) + f_router / (PEAK_TFLOPS["bf16"] * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    if t_hbm >= t_mfma:
        ach = nbytes / t_s / 1e9
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4)}, t_mfma, t_hbm
    ach = (f_exp + f_router) / t_s / 1e12
    peak = PEAK_TFLOPS[exp_fmt]
    return {"bound": "mfma", "achieved": round(ach, 1), "peak": peak, "unit": "TFLOP/s",
            "frac": round(ach / peak, 4)}, t_mfma, t_hbm


def measure_peaks(dev, cus: int):
    """Measured matrix-core rates (per operand format) and HBM read bandwidth
    on this device, with the library's microbenchmarks (moe_peaks.h): one
    workgroup per SIMD quad on every CU, 8 independent MFMA chains per wave;
    a 4 GiB read with 16-byte loads."""
    import torch
    from moe_layer_router_amd import lib
    out = {}
    blocks = cus * 2
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    cyc = torch.empty(blocks * 4, dtype=torch.int64, device=dev)
    for kind in lib.MOE_PEAK_KINDS:
        iters = 2000 if "32" not in kind else 1000
        lib.moe_peak_mfma(kind, 50, blocks, sink, cyc)              # warm-up
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        lib.moe_peak_mfma(kind, iters, blocks, sink, cyc)
        b.record()
        torch.cuda.synchronize()
        t = a.elapsed_time(b) / 1e3
        per_instr = float(np.median(cyc.cpu().numpy())) / (iters * 8)
        out[kind] = {"tflops": round(lib.moe_peak_mfma_flops(kind, iters, blocks) / t / 1e12, 1),
                     "cycles_per_instr_per_wave": round(per_instr, 2)}
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(3)
    rsink = torch.empty(cus * 8 * 256, dtype=torch.int32, device=dev)
    lib.moe_peak_hbm_read(buf, nbytes, cus * 8, rsink)
    torch.cuda.synchronize()
    ts = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        lib.moe_peak_hbm_read(buf, nbytes, cus * 8, rsink)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) / 1e3)
    out["hbm_read_gbs"] = round(nbytes / min(ts) / 1e9, 1)
    del buf
    return out


def cpu_baseline(cfg, inputs, n_experts=4):
    """The oracle as it stands, on a bounded sample of the same workload:
    routing and the permutation for all T tokens, then the complete expert
    work (decode, gate|up, SwiGLU, requant, down, combine) of `n_experts`
    experts.  The full-layer time is extrapolated as
    t_route + E * (mean time per expert)."""
    from threadpoolctl import threadpool_info
    from oracle import moe_oracle as O
    from workloads import gen

    spec = gen.spec_of(cfg)
    ov = gen.oracle_view(inputs, lazy_weights=True)
    t0 = time.perf_counter()
    xhat, logits, ids, w = O.route(spec, ov)
    counts, offsets, perm, row_of = O.permutation(ids, cfg.E)
    t_route = time.perf_counter() - t0
    busy = np.argsort(-counts, kind="stable")
    sample = [int(e) for e in busy[np.linspace(0, min(cfg.E, int((counts > 0).sum())) - 1, n_experts).astype(int)]]
    y = np.zeros((cfg.T, cfg.H))
    t1 = time.perf_counter()
    for e in sample:
        rows = perm[offsets[e]: offsets[e + 1]]
        toks = rows // cfg.k
        s1 = None if ov["w_gate_up_scales"] is None else ov["w_gate_up_scales"][e]
        s2 = None if ov["w_down_scales"] is None else ov["w_down_scales"][e]
        wgu = O.decode_weight(spec, ov["w_gate_up"][e], s1)
        wd = O.decode_weight(spec, ov["w_down"][e], s2)
        y[toks] += w.reshape(-1)[rows][:, None] * O.expert_ffn(spec, xhat[toks], wgu, wd)
    t_exp = (time.perf_counter() - t1) / len(sample)
    active = int((counts > 0).sum())
    t_full = t_route + active * t_exp
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": round(cfg.T / t_full, 3), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"fp64 numpy oracle: routing + permutation of all {cfg.T} tokens ({t_route:.2f} s) and the "
                       f"full expert work of {len(sample)} of {active} active experts ({t_exp:.2f} s each, "
                       f"experts {sample}); layer time extrapolated as t_route + {active} * t_expert = {t_full:.1f} s"),
            "host_cpus": len(os.sched_getaffinity(0))}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3_fp8")
    ap.add_argument("--mode", default="mega", choices=["mega", "separate"])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-experts", type=int, default=64, choices=range(1, 1 << 16), metavar="N")
    ap.add_argument("--no-ablation", action="store_true", help="skip timing the other mode")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one device copy of 1 GiB (a counter calibration point for profiling runs)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the peak-rate microbenchmarks")
    ap.add_argument("--trace", action="store_true",
                    help="one extra persistent-kernel call with per-workgroup phase stamps (reported as 'phases')")
    ap.add_argument("--inter-scale", default="f32", choices=["f32", "pow2"],
                    help="scale rule of the layer's own FP8 quantisations (moe_desc.inter_scale)")
    ap.add_argument("--no-evict", action="store_true", help="skip the cache-evicted per-call timing")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (moe_backward) of a BF16 layer instead (default workload dsv3_bf16)")
    ap.add_argument("--e5m6", action="store_true",
                    help="time the E5M6 quantisation and dequantisation of the workload's activations instead")
    ap.add_argument("--wscale", default=None, choices=["block", "channel"],
                    help="FP8 weight scale granularity (moe_desc.weight_scale; default: the workload's)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested): the layer is measured on a "
              "single MI355X; expert parallelism across GPUs is not part of this build.", file=sys.stderr)
        sys.exit(2)

    import torch
    from moe_layer_router_amd import layer
    from workloads import gen

    if args.backward:
        bench_backward(args)
        return
    if args.e5m6:
        bench_e5m6(args)
        return
    cfg = gen.CONFIGS[args.workload]
    if args.wscale is not None:
        if cfg.weight != "fp8" and args.wscale == "channel":
            print("--wscale channel needs FP8 weights", file=sys.stderr)
            sys.exit(2)
        cfg = dataclasses.replace(cfg, wscale=args.wscale)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating {cfg.name} inputs on {dev}", file=sys.stderr, flush=True)
    raw = gen.make_inputs(cfg, seed=args.seed, device=dev)
    # weights go into the MFMA-tiled layout once, as at model load time
    inputs = layer.pack_weights(raw)
    torch.cuda.synchronize()
    if args.calib_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    ws = layer.Workspace(dev)
    stream = torch.cuda.current_stream()

    def timed(mode):
        """Warm-up, then K back-to-back layer calls on the current stream,
        timed as a whole and per call (one event pair per call: the counter
        clearing kernel (a few microseconds) and the layer's kernels)."""
        out = layer.forward(inputs, cfg.k, mode=mode, workspace=ws, inter_scale=args.inter_scale)
        torch.cuda.synchronize()
        if int(out["workspace"][:4].view(torch.int32).item()) != 0:
            raise RuntimeError("device watchdog fired")
        print(f"[bench] {mode}: warmup {args.warmup}", file=sys.stderr, flush=True)
        for _ in range(args.warmup):
            layer.forward(inputs, cfg.k, mode=mode, workspace=ws, out=out, inter_scale=args.inter_scale)
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        t_begin = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_begin.record(stream)
        for i in range(args.steps):
            starts[i].record(stream)
            layer.forward(inputs, cfg.k, mode=mode, workspace=ws, out=out, inter_scale=args.inter_scale)
            ends[i].record(stream)
        t_end.record(stream)
        torch.cuda.synchronize()
        print(f"[bench] {mode}: timed {args.steps} steps", file=sys.stderr, flush=True)
        if not torch.isfinite(out["y"].float()).all():
            raise RuntimeError("non-finite output")
        per = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
        return out, t_begin.elapsed_time(t_end) / args.steps, per

    out, ms, per = timed(args.mode)
    counts = np.diff(out["expert_offsets"].cpu().numpy())
    evicted = None
    if not args.no_evict:
        # per-call times with the 256 MB last-level cache overwritten before
        # each call (a 1 GiB write between calls, outside the timed calls)
        junk = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        ev = []
        for _ in range(max(5, min(args.steps, 20))):
            junk.fill_(7)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            layer.forward(inputs, cfg.k, mode=args.mode, workspace=ws, out=out, inter_scale=args.inter_scale)
            b.record(stream)
            torch.cuda.synchronize()
            ev.append(a.elapsed_time(b))
        del junk
        ev = np.array(ev)
        evicted = {"median_ms": round(float(np.median(ev)), 4), "min_ms": round(float(ev.min()), 4),
                   "mean_ms": round(float(ev.mean()), 4), "calls": int(ev.size)}
        print(f"[bench] {args.mode}: cache-evicted per-call median {np.median(ev):.4f} ms", file=sys.stderr, flush=True)
    other = "separate" if args.mode == "mega" else "mega"
    ablation = None
    if not args.no_ablation:
        _, ms_other, _ = timed(other)
        ablation = {"mode": other, "ms_per_step": round(ms_other, 4), "tokens_per_s": round(cfg.T / (ms_other / 1e3), 1)}

    f_exp, f_router, nbytes, active = algorithmic_cost(cfg, inputs, counts)
    t_launch = float(per.mean()) / 1e3
    roof, t_mfma, t_hbm = roofline(cfg, f_exp, f_router, nbytes, t_launch)
    kernel = "k_mega" if args.mode == "mega" else "layer_separate"
    roof["kernel"] = kernel
    # what the timed interval holds (the per-call HIP event pair)
    roof["covers"] = ("one moe_forward call: the counter clear, the routing and permutation kernels (from 2048 "
                      "tokens on; below that they run inside k_mega) and k_mega" if args.mode == "mega" else
                      "one moe_forward call: every kernel of the separate pipeline")
    # (the committed counter summaries are of the workloads' own weight scales)
    roof["traffic"] = measured_traffic(kernel, cfg.name) if cfg == gen.CONFIGS[cfg.name] else None
    tflops = (f_exp + f_router) / (ms / 1e3) / 1e12
    exp_fmt = cfg.weight if cfg.weight == "bf16" else "fp8"
    result = {
        "metric": "MoE-layer tokens/s & TFLOP/s (% MFMA peak), T=8192 H=7168 E=256 top-8 FP8",
        "value": round(cfg.T / (ms / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp8": "fp8 e4m3 x fp8 e4m3", "fp4": "fp8 e4m3 x fp4 e2m1", "bf16": "bf16"}[cfg.weight],
        "data": "synthetic (seeded N(0,1) activations, N(0,1/fan_in) weights, quantised; no real weights)",
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "E": cfg.E, "top_k": cfg.k, "I": cfg.I,
                   "act": cfg.act, "weight": cfg.weight, "zipf": cfg.zipf, "mode": args.mode,
                   "inter_scale": args.inter_scale, "weight_scale": cfg.wscale,
                   "active_experts": active},
        "tflops": round(tflops, 1),
        "mfma_peak_frac": round(tflops / PEAK_TFLOPS[exp_fmt], 4),
        "hbm_gbs": round(nbytes / (ms / 1e3) / 1e9, 1),
        "roofline": roof,
        "roofline_model": {"algorithmic_tflop": round((f_exp + f_router) / 1e12, 4),
                           "algorithmic_gb": round(nbytes / 1e9, 4),
                           "t_mfma_ms": round(t_mfma * 1e3, 4), "t_hbm_ms": round(t_hbm * 1e3, 4),
                           "kernel_ms": round(t_launch * 1e3, 4),
                           "roofline_frac": round(max(t_mfma, t_hbm) / t_launch, 4)},
        "ablation": ablation,
        "per_call_ms": {"median": round(float(np.median(per)), 4), "min": round(float(per.min()), 4),
                        "mean": round(float(per.mean()), 4)},
        "per_call_cache_evicted_ms": evicted,
    }
    if args.trace:
        # two traced calls on a fresh workspace: the first touches its pages,
        # the second (reported) runs as the timed calls do
        tws = layer.Workspace(dev)
        tout = layer.forward(inputs, cfg.k, mode="mega", workspace=tws, inter_scale=args.inter_scale, trace=True)
        tout = layer.forward(inputs, cfg.k, mode="mega", workspace=tws, inter_scale=args.inter_scale, trace=True,
                             out=tout)
        torch.cuda.synchronize()
        result["phases"] = layer.trace_phases(tout)
        print(f"[bench] phases: {json.dumps(result['phases'])}", file=sys.stderr, flush=True)
        del tws, tout
    if not args.no_peaks:
        print("[bench] peak-rate microbenchmarks", file=sys.stderr, flush=True)
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        pk = measure_peaks(dev, cus)
        result["measured_peaks"] = pk
        kind = {"fp8": "mfma16_fp8_fp8", "fp4": "mfma16_fp4_fp8", "bf16": "mfma16_bf16"}[cfg.weight]
        result["roofline_model"]["measured_peak_tflops"] = pk[kind]["tflops"]
        result["roofline_model"]["measured_hbm_gbs"] = pk["hbm_read_gbs"]
        t_m = f_exp / (pk[kind]["tflops"] * 1e12) + f_router / (pk["mfma16_bf16"]["tflops"] * 1e12)
        t_h = nbytes / (pk["hbm_read_gbs"] * 1e9)
        result["roofline_model"]["roofline_frac_measured_peaks"] = round(max(t_m, t_h) / t_launch, 4)
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on a bounded sample (host cores)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(cfg, raw, args.cpu_experts)
    print(json.dumps(result), flush=True)


def backward_cost(cfg, active: int):
    """Algorithmic FLOPs and HBM bytes of one backward pass: the gate|up
    recompute, the unweighted intermediate gradient, the linear-1 input
    gradient and the two weight gradients (16*T*k*H*I), the router's two
    products (4*T*E*H); bytes: x, dy and the active experts' weights read,
    dx and every gradient written in fp32."""
    T, H, E, k, I = cfg.T, cfg.H, cfg.E, cfg.k, cfg.I
    flops = 16.0 * T * k * H * I + 4.0 * T * E * H
    nbytes = 2 * T * H * 2 + active * 3 * I * H * 2 + E * H * 2
    nbytes += T * H * 4 + E * 3 * I * H * 4 + E * H * 4 + E * 4
    return flops, nbytes


def cpu_baseline_backward(cfg, raw, ids, dy, n_tokens=12, n_experts=4):
    """The oracle's backward pass (backward_exact, fp64) on a bounded sample:
    `n_tokens` tokens, each routed to all of the `n_experts` busiest experts
    of the real routing (the oracle's cost per (token, expert) pair does not
    depend on which pair it is), with those experts' weights.  The layer time
    is extrapolated as T*k pairs x the time per pair (the router's products,
    E*H per token, are under 3% of a pair's work and are not scaled up)."""
    import torch
    from threadpoolctl import threadpool_info
    from oracle import moe_oracle as O
    from oracle import formats as F
    T, k = ids.shape
    busy = np.argsort(-np.bincount(ids.ravel(), minlength=cfg.E), kind="stable")[:n_experts]
    bf = lambda x: F.bf16_decode(x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16))
    idx = torch.as_tensor(busy)
    xh = bf(raw["x"][:n_tokens])
    wr = bf(raw["router_w"][idx.to(raw["router_w"].device)])
    w_gu = bf(raw["w_gate_up"][idx.to(raw["w_gate_up"].device)])
    w_d = bf(raw["w_down"][idx.to(raw["w_down"].device)])
    dys = bf(dy[:n_tokens])
    ids_s = np.tile(np.arange(n_experts, dtype=np.int64), (n_tokens, 1))
    t0 = time.perf_counter()
    O.backward_exact(xh, xh, wr, np.zeros(n_experts), w_gu, w_d, ids_s, dys, cfg.I)
    dt = time.perf_counter() - t0
    per_pair = dt / (n_tokens * n_experts)
    t_layer = per_pair * T * k
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": round(T / t_layer, 3), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"fp64 numpy oracle backward_exact on {n_tokens} tokens x the {n_experts} busiest experts "
                       f"({dt:.2f} s, {per_pair * 1e3:.1f} ms per token-expert pair); layer time extrapolated as "
                       f"{T}*{k} pairs = {t_layer:.1f} s"),
            "host_cpus": len(os.sched_getaffinity(0))}


def bench_backward(args):
    import torch
    from moe_layer_router_amd import layer
    from workloads import gen
    name = args.workload if args.workload != "dsv3_fp8" else "dsv3_bf16"
    cfg = gen.CONFIGS[name]
    if cfg.act != "bf16" or cfg.weight != "bf16":
        print("--backward needs a BF16 layer workload", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] backward: generating {cfg.name} inputs on {dev}", file=sys.stderr, flush=True)
    raw = gen.make_inputs(cfg, seed=args.seed, device=dev)
    fwd = layer.forward(layer.pack_weights(raw), cfg.k, mode="mega")
    ids, wts = fwd["topk_ids"].clone(), fwd["topk_weights"].clone()
    del fwd
    g = torch.Generator(device="cpu").manual_seed(args.seed + 1)
    dy = torch.randn(cfg.T, cfg.H, generator=g).to(torch.bfloat16).to(dev)
    ws = layer.Workspace(dev)
    stream = torch.cuda.current_stream()
    out = layer.backward(raw, ids, wts, dy, workspace=ws)
    torch.cuda.synchronize()
    print(f"[bench] backward: warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        layer.backward(raw, ids, wts, dy, workspace=ws, out=out)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t_begin, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_begin.record(stream)
    for i in range(args.steps):
        starts[i].record(stream)
        layer.backward(raw, ids, wts, dy, workspace=ws, out=out)
        ends[i].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    print(f"[bench] backward: timed {args.steps} steps", file=sys.stderr, flush=True)
    for key, v in out.items():
        if v is not None and not torch.isfinite(v).all():
            raise RuntimeError(f"non-finite {key}")
    ms = t_begin.elapsed_time(t_end) / args.steps
    per = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
    active = int((torch.bincount(ids.view(-1).long(), minlength=cfg.E) > 0).sum().item())
    flops, nbytes = backward_cost(cfg, active)
    t_call = float(per.mean()) / 1e3
    t_mfma = flops / (PEAK_TFLOPS["bf16"] * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    if t_hbm >= t_mfma:
        roof = {"bound": "hbm", "achieved": round(nbytes / t_call / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(nbytes / t_call / 1e9 / PEAK_HBM_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(flops / t_call / 1e12, 1), "peak": PEAK_TFLOPS["bf16"],
                "unit": "TFLOP/s", "frac": round(flops / t_call / 1e12 / PEAK_TFLOPS["bf16"], 4)}
    roof["kernel"] = "moe_backward (10 kernels)"
    roof["traffic"] = None
    result = {
        "metric": "MoE-layer backward tokens/s (BF16 layer, routing given)",
        "value": round(cfg.T / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 operands, fp32 sums and gradients",
        "data": "synthetic (seeded N(0,1) activations and output gradients, N(0,1/fan_in) weights)",
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "E": cfg.E, "top_k": cfg.k, "I": cfg.I,
                   "active_experts": active},
        "tflops": round(flops / (ms / 1e3) / 1e12, 1),
        "roofline": roof,
        "roofline_model": {"algorithmic_tflop": round(flops / 1e12, 4), "algorithmic_gb": round(nbytes / 1e9, 4),
                           "t_mfma_ms": round(t_mfma * 1e3, 4), "t_hbm_ms": round(t_hbm * 1e3, 4),
                           "kernel_ms": round(t_call * 1e3, 4)},
        "per_call_ms": {"median": round(float(np.median(per)), 4), "min": round(float(per.min()), 4),
                        "mean": round(float(per.mean()), 4)},
    }
    if not args.no_cpu_baseline:
        print("[bench] backward: timing the oracle on a bounded sample (host cores)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline_backward(cfg, raw, ids.cpu().numpy().astype(np.int64), dy)
    print(json.dumps(result), flush=True)


def bench_e5m6(args):
    """E5M6 conversion of the workload's activations x [T][H] (BF16): the
    quantisation (2 bytes read, 1.5 written per element, plus a 4-byte scale
    per 128) and the dequantisation to fp32 (1.5 + 4/128 read, 4 written),
    each HBM-bound; timed with HIP events over `steps` launches each."""
    import torch
    from moe_layer_router_amd import layer
    from workloads import gen
    cfg = gen.CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = torch.Generator(device="cpu").manual_seed(args.seed)
    x = torch.randn(cfg.T, cfg.H, generator=g).to(torch.bfloat16).to(dev)
    stream = torch.cuda.current_stream()
    xq, xs = layer.quantize_e5m6(x)
    out = layer.dequantize_e5m6(xq, xs)
    torch.cuda.synchronize()
    n = cfg.T * cfg.H

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(args.steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps / 1e3

    from moe_layer_router_amd import lib
    t_q = timed(lambda: lib.moe_quantize_e5m6(x, xq, xs, "f32"))
    t_d = timed(lambda: lib.moe_dequantize_e5m6(xq, xs, out))
    bq = n * 2 + n * 1.5 + n / 128 * 4
    bd = n * 1.5 + n / 128 * 4 + n * 4
    roof = {"bound": "hbm", "achieved": round(bq / t_q / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(bq / t_q / 1e9 / PEAK_HBM_GBS, 4), "kernel": "k_quant_e5m6", "traffic": None}
    result = {
        "metric": "E5M6 per-token quantisation tokens/s (BF16 activations)", "value": round(cfg.T / t_q, 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(t_q * 1e3, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 in, 12-bit E5M6 codes + fp32 scales out", "data": "synthetic (seeded N(0,1) activations)",
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H},
        "roofline": roof,
        "dequantise": {"ms": round(t_d * 1e3, 5), "achieved_GBs": round(bd / t_d / 1e9, 1),
                       "frac": round(bd / t_d / 1e9 / PEAK_HBM_GBS, 4)},
    }
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_info
        from oracle import moe_oracle as O
        rows = min(cfg.T, 512)
        xv = x[:rows].float().cpu().double().numpy()
        t0 = time.perf_counter()
        O.quantise_tokens_e5m6(xv)
        dt = time.perf_counter() - t0
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        result["cpu_baseline"] = {"value": round(rows / dt, 1), "unit": "tokens/s", "cores": int(threads),
                                  "kind": "oracle", "sample": f"fp64 numpy oracle quantise_tokens_e5m6 on the first "
                                                              f"{rows} tokens ({dt:.2f} s)"}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
