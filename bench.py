#!/usr/bin/env python3
"""Throughput of the int4-g64 grouped MoE layer on one MI355X.

Headline: MoE-layer prefill tokens/s at T=4096 (d=2048, f=512, E=256, top-8
+ 1 shared, Zipf(1.1)-skewed expert load), one moe_layer_forward call per
step, inputs resident in HBM. Also reported on the same JSON line:
  roofline      the gate/up grouped GEMM (the dominant kernel): algorithmic
                FLOP per launch / its mean duration (HIP events on the stream
                the kernel runs on), against the 2516.6 TFLOP/s bf16 dense peak;
  kernels       every kernel's mean duration and rate;
  decode        batch-1 decode: 1000 steps through the T=1 path, 32 weight
                copies rotated so no step re-reads weights from cache, replayed
                as a HIP graph; algorithmic bytes / time per step; and the
                first 256 steps from hidden states (router projection first);
  configs       the other workloads: T=16 (median latency), T=512 (two
                weight copies alternated; GB/s of the used experts' weights and
                I/O against 8 TB/s), T=16384 with 8 forced-empty experts
                (TFLOP/s against the bf16 peak, per-kernel times);
  mixed_bias    the headline layer with mixed dequantisation biases;
  cpu_baseline  the CPU oracle on the whole headline layer (and, under
                configs, on the whole layer of each other workload);
  small_batch   the layer at T = 1, 2, 8, 32, 64 (skipped with
                --no-small-batch), bytes of the used experts' weights / time,
                timed in 32-call HIP graphs (us) and call by call (us_eager).
Usage: python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA: 256 CUs x 2.4 GHz x 4096 FLOP/clock
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
W4_BYTES_PER_EXPERT = None    # filled from the shapes


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def expert_bytes(d, f):
    # 3 matrices of d*f weights: 4-bit codes + one bf16 scale and bias per 64 weights
    return 3 * d * f // 2 + 3 * d * f // 64 * 4


# sources the grouped GEMM kernels are compiled from, and the one that builds the
# tile schedule they follow (which XCD reads which expert's weights)
GEMM_SOURCES = [os.path.join("bit_quantized_grouped_router_amd", "csrc", n)
                for n in ("moe_ffn.hip", "moe_device.h", "moe_launch.h", "moe_permute.hip")]


def sources_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profile(sources, launches_key):
    """HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE counters (scaled by a
    plain copy of known size), if they were taken on these kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p)).get(launches_key)
        if rec and rec.get("source_sha") == sources_hash(sources):
            return rec["bytes_per_launch"]
    except Exception:
        return None
    return None


def event_us(fn, n, stream, warm=3):
    """Per-call durations (us) of fn() with HIP events on `stream`, all calls enqueued
    before one synchronisation."""
    import torch
    for _ in range(warm):
        fn()
    evs = []
    for _ in range(n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        evs.append((a, b))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e3 for a, b in evs]


def median(v):
    v = sorted(v)
    return v[len(v) // 2] if len(v) % 2 else 0.5 * (v[len(v) // 2 - 1] + v[len(v) // 2])


def kernel_times(M, dm, x, logits, w, n_iter, stream):
    """Mean duration (us) of each kernel of the layer, HIP events around each call on
    `stream` (all iterations enqueued before one synchronisation)."""
    import torch
    k = dm.k
    ids, wts = M.moe_route(logits, k, stream=stream)
    perm = M.moe_permute(dm, ids, stream=stream)
    h, o_r, o_sh = M.moe_expert_ffn_w4(dm, x, w, perm["sorted_token"], perm["tile_map"],
                                       perm["num_tiles"], stream=stream)
    yk = M.moe_unpermute_combine(dm, o_r, o_sh, wts, perm["row_of"], stream=stream)
    torch.cuda.synchronize()
    names = ["route", "permute", "gate_up", "down", "combine"]
    acc = {n: 0.0 for n in names}
    evs = []
    for it in range(n_iter + 2):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        ev[0].record(stream)
        M.moe_route(logits, k, ids, wts, stream=stream)
        ev[1].record(stream)
        M.moe_permute(dm, ids, out=perm, stream=stream)
        ev[2].record(stream)
        M.moe_expert_gate_up_w4(dm, x, w, perm["sorted_token"], perm["tile_map"],
                                perm["num_tiles"], h=h, stream=stream)
        ev[3].record(stream)
        M.moe_expert_down_w4(dm, h, w, perm["tile_map"], perm["num_tiles"], o_routed=o_r,
                             o_shared=o_sh, stream=stream)
        ev[4].record(stream)
        M.moe_unpermute_combine(dm, o_r, o_sh, wts, perm["row_of"], y=yk, stream=stream)
        ev[5].record(stream)
        if it >= 2:
            evs.append(ev)
    torch.cuda.synchronize()
    for ev in evs:
        for i, n in enumerate(names):
            acc[n] += ev[i].elapsed_time(ev[i + 1]) * 1e3 / len(evs)
    nonempty = int((perm["counts"] > 0).sum().item())
    return acc, nonempty


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (T=16, T=512, T=16384) and the mixed-bias row")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-headline-only", action="store_true",
                    help="time the CPU oracle on the headline layer only")
    ap.add_argument("--small-batch", action="store_true",
                    help="time moe_layer_forward at T = 1, 2, 8, 32, 64 (the default; kept "
                         "for older command lines)")
    ap.add_argument("--no-small-batch", action="store_true",
                    help="skip the small-batch timings")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 256 MiB device-to-device copy (a reference "
                         "kernel of known traffic for hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported (the "
              "layer has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bit_quantized_grouped_router_amd as M
    import moe_inputs as G

    if not os.path.exists(M.LIB_PATH):
        from bit_quantized_grouped_router_amd import build
        build.build()
    M.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()

    if args.calibrate_copy:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy: {src.numel() * 4} bytes read and written")
        del src, dst

    def upload(cfg, weights=None):
        a = G.make_activations(cfg)
        x = torch.from_numpy(a["x"].view(np.int16)).to(dev)
        lg = torch.from_numpy(a["logits"]).to(dev)
        wt = weights if weights is not None else G.make_weights(cfg)
        return a, x, lg, wt, M.W4Weights.from_numpy(wt, device=dev)

    def flops(T, d, f, k):
        rows = T * (k + 1)
        return 2.0 * rows * d * 2 * f, 2.0 * rows * f * d

    cfg = G.CONFIGS["prefill_t4096_zipf"]
    T, d, f, E, k = cfg.T, cfg.d, cfg.f, cfg.E, cfg.k
    log(f"[bench] generating {cfg.name}")
    act, x, logits, weights_np, w = upload(cfg)
    inp = {"x": act["x"], "logits": act["logits"], "weights": weights_np}
    wc = w.c()
    dm = M.dims(T, d, f, E, k)
    ws = torch.empty(M.moe_layer_workspace_bytes(dm), dtype=torch.uint8, device=dev)
    y = torch.empty((T, d), dtype=torch.float32, device=dev)
    flop_gate_up, flop_down = flops(T, d, f, k)
    flop_layer = flop_gate_up + flop_down

    # ---------------------------------------------------------------- headline: whole layer
    log(f"[bench] layer T={T}: warmup {args.warmup}, timed {args.steps}")
    for _ in range(args.warmup):
        M.moe_layer_forward(dm, x, logits, w, y=y, ws=ws, wc=wc)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        M.moe_layer_forward(dm, x, logits, w, y=y, ws=ws, wc=wc)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    tok_s = T / (ms_per_step / 1e3)
    log(f"[bench] layer: {ms_per_step:.3f} ms/step, {tok_s:,.0f} tok/s")

    # ---------------------------------------------------------------- per-kernel timing
    log("[bench] per-kernel timing with HIP events")
    acc, nonempty = kernel_times(M, dm, x, logits, w, max(args.steps, 5), stream)
    bytes_layer = ((nonempty + 1) * expert_bytes(d, f) + x.numel() * 2 + logits.numel() * 4
                   + y.numel() * 4)
    kernels = {n: {"us": round(v, 2)} for n, v in acc.items()}
    kernels["gate_up"]["TFLOP/s"] = round(flop_gate_up / (acc["gate_up"] * 1e-6) / 1e12, 1)
    kernels["gate_up"]["frac_bf16_peak"] = round(kernels["gate_up"]["TFLOP/s"] / PEAK_BF16_TFLOPS, 4)
    kernels["down"]["TFLOP/s"] = round(flop_down / (acc["down"] * 1e-6) / 1e12, 1)
    kernels["down"]["frac_bf16_peak"] = round(kernels["down"]["TFLOP/s"] / PEAK_BF16_TFLOPS, 4)
    comb_bytes = T * k * d * 2 + T * d * 4 * 2 + T * k * 8
    kernels["combine"]["GB/s"] = round(comb_bytes / (acc["combine"] * 1e-6) / 1e9, 1)
    # router projection (the step before routing when the layer starts from
    # hidden states); timed on its own, the headline step starts from logits
    wr = torch.from_numpy(G.make_router(cfg).view(np.int16)).to(dev)
    lg = torch.empty((T, E), dtype=torch.float32, device=dev)
    us = sum(event_us(lambda: M.moe_router_logits(x, wr, logits=lg, stream=stream),
                      max(args.steps, 5), stream)) / max(args.steps, 5)
    rflop = 2.0 * T * d * E
    kernels["router_logits"] = {"us": round(us, 2),
                                "TFLOP/s": round(rflop / (us * 1e-6) / 1e12, 1),
                                "frac_bf16_peak": round(rflop / (us * 1e-6) / 1e12
                                                        / PEAK_BF16_TFLOPS, 4),
                                "GB/s": round((T * d * 2 + E * d * 2 + T * E * 4) / (us * 1e-6)
                                              / 1e9, 1)}
    log(f"[bench] kernels: {kernels}")
    achieved = flop_gate_up / (acc["gate_up"] * 1e-6) / 1e12
    roofline = {"kernel": "gate_up_kernel", "bound": "mfma", "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic_from_profile(GEMM_SOURCES, "gate_up_prefill_t4096_zipf"),
                "algorithmic_flop_per_launch": flop_gate_up}

    # ---------------------------------------------------------------- the other workloads
    configs = None
    mixed = None
    big = None
    if not args.no_configs:
        configs = {}
        # tiny layer: per-call latency
        c0 = G.CONFIGS["tiny_t16"]
        a0, x0, l0, w0np, w0 = upload(c0)
        dm0 = M.dims(c0.T, c0.d, c0.f, c0.E, c0.k)
        ws0 = torch.empty(M.moe_layer_workspace_bytes(dm0), dtype=torch.uint8, device=dev)
        y0 = torch.empty((c0.T, c0.d), dtype=torch.float32, device=dev)
        t = event_us(lambda: M.moe_layer_forward(dm0, x0, l0, w0, y=y0, ws=ws0, stream=stream),
                     100, stream)
        configs["tiny_t16"] = {"T": c0.T, "us_median": round(median(t), 2),
                               "tok/s": round(c0.T / (median(t) * 1e-6), 1),
                               "_inputs": (a0, w0np)}
        log(f"[bench] tiny_t16: {configs['tiny_t16']['us_median']} us")
        # T = 512, near-uniform routing: every expert used; two weight copies
        # alternated so consecutive calls do not find the weights in the caches
        c1 = G.CONFIGS["prefill_t512"]
        a1, x1, l1, w1np, w1 = upload(c1)
        w1b = M.W4Weights(*[M.W4Matrix(m.codes.clone(), m.scales.clone(), m.biases.clone())
                            for m in (w1.w13, w1.w2, w1.s13, w1.s2)])
        wcs1 = [w1.c(), w1b.c()]
        dm1 = M.dims(c1.T, c1.d, c1.f, c1.E, c1.k)
        ws1 = torch.empty(M.moe_layer_workspace_bytes(dm1), dtype=torch.uint8, device=dev)
        y1 = torch.empty((c1.T, c1.d), dtype=torch.float32, device=dev)
        it = [0]

        def call1():
            M.moe_layer_forward(dm1, x1, l1, None, y=y1, ws=ws1, wc=wcs1[it[0] % 2],
                                stream=stream)
            it[0] += 1

        t = event_us(call1, 50, stream)
        ne1 = len(np.unique(M.moe_route(l1, c1.k)[0].cpu().numpy()))
        by1 = ((ne1 + 1) * expert_bytes(c1.d, c1.f) + c1.T * (c1.d * 2 + c1.E * 4 + c1.d * 4))
        fl1 = sum(flops(c1.T, c1.d, c1.f, c1.k))
        us1 = median(t)
        configs["prefill_t512"] = {
            "T": c1.T, "bound": "hbm", "us_median": round(us1, 2),
            "tok/s": round(c1.T / (us1 * 1e-6), 1), "nonempty_experts": ne1,
            "algorithmic_bytes": by1, "GB/s": round(by1 / (us1 * 1e-6) / 1e9, 1),
            "frac_hbm": round(by1 / (us1 * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
            "TFLOP/s": round(fl1 / (us1 * 1e-6) / 1e12, 1), "weight_copies": 2,
            "_inputs": (a1, w1np)}
        log(f"[bench] prefill_t512: "
            f"{ {k_: v for k_, v in configs['prefill_t512'].items() if k_ != '_inputs'} }")
        del w1b, wcs1
        # T = 16384, skewed routing with 8 forced-empty experts
        c4 = G.CONFIGS["prefill_t16384_zipf_empty"]
        a4, x4, l4, w4np, w4 = upload(c4, weights=weights_np)  # same weights (same seed and shapes)
        dm4 = M.dims(c4.T, c4.d, c4.f, c4.E, c4.k)
        ws4 = torch.empty(M.moe_layer_workspace_bytes(dm4), dtype=torch.uint8, device=dev)
        y4 = torch.empty((c4.T, c4.d), dtype=torch.float32, device=dev)
        t = event_us(lambda: M.moe_layer_forward(dm4, x4, l4, w4, y=y4, ws=ws4, stream=stream),
                     20, stream)
        us4 = median(t)
        fg4, fd4 = flops(c4.T, c4.d, c4.f, c4.k)
        acc4, ne4 = kernel_times(M, dm4, x4, l4, w4, 5, stream)
        configs["prefill_t16384_zipf_empty"] = {
            "T": c4.T, "bound": "mfma", "us_median": round(us4, 2),
            "tok/s": round(c4.T / (us4 * 1e-6), 1), "nonempty_experts": ne4,
            "TFLOP/s": round((fg4 + fd4) / (us4 * 1e-6) / 1e12, 1),
            "frac_bf16_peak": round((fg4 + fd4) / (us4 * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "kernels": {n: round(v, 2) for n, v in acc4.items()},
            "gate_up_frac_bf16_peak": round(fg4 / (acc4["gate_up"] * 1e-6) / 1e12
                                            / PEAK_BF16_TFLOPS, 4),
            "down_frac_bf16_peak": round(fd4 / (acc4["down"] * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "_inputs": (a4, w4np)}
        log(f"[bench] prefill_t16384_zipf_empty: "
            f"{ {k_: v for k_, v in configs['prefill_t16384_zipf_empty'].items() if k_ != '_inputs'} }")
        del x4, l4, w4, ws4, y4
        # the headline layer with mixed dequantisation biases (some weight rows
        # with general biases: those wavefronts take the plain dequantisation)
        cm = G.MoeConfig("prefill_t4096_zipf_mixed_bias", T=T, d=d, f=f, E=E, k=k, zipf_s=1.1,
                         bias_mode=G.BIAS_MIXED)
        wm = M.W4Weights.from_numpy(G.make_weights(cm), device=dev)
        t = event_us(lambda: M.moe_layer_forward(dm, x, logits, wm, y=y, ws=ws, stream=stream),
                     20, stream)
        accm, _ = kernel_times(M, dm, x, logits, wm, 5, stream)
        mixed = {"workload": "prefill_t4096_zipf with mixed biases: 1% of the weight rows draw a "
                             "general bf16 bias per group, the rest bias = -8 scale",
                 "us_median": round(median(t), 2),
                 "TFLOP/s": round(flop_layer / (median(t) * 1e-6) / 1e12, 1),
                 "kernels": {n: round(v, 2) for n, v in accm.items()}}
        log(f"[bench] mixed biases: {mixed}")
        del wm

    # ---------------------------------------------------------------- small batches
    # moe_layer_forward at T = 1 .. 64 (the general path; T = 1 takes the
    # decode kernels), two weight copies alternated: a HIP graph of 32 calls
    # replayed three times (as a serving loop would run them), and events
    # around 100 calls issued one by one
    small = None
    if not args.no_small_batch:
        log("[bench] small batches")
        w2 = M.W4Weights.from_numpy(weights_np, device=dev)
        wcs = [wc, w2.c()]
        small = {}
        for Ts in (1, 2, 8, 32, 64):
            sc = G.small_config(f"small_t{Ts}", T=Ts, d=d, f=f, E=E, k=k, seed=7)
            sa = G.make_activations(sc)
            xs = torch.from_numpy(sa["x"].view(np.int16)).to(dev)
            ls = torch.from_numpy(sa["logits"]).to(dev)
            dms = M.dims(Ts, d, f, E, k)
            wss = torch.empty(M.moe_layer_workspace_bytes(dms), dtype=torch.uint8, device=dev)
            ys = torch.empty((Ts, d), dtype=torch.float32, device=dev)
            ne = len(np.unique(M.moe_route(ls, k)[0].cpu().numpy()))
            for i in range(10):
                M.moe_layer_forward(dms, xs, ls, w, y=ys, ws=wss, wc=wcs[i % 2])
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(100):
                M.moe_layer_forward(dms, xs, ls, w, y=ys, ws=wss, wc=wcs[i % 2])
            e1.record()
            torch.cuda.synchronize()
            us_eager = e0.elapsed_time(e1) * 10.0
            graph, gs = torch.cuda.CUDAGraph(), torch.cuda.Stream()
            with torch.cuda.stream(gs):
                with torch.cuda.graph(graph, stream=gs):
                    for i in range(32):
                        M.moe_layer_forward(dms, xs, ls, w, y=ys, ws=wss, wc=wcs[i % 2])
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            e0.record()
            for _ in range(3):
                graph.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / 96
            del graph
            by = (ne + 1) * expert_bytes(d, f) + Ts * (d * 2 + E * 4 + d * 4)
            small[f"T={Ts}"] = {"us": round(us, 2), "us_eager": round(us_eager, 2), "experts": ne,
                                "bytes": by, "GB/s": round(by / us / 1e3, 1),
                                "frac_hbm": round(by / us / 1e3 / PEAK_HBM_GBPS, 4)}
        del w2
        log(f"[bench] small batches: {small}")

    # ---------------------------------------------------------------- decode
    decode = None
    if not args.no_decode:
        dcfg = G.CONFIGS["decode_b1"]
        n_copies = 32
        log(f"[bench] decode: {args.decode_steps} steps, {n_copies} weight copies")
        steps = G.make_decode_steps(dcfg, args.decode_steps)
        xs = torch.from_numpy(steps["x"].view(np.int16)).to(dev)
        ls = torch.from_numpy(steps["logits"]).to(dev)
        wd = M.W4Weights.from_numpy(G.make_weights(dcfg), device=dev)
        copies = [wd]
        for _ in range(n_copies - 1):
            copies.append(M.W4Weights(*[M.W4Matrix(m.codes.clone(), m.scales.clone(),
                                                   m.biases.clone())
                                        for m in (wd.w13, wd.w2, wd.s13, wd.s2)]))
        cstructs = [c.c() for c in copies]
        dmd = M.dims(1, dcfg.d, dcfg.f, dcfg.E, dcfg.k)
        wsd = torch.empty(M.moe_layer_workspace_bytes(dmd), dtype=torch.uint8, device=dev)
        yd = torch.empty((args.decode_steps, dcfg.d), dtype=torch.float32, device=dev)

        def run_steps(lo, hi, st=None):
            for s in range(lo, hi):
                M.moe_layer_forward(dmd, xs[s:s + 1], ls[s:s + 1], None, y=yd[s:s + 1], ws=wsd,
                                    wc=cstructs[s % n_copies], stream=st)

        run_steps(0, min(64, args.decode_steps))
        torch.cuda.synchronize()
        # stream-launched loop (includes host launch overhead between steps)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run_steps(0, args.decode_steps)
        e1.record(stream)
        torch.cuda.synchronize()
        us_stream = e0.elapsed_time(e1) * 1e3 / args.decode_steps
        # the same steps captured as HIP graphs of n_copies steps each
        us_graph = None
        try:
            graphs = []
            gs = torch.cuda.Stream()
            chunk = n_copies
            with torch.cuda.stream(gs):
                for lo in range(0, args.decode_steps, chunk):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=gs):
                        run_steps(lo, min(lo + chunk, args.decode_steps), st=gs)
                    graphs.append(g)
            torch.cuda.synchronize()
            for g in graphs[:2]:
                g.replay()
            torch.cuda.synchronize()
            e0.record(stream)
            for g in graphs:
                g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            us_graph = e0.elapsed_time(e1) * 1e3 / args.decode_steps
        except Exception as ex:  # graph capture unavailable: keep the stream figure
            log(f"[bench] decode graph capture failed: {ex}")
        # the first 256 steps again from hidden states: the router projection
        # (x . Wr^T) and the layer, in graphs of n_copies steps
        us_hidden = None
        try:
            wrd = torch.from_numpy(G.make_router(dcfg).view(np.int16)).to(dev)
            nh = min(256, args.decode_steps)

            def run_hidden(lo, hi, st=None):
                for s in range(lo, hi):
                    M.moe_layer_forward_hidden(dmd, xs[s:s + 1], wrd, None, y=yd[s:s + 1], ws=wsd,
                                               wc=cstructs[s % n_copies], stream=st)

            run_hidden(0, min(n_copies, nh))
            torch.cuda.synchronize()
            hgraphs, hs = [], torch.cuda.Stream()
            with torch.cuda.stream(hs):
                for lo in range(0, nh, n_copies):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=hs):
                        run_hidden(lo, min(lo + n_copies, nh), st=hs)
                    hgraphs.append(g)
            torch.cuda.synchronize()
            hgraphs[0].replay()
            torch.cuda.synchronize()
            e0.record(stream)
            for g in hgraphs:
                g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            us_hidden = e0.elapsed_time(e1) * 1e3 / nh
            del hgraphs
        except Exception as ex:  # graph capture unavailable
            log(f"[bench] decode from hidden states: graph capture failed: {ex}")
        bytes_step = 9 * expert_bytes(dcfg.d, dcfg.f) + dcfg.d * 2 + dcfg.E * 4 + dcfg.d * 4
        best = us_graph if us_graph is not None else us_stream
        decode = {"workload": "decode_b1 (T=1, d=2048, f=512, E=256, top-8 + shared, 1000 steps)",
                  "bytes_per_step": bytes_step, "us_per_step": round(best, 3),
                  "GB/s": round(bytes_step / (best * 1e-6) / 1e9, 1),
                  "frac_hbm": round(bytes_step / (best * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
                  "us_per_step_stream_loop": round(us_stream, 3),
                  "us_per_step_graph": None if us_graph is None else round(us_graph, 3),
                  "us_per_step_from_hidden_states": None if us_hidden is None else round(us_hidden, 3),
                  "tok/s": round(1e6 / best, 1), "weight_copies": n_copies}
        log(f"[bench] decode: {decode}")
        del copies, cstructs

    # ---------------------------------------------------------------- CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import moe_oracle as O
        try:
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        except Exception:
            cores = os.cpu_count()
        granted = len(os.sched_getaffinity(0))

        def oracle_time(a, wt, c):
            t_ = time.perf_counter()
            O.layer_forward(a["x"], a["logits"], wt, c.k, BM=M.moe_block_m())
            return time.perf_counter() - t_

        log(f"[bench] CPU oracle on the whole {cfg.name} layer")
        dt = oracle_time(inp, weights_np, cfg)
        cpu = {"value": round(T / dt, 2), "unit": "tok/s", "cores": cores, "kind": "oracle",
               "sample": f"the whole {cfg.name} layer ({T} tokens; route, permute, dequantise "
                         f"every used expert, fp64 FFNs, combine) in {dt:.1f} s; host cores "
                         f"granted {granted}, BLAS threads {cores}"}
        if configs is not None and not args.cpu_headline_only:
            for name, c_ in (("tiny_t16", G.CONFIGS["tiny_t16"]),
                             ("prefill_t512", G.CONFIGS["prefill_t512"]),
                             ("prefill_t16384_zipf_empty",
                              G.CONFIGS["prefill_t16384_zipf_empty"])):
                a_, wt_ = configs[name]["_inputs"]
                log(f"[bench] CPU oracle on the whole {name} layer")
                dt_ = oracle_time(a_, wt_, c_)
                configs[name]["cpu_oracle"] = {"s": round(dt_, 3),
                                               "tok/s": round(c_.T / dt_, 2), "cores": cores}
    if configs is not None:
        for v in configs.values():
            v.pop("_inputs", None)

    out = {
        "metric": "MoE-layer prefill tok/s @T=4096 (% bf16 MFMA peak); decode B=1 HBM GB/s",
        "value": round(tok_s, 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "precision": "bf16 MFMA operands (int4-g64 weights dequantised to bf16), fp32 "
                     "accumulation, fp32 output",
        "data": "synthetic (seeded; random int4 codes, bf16 scales U(0.005,0.02), bias -8*scale)",
        "config": {"workload": "prefill_t4096_zipf: one MoE layer, T=4096, d=2048, f=512, "
                               "E=256, top-8 + 1 shared expert, Zipf(1.1)-skewed routing",
                   "T": T, "d": d, "f": f, "E": E, "k": k, "nonempty_experts": int(nonempty)},
        "layer": {"TFLOP/s": round(flop_layer / (ms_per_step / 1e3) / 1e12, 1),
                  "frac_bf16_peak": round(flop_layer / (ms_per_step / 1e3) / 1e12
                                          / PEAK_BF16_TFLOPS, 4),
                  "algorithmic_bytes": int(bytes_layer),
                  "GB/s": round(bytes_layer / (ms_per_step / 1e3) / 1e9, 1)},
        "roofline": roofline,
        "kernels": kernels,
        "configs": configs,
        "mixed_bias": mixed,
        "decode": decode,
        "small_batch": small,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
