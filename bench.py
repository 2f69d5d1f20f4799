#!/usr/bin/env python3
"""MoE decode layer benchmark on one MI355X.

A step is one whole MoE layer forward (router GEMV, top-k selection, counting
sort, pass 1, pass 2, combine) over one decode batch, all through
``moe_layer_fwd``.  The default workload is the uniform-routing batch sweep
layer: E=256 experts, top_k=8, H=2048, I=768, bf16 experts (9 MiB each).
Steps rotate over several resident copies of the layer (distinct seeded
weights) and several seeded activation draws, so consecutive steps never
re-read the same expert bytes from the 256 MiB Infinity Cache; the steps are
recorded once into a HIP graph and replayed.

Reported: layer steps/s at the headline batch size, and for every batch size
of the sweep the achieved HBM GB/s on unique-expert bytes
(n_uniq * 3 * H * I * bytes per weight, n_uniq read back from each step's
statistics), the roofline of the expert phase, and the CPU oracle timed on
a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0

# HBM traffic of pass1_kernel per launch at the headline configuration
# (uniform routing, bs=64), from rocprofv3 FETCH_SIZE / WRITE_SIZE runs
# scaled by a 1 GiB copy calibration: profiles/pass_kernels_uniform_bs64_hbm_counters.md.
# Reported only while the kernel source is the one that was measured.
PASS1_TRAFFIC_BS64 = {"read_bytes": 1.39999e9, "write_bytes": 1.83531e6, "source": "3ce981aa6142f3dc"}


def pass1_source_fingerprint():
    """Hash of the pass-1 GEMV kernel source: the grouped-GEMV section of
    experts_impl.h (segments through pass 1), the chunk dot products of
    common.h and the persistent grid size of experts.hip."""
    import hashlib

    d = os.path.join(ROOT, "mixture_experts_decode_gemv_amd", "csrc")
    impl = open(os.path.join(d, "experts_impl.h")).read()
    common = open(os.path.join(d, "common.h")).read()
    launch = open(os.path.join(d, "experts.hip")).read()
    a = impl[impl.index("struct SegArgs"):impl.index("// ---- pass 2: down rows")]
    b = common[common.index("// acc + sum_e w[e]"):common.index("// Sum over the 64 lanes")]
    c = launch[launch.index("static int persistent_grid"):launch.index("// Segments with at least kMfmaMinRoutes")]
    return hashlib.sha256((a + b + c).encode()).hexdigest()[:16]
MFMA_PEAK_TFS = 2500.0  # dense bf16


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--bs", type=int, default=64, help="headline batch size")
    ap.add_argument("--sweep", default="1,4,8,16,32,64", help="batch sizes reported besides the headline")
    ap.add_argument("--layers", type=int, default=4, help="resident layer copies rotated over")
    ap.add_argument("--draws", type=int, default=16, help="activation draws rotated over")
    ap.add_argument("--walk", default="dedup", choices=["dedup", "per_route", "dedup_pass1"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU oracle sample")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-mfma", action="store_true", help="keep every segment on the GEMV kernels")
    ap.add_argument("--workload", default="sweep", choices=["sweep", "skewed", "stack", "large"],
                    help="sweep: one layer, uniform routing, batch sweep (headline); "
                         "skewed: E=256 top_k=6 Zipf(1.1) routing, bs 1/8/32/64; "
                         "stack: 30-layer stack, one HIP graph vs a host-sync arm; "
                         "large: E=256 H=4096 I=1536 Zipf layer at bs 128/256/512 with MFMA segments")
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "fp8", "mxfp4"],
                    help="expert weights: bf16 or mxfp4 (every workload but stack), fp8 (large workload)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a device-to-device copy of this many MiB, 3 times (reference for HBM counters)")
    return ap.parse_args()


def copy_calibration(mib):
    """A plain device-to-device copy of known size, for scaling the HBM
    traffic counters (FETCH_SIZE / WRITE_SIZE) of the other kernels."""
    import torch

    n = mib * 2 ** 20 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4, "repeats": 3}), flush=True)


def stage_events(torch, n):
    """n sets of MOE_N_STAGES + 1 timing events, each recorded once so that
    its HIP handle exists."""
    import mixture_experts_decode_gemv_amd as moe

    sets = []
    for _ in range(n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(moe.MOE_N_STAGES + 1)]
        for e in evs:
            e.record()
        sets.append(evs)
    torch.cuda.synchronize()
    return sets


def time_layer(torch, moe, layers, xs, T, walk, steps, warmup, graph=True, stage_steps=None):
    """Replay len(plan) layer steps (layer l, draw d) in a HIP graph; then the
    same steps eagerly through moe_layer_fwd_events for per-stage times.
    Returns a dict with ms/step, per-draw routing statistics and stage times."""
    dev = xs[0].device
    stream = torch.cuda.Stream(dev)
    spec = layers[0].spec
    G = max(len(layers), len(xs))
    plan = [(s % len(layers), s % len(xs)) for s in range(G)]
    ws = layers[0].workspace(T, stream)
    out = torch.empty((T, spec.H), dtype=torch.float32, device=dev)

    def step(i):
        li, di = plan[i % G]
        moe.moe_layer_fwd(layers[li].struct, xs[di], T, out, walk, ws, ws.numel(), stream)

    # routing statistics of every planned step (read back outside the timed region)
    uniq, counts = [], []
    with torch.cuda.stream(stream):
        for i in range(G):
            step(i)
            stream.synchronize()
            uniq.append(int(ws[:4].view(torch.int32).item()))
            off = moe.moe_layer_routing(layers[plan[i][0]].struct, T, ws, ws.numel())["counts"] - ws.data_ptr()
            counts.append(ws[off:off + 4 * spec.E].view(torch.int32).cpu().numpy())
    g = None
    if graph:
        with torch.cuda.stream(stream):
            for i in range(3 * G):
                step(i)
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(G):
                step(i)
        stream.synchronize()
    reps = max(1, (steps + G - 1) // G)
    wreps = max(1, (warmup + G - 1) // G)

    def run(n):
        for _ in range(n):
            if g is not None:
                g.replay()
            else:
                for i in range(G):
                    step(i)

    with torch.cuda.stream(stream):
        run(wreps)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        run(reps)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (reps * G)
    # spread: a separate short run with an event between consecutive replays
    # (G steps each), kept out of the timed region above
    nsp = min(reps, 8)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(nsp + 1)]
    with torch.cuda.stream(stream):
        evs[0].record(stream)
        for r in range(nsp):
            run(1)
            evs[r + 1].record(stream)
    torch.cuda.synchronize()
    per_replay = np.array([evs[r].elapsed_time(evs[r + 1]) / G for r in range(nsp)])
    spread = {"p10": float(np.percentile(per_replay, 10)), "p50": float(np.percentile(per_replay, 50)),
              "p90": float(np.percentile(per_replay, 90))}

    # per-stage times: the same steps, eager, with events between the stages
    ns = stage_steps or G
    sets = stage_events(torch, ns)
    with torch.cuda.stream(stream):
        for i in range(G):
            step(i)
        for i in range(ns):
            li, di = plan[i % G]
            moe.moe_layer_fwd_events(layers[li].struct, xs[di], T, out, walk, ws, ws.numel(), stream,
                                     [e.cuda_event for e in sets[i]])
    torch.cuda.synchronize()
    st = np.array([[sets[i][j].elapsed_time(sets[i][j + 1]) for j in range(moe.MOE_N_STAGES)] for i in range(ns)])
    stage_ms = dict(zip(moe.STAGES, st.mean(axis=0).tolist()))
    del g
    # stage_steps: index into uniq/counts of each event-timed step
    return dict(ms=ms, timed_steps=reps * G, uniq=uniq, counts=counts, plan=plan, stage_ms=stage_ms,
                stage_steps=[i % G for i in range(ns)], spread_ms=spread)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the layer is built and timed on a single MI355X; "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)
        return
    if args.workload == "stack":
        bench_stack(args)
        return
    if args.workload == "large":
        bench_large(args)
        return

    import torch

    import mixture_experts_decode_gemv_amd as moe
    import workload as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    skewed = args.workload == "skewed"
    spec = wl.SKEWED if skewed else wl.SWEEP
    if args.dtype not in ("bf16", "mxfp4"):
        print("bench.py: the %s workload takes bf16 or mxfp4 experts" % args.workload, file=sys.stderr)
        sys.exit(2)
    mx = args.dtype == "mxfp4"
    if mx:
        spec = wl.LayerSpec(E=spec.E, top_k=spec.top_k, H=spec.H, I=spec.I, expert_dtype=wl.MXFP4,
                            router_dtype=spec.router_dtype)
    wname = "MXFP4 (E2M1, E8M0 scale per 32)" if mx else "bf16"
    bias = wl.zipf_bias(spec.E) if skewed else None
    walk = {"dedup": moe.MOE_WALK_DEDUP, "per_route": moe.MOE_WALK_PER_ROUTE,
            "dedup_pass1": moe.MOE_WALK_DEDUP_PASS1}[args.walk]
    if args.no_mfma:
        walk |= moe.MOE_NO_MFMA
    bpw = 17 / 32 if mx else 2  # bytes per weight: MXFP4 half a byte plus one scale byte per 32
    expert_bytes = 3 * spec.H * spec.I * bpw
    gate_up_bytes = 2 * spec.H * spec.I * bpw

    t0 = time.time()
    layers = []
    host0 = None
    for l in range(args.layers):
        w = wl.make_layer(spec, layer=l)
        layers.append(moe.DeviceLayer(w, bias, device=dev))
        if l == 0:
            host0 = w
        del w
    print("[bench] %d layers generated and resident (%.1f s)" % (args.layers, time.time() - t0), file=sys.stderr,
          flush=True)

    sweep = args.sweep
    if skewed and sweep == "1,4,8,16,32,64":
        sweep = ",".join(str(t) for t in wl.SKEWED_BS)
    sizes = sorted(set([args.bs] + [int(s) for s in sweep.split(",") if s]))
    results, head_run = {}, None
    for T in sizes:
        xs = [torch.from_numpy(wl.make_x(T, spec.H, draw=d)).to(dev) for d in range(args.draws)]
        run = time_layer(torch, moe, layers, xs, T, walk, args.steps, args.warmup, graph=not args.no_graph)
        ms = run["ms"]
        mean_u = float(np.mean(run["uniq"]))
        gbs = mean_u * expert_bytes / (ms * 1e-3) / 1e9
        results[T] = dict(bs=T, ms_per_step=ms, steps_per_s=1e3 / ms, unique_experts=mean_u,
                          reuse=T * spec.top_k / mean_u, unique_expert_MiB=mean_u * expert_bytes / 2 ** 20,
                          hbm_GBps=gbs, hbm_frac=gbs / HBM_PEAK_GBS, timed_steps=run["timed_steps"],
                          us_per_step_over_replays={k: v * 1e3 for k, v in run["spread_ms"].items()},
                          stage_us={k: v * 1e3 for k, v in run["stage_ms"].items()})
        if T == args.bs:
            head_run = run
        sp = run["spread_ms"]
        print("[bench] bs=%d  %.1f us/step (p10/p50/p90 %.1f/%.1f/%.1f)  %.0f steps/s  U=%.1f  %.0f GB/s (%.1f%% of 8 TB/s)"
              "  stages(us) %s"
              % (T, ms * 1e3, sp["p10"] * 1e3, sp["p50"] * 1e3, sp["p90"] * 1e3, 1e3 / ms, mean_u, gbs,
                 100 * gbs / HBM_PEAK_GBS, " ".join("%s=%.1f" % (k, v * 1e3) for k, v in run["stage_ms"].items())),
              file=sys.stderr, flush=True)
        del xs

    # roofline of the dominant kernel at the headline batch: pass 1 (grouped
    # GEMV), algorithmic bytes = gate_up bytes of the unique experts
    T = args.bs
    # experts that the GEMV kernel streams: those below the MFMA threshold
    # (all of them when the MFMA path is off or T < 16)
    mfma_on = not args.no_mfma and T >= 16 and args.walk != "per_route"
    u_gemv = [int((c > 0).sum() - ((c >= 16).sum() if mfma_on else 0)) for c in
              (head_run["counts"][i] for i in head_run["stage_steps"])]
    p1_ms = head_run["stage_ms"]["pass1_gemv"]
    p1_bytes = float(np.mean(u_gemv)) * gate_up_bytes
    p1_gbs = p1_bytes / (p1_ms * 1e-3) / 1e9

    # measured HBM bytes per pass-1 launch (headline configuration only, and
    # only for the kernel source the counters were taken on)
    traffic = None
    if (not skewed and not mx and args.bs == 64 and args.walk == "dedup" and not args.no_mfma
            and pass1_source_fingerprint() == PASS1_TRAFFIC_BS64["source"]):
        traffic = PASS1_TRAFFIC_BS64["read_bytes"] + PASS1_TRAFFIC_BS64["write_bytes"]

    # ---- CPU oracle on a bounded sample ------------------------------------------
    cpu = None
    if not args.no_cpu:
        import oracle

        olayer = oracle.Layer(host0, bias)
        nthreads = max(1, min(os.cpu_count() or 1, 16))
        done, t_start = 0, time.time()
        while True:
            oracle.moe_layer(olayer, wl.make_x(T, spec.H, draw=done), nthreads=nthreads)
            done += 1
            if time.time() - t_start >= args.cpu_seconds:
                break
        el = time.time() - t_start
        cpu = dict(value=done / el, unit="steps/s", cores=nthreads, kind="oracle",
                   sample="%d whole layer steps at bs=%d (E=256, k=%d, H=2048, I=768, %s%s), fp64 "
                          "accumulation, %.1f s" % (done, T, spec.top_k, wname, ", Zipf bias" if skewed else "", el))

    head = results[args.bs]
    line = {
        "metric": "MoE layer steps/s at bs=%d (%s routing, E=256, top_k=%d, H=2048, I=768, %s); "
                  "achieved HBM GB/s on unique-expert bytes" % (args.bs, "Zipf(1.1)" if skewed else "uniform",
                                                              spec.top_k, "mxfp4" if mx else "bf16"),
        "value": head["steps_per_s"],
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": head["timed_steps"],
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4" if mx else "bf16",
        "data": "synthetic (seeded N(0, 1/sqrt(fan_in)) weights, N(0,1) activations)",
        "config": {"workload": "single MoE layer, %s routing, E=256 top_k=%d H=2048 I=768 %s experts, batch "
                               "sweep" % ("Zipf(1.1)" if skewed else "uniform", spec.top_k, wname), "bs": args.bs,
                   "walk": args.walk, "mfma": not args.no_mfma, "resident_layers": args.layers,
                   "draws": args.draws, "graph": not args.no_graph, "parallelism": "none (1 GPU)"},
        "hbm_GBps_unique_expert_bytes": head["hbm_GBps"],
        "sweep": [results[t] for t in sizes],
        "roofline": {"bound": "hbm", "kernel": "pass1_kernel (grouped GEMV, gate_up rows x routes)",
                     "achieved": p1_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": p1_gbs / HBM_PEAK_GBS,
                     "traffic": traffic, "avg_launch_us": p1_ms * 1e3, "bytes_per_launch": p1_bytes,
                     "bytes_rule": "unique experts on the GEMV path x 2I x H x %s (gate_up, %s)" %
                                   ("17/32 B (codes and E8M0 scales)" if mx else "2 B", "mxfp4" if mx else "bf16")},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def bench_large(args):
    """Large-batch regime: one layer E=256, top_k=8, H=4096, I=1536 with
    Zipf(1.1)-skewed routing, bs 128/256/512, bf16, fp8 e4m3 experts with
    128x128 block scales or MXFP4 experts.  Experts holding >= 16 routes run
    on MFMA."""
    import torch

    import mixture_experts_decode_gemv_amd as moe
    import workload as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    spec = {"fp8": wl.LARGE_FP8, "mxfp4": wl.LARGE_MXFP4}.get(args.dtype, wl.LARGE)
    # bytes per weight, scales included: fp8 1 (+ 4 per 128x128 block), MXFP4
    # half a byte plus one scale byte per 32
    bpw = {wl.FP8: 1 + 4 / (128 * 128), wl.MXFP4: 17 / 32}.get(spec.expert_dtype, 2)
    H, I = spec.H, spec.I
    expert_bytes = 3 * H * I * bpw
    bias = wl.zipf_bias(spec.E)
    t0 = time.time()
    host = wl.make_layer(spec)
    layer = moe.DeviceLayer(host, bias, device=dev)
    print("[bench] large %s layer resident (%.1f s)" % (args.dtype, time.time() - t0), file=sys.stderr, flush=True)
    sizes = [int(s) for s in args.sweep.split(",")] if args.sweep != "1,4,8,16,32,64" else list(wl.LARGE_BS)
    bs_head = args.bs if args.bs in sizes else max(sizes)
    rows = {}
    for T in sizes:
        xs = [torch.from_numpy(wl.make_x(T, H, draw=d)).to(dev) for d in range(args.draws)]
        run = time_layer(torch, moe, [layer], xs, T, moe.MOE_WALK_DEDUP, args.steps, args.warmup,
                         graph=not args.no_graph)
        ms = run["ms"]
        st = run["stage_ms"]
        ev_idx = run["stage_steps"]
        u = float(np.mean(run["uniq"]))
        u_ev = float(np.mean([run["uniq"][i] for i in ev_idx]))
        cs = [run["counts"][i] for i in ev_idx]
        big = [c[c >= 16] for c in cs]
        n_big = float(np.mean([len(b) for b in big]))
        routes_big = float(np.mean([b.sum() for b in big]))
        tiles_big = float(np.mean([(np.ceil(b / 16) * 16).sum() for b in big]))
        flops_useful = 2 * routes_big * 3 * H * I
        flops_issued = 2 * tiles_big * 3 * H * I
        mfma_ms = st["pass1_mfma"] + st["pass2_mfma"]
        mfma_tf = flops_useful / (mfma_ms * 1e-3) / 1e12 if mfma_ms > 0 else 0.0
        p1m_bytes = n_big * 2 * I * H * bpw
        p1m_gbs = p1m_bytes / (st["pass1_mfma"] * 1e-3) / 1e9 if st["pass1_mfma"] > 0 else 0.0
        gbs = u * expert_bytes / (ms * 1e-3) / 1e9
        rows[T] = dict(bs=T, ms_per_step=ms, steps_per_s=1e3 / ms, unique_experts=u, mfma_experts=n_big,
                       mfma_route_frac=routes_big / (T * spec.top_k), hbm_GBps=gbs, hbm_frac=gbs / HBM_PEAK_GBS,
                       stage_us={k: v * 1e3 for k, v in st.items()},
                       mfma_TFLOPs_useful=mfma_tf, mfma_frac_of_peak=mfma_tf / MFMA_PEAK_TFS,
                       mfma_issued_over_useful=flops_issued / max(flops_useful, 1.0),
                       pass1_mfma_GBps=p1m_gbs, timed_steps=run["timed_steps"], unique_ev=u_ev,
                       us_per_step_over_replays={k: v * 1e3 for k, v in run["spread_ms"].items()})
        print("[bench] large %s bs=%d  %.1f us/step  U=%.1f (MFMA %.1f, %.0f%% of routes)  %.0f GB/s (%.1f%%)  "
              "MFMA %.0f TF/s useful  stages(us) %s" %
              (args.dtype, T, ms * 1e3, u, n_big, 100 * routes_big / (T * spec.top_k), gbs,
               100 * gbs / HBM_PEAK_GBS, mfma_tf, " ".join("%s=%.1f" % (k, v * 1e3) for k, v in st.items())),
              file=sys.stderr, flush=True)
        del xs
    head = rows[bs_head]
    cpu = None
    if not args.no_cpu:
        import oracle

        olayer = oracle.Layer(host, bias)
        nthreads = max(1, min(os.cpu_count() or 1, 16))
        x = wl.make_x(bs_head, H, draw=0)
        done, t_start = 0, time.time()
        while done < bs_head:
            n = min(4, bs_head - done)
            oracle.moe_layer(olayer, x[done:done + n], nthreads=nthreads)
            done += n
            if time.time() - t_start >= args.cpu_seconds:
                break
        el = time.time() - t_start
        cpu = dict(value=(done / bs_head) / el, unit="steps/s", cores=nthreads, kind="oracle",
                   sample="%d of the %d tokens of one bs=%d step (whole layer per token, fp64), %.1f s, scaled "
                          "to a step" % (done, bs_head, bs_head, el))
    st = head["stage_us"]
    dom = max(st, key=st.get)
    # algorithmic bytes of each stage at the headline batch: weights of the
    # experts it streams (GEMV: below 16 routes, MFMA: 16 or more)
    n_gemv = head["unique_ev"] - head["mfma_experts"]
    per_expert = {"pass1": 2 * I * H * bpw, "pass2": H * I * bpw}
    stage_bytes = {"pass1_gemv": n_gemv * per_expert["pass1"], "pass1_mfma": head["mfma_experts"] * per_expert["pass1"],
                   "pass2_gemv": n_gemv * per_expert["pass2"], "pass2_mfma": head["mfma_experts"] * per_expert["pass2"],
                   "routing": spec.E * H * 2, "combine": 0}
    dom_gbs = stage_bytes[dom] / (st[dom] * 1e-6) / 1e9 if st[dom] > 0 else 0.0
    kernel_of = {"pass1_gemv": "pass1_kernel", "pass1_mfma": "mfma_kernel (pass 1)", "pass2_gemv": "pass2_kernel",
                 "pass2_mfma": "mfma_kernel (pass 2)", "routing": "route_kernel", "combine": "combine_kernel"}
    line = {
        "metric": "MoE layer steps/s at bs=%d (Zipf(1.1) routing, E=256, top_k=8, H=4096, I=1536, %s); "
                  "achieved HBM GB/s on unique-expert bytes; MFMA TFLOP/s" % (bs_head, spec_name(args.dtype)),
        "value": head["steps_per_s"], "unit": "steps/s", "n_gpus": 1, "steps": head["timed_steps"],
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": {"fp8": "fp8_e4m3 weights, bf16 MFMA operands",
                                       "mxfp4": "mxfp4 weights, bf16 MFMA operands"}.get(args.dtype, "bf16"),
        "data": "synthetic (seeded)",
        "config": {"workload": "large-batch single MoE layer, Zipf(1.1) routing, E=256 top_k=8 H=4096 I=1536 "
                               "%s experts, MFMA for experts with >= 16 routes" % spec_name(args.dtype),
                   "bs": bs_head, "draws": args.draws, "graph": not args.no_graph},
        "hbm_GBps_unique_expert_bytes": head["hbm_GBps"],
        "sweep": [rows[t] for t in sizes],
        "roofline": {"bound": "hbm", "kernel": kernel_of[dom], "stage": dom, "achieved": dom_gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": dom_gbs / HBM_PEAK_GBS, "traffic": None,
                     "avg_launch_us": st[dom], "bytes_per_launch": stage_bytes[dom],
                     "bytes_rule": "experts the stage streams x their weight bytes (GEMV: < 16 routes, MFMA: >= 16)"},
        "mfma": {"achieved": head["mfma_TFLOPs_useful"], "peak": MFMA_PEAK_TFS, "unit": "TFLOP/s",
                 "frac": head["mfma_frac_of_peak"], "rule": "2 x MFMA routes x 3HI over pass 1 + pass 2 MFMA time"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def spec_name(dtype):
    return {"fp8": "fp8 e4m3 (128x128 block scales)", "mxfp4": "MXFP4 (E2M1, E8M0 scale per 32)"}.get(dtype, "bf16")


def host_topk(logits, k):
    """Host-side top-k of the host-sync arm: (logit desc, index asc), weights
    = softmax over the chosen logits (the pages' host selection)."""
    T, E = logits.shape
    order = np.lexsort((np.broadcast_to(np.arange(E), (T, E)), -logits), axis=1)[:, :k]
    chosen = np.take_along_axis(logits, order, axis=1).astype(np.float64)
    w = np.exp(chosen - chosen[:, :1])
    w /= w.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w.astype(np.float32)


def bench_stack(args):
    """30 layers (E=128, top_k=2, H=2048, I=1024, bf16, distinct weights per
    layer), RMSNorm before each router and a residual after each combine.
    Arm 1: all 30 moe_layer_fwd calls recorded in one HIP graph.  Arm 2: one
    moe_stack_fwd call recorded in one HIP graph (each layer's combine runs in
    the next layer's routing launch; bitwise the same output).  Arm 3: the
    host-synchronous design of the pages: after each router the logits are
    copied to the host, the stream is synchronised and the top-k is taken on
    the host, then the experts run on the device."""
    import torch

    import mixture_experts_decode_gemv_amd as moe
    import workload as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(dev)
    spec = wl.STACK
    nl = wl.STACK_LAYERS
    t0 = time.time()
    layers = []
    for l in range(nl):
        layers.append(moe.DeviceLayer(wl.make_layer(spec, layer=l), device=dev))
    print("[bench] %d stack layers resident (%.1f s)" % (nl, time.time() - t0), file=sys.stderr, flush=True)
    flags = moe.MOE_RMSNORM_IN | moe.MOE_ACCUM_RESIDUAL
    expert_bytes = 3 * spec.H * spec.I * 2
    rows = []
    for T in wl.STACK_BS:
        x0 = torch.from_numpy(wl.make_x(T, spec.H)).to(dev)
        h = x0.clone()
        ws = layers[0].workspace(T, stream)
        with torch.cuda.stream(stream):
            def step():
                for L in layers:
                    moe.moe_layer_fwd(L.struct, h, T, h, flags, ws, ws.numel(), stream)
            # unique experts per layer of one step (read outside the timed region)
            h.copy_(x0)
            uniq = []
            for L in layers:
                moe.moe_layer_fwd(L.struct, h, T, h, flags, ws, ws.numel(), stream)
                stream.synchronize()
                uniq.append(int(ws[:4].view(torch.int32).item()))
            step()
            stream.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                step()
            for _ in range(3):
                graph.replay()
        torch.cuda.synchronize()
        reps = max(5, args.steps // 10)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            h.copy_(x0)
            e0.record(stream)
            for _ in range(reps):
                graph.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        graph_ms = e0.elapsed_time(e1) / reps

        # fused arm: one moe_stack_fwd call in one graph
        sws_n = moe.moe_stack_workspace_bytes(layers[0].struct, T)
        sws = torch.empty(sws_n, dtype=torch.uint8, device=dev)
        structs = [L.struct for L in layers]
        with torch.cuda.stream(stream):
            moe.moe_stack_workspace_init(layers[0].struct, T, sws, sws_n, stream)
            h.copy_(x0)
            moe.moe_stack_fwd(structs, h, T, h, 0, sws, sws_n, stream)
            stream.synchronize()
            fgraph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(fgraph, stream=stream):
                moe.moe_stack_fwd(structs, h, T, h, 0, sws, sws_n, stream)
            for _ in range(3):
                fgraph.replay()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            h.copy_(x0)
            e0.record(stream)
            for _ in range(reps):
                fgraph.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        fused_ms = e0.elapsed_time(e1) / reps
        del fgraph

        # host-sync arm
        R = T * spec.top_k
        logits = torch.empty((T, spec.E), dtype=torch.float32, device=dev)
        ids_d = torch.empty((T, spec.top_k), dtype=torch.int32, device=dev)
        w_d = torch.empty((T, spec.top_k), dtype=torch.float32, device=dev)
        counts = torch.empty(spec.E, dtype=torch.int32, device=dev)
        offsets = torch.empty(spec.E + 1, dtype=torch.int32, device=dev)
        sorted_r = torch.empty(R, dtype=torch.int32, device=dev)
        uq = torch.empty(spec.E, dtype=torch.int32, device=dev)
        nu = torch.empty(1, dtype=torch.int32, device=dev)
        y = torch.empty_like(h)
        lg_host = torch.empty((T, spec.E), dtype=torch.float32, pin_memory=True)
        ids_host = torch.empty((T, spec.top_k), dtype=torch.int32, pin_memory=True)
        w_host = torch.empty((T, spec.top_k), dtype=torch.float32, pin_memory=True)
        scratch_ids = torch.empty((T, spec.top_k), dtype=torch.int32, device=dev)
        scratch_w = torch.empty((T, spec.top_k), dtype=torch.float32, device=dev)

        def host_sync_step():
            for L in layers:
                xn = h * torch.rsqrt(h.pow(2).mean(dim=1, keepdim=True) + 1e-6)
                moe.moe_route(L.struct, xn, None, T, logits, scratch_ids, scratch_w, ws, ws.numel(), stream)
                lg_host.copy_(logits, non_blocking=True)
                stream.synchronize()
                i_h, w_h = host_topk(lg_host.numpy(), spec.top_k)
                ids_host.numpy()[:] = i_h
                w_host.numpy()[:] = w_h
                ids_d.copy_(ids_host, non_blocking=True)
                w_d.copy_(w_host, non_blocking=True)
                moe.moe_sort(ids_d, T, spec.top_k, spec.E, counts, offsets, sorted_r, uq, nu, stream)
                moe.moe_expert_fwd(L.struct, xn, T, ids_d, w_d, counts, offsets, sorted_r, uq, nu, y, 0, ws,
                                   ws.numel(), stream)
                h.add_(y)

        with torch.cuda.stream(stream):
            h.copy_(x0)
            host_sync_step()
            stream.synchronize()
            hreps = max(3, reps // 2)
            t_start = time.perf_counter()
            for _ in range(hreps):
                host_sync_step()
            stream.synchronize()
            sync_ms = (time.perf_counter() - t_start) * 1e3 / hreps
        mean_u = float(np.mean(uniq))
        gbs = mean_u * nl * expert_bytes / (fused_ms * 1e-3) / 1e9
        rows.append(dict(bs=T, fused_graph_ms_per_step=fused_ms, graph_ms_per_step=graph_ms,
                         host_sync_ms_per_step=sync_ms, speedup=sync_ms / fused_ms, host_syncs_per_step_graph=0,
                         host_syncs_per_step_sync_arm=nl, unique_experts_per_layer=mean_u,
                         hbm_GBps_unique_expert_bytes=gbs))
        print("[bench] stack bs=%d  fused graph %.1f us/step  layer-call graph %.1f us/step  host-sync %.1f us/step  "
              "U/layer=%.2f  %.0f GB/s" % (T, fused_ms * 1e3, graph_ms * 1e3, sync_ms * 1e3, mean_u, gbs),
              file=sys.stderr, flush=True)
        del graph
    head = rows[0]
    print(json.dumps({
        "metric": "30-layer MoE decode stack steps/s (moe_stack_fwd in one HIP graph, zero host syncs) vs "
                  "layer calls in one graph and the host-sync arm",
        "value": 1.0 / head["fused_graph_ms_per_step"] * 1e3, "unit": "steps/s", "n_gpus": 1,
        "ms_per_step": head["fused_graph_ms_per_step"], "higher_is_better": True, "dtype": "bf16",
        "data": "synthetic (seeded)",
        "config": {"workload": "30 layers, E=128, top_k=2, H=2048, I=1024, bf16, RMSNorm + residual",
                   "bs": head["bs"]},
        "stack": rows}), flush=True)


if __name__ == "__main__":
    main()
