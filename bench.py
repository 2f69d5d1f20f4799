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
    ap.add_argument("--workload", default="sweep", choices=["sweep", "stack"],
                    help="sweep: one layer, uniform routing, batch sweep (headline); "
                         "stack: 30-layer stack, one HIP graph vs a host-sync arm")
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

    import torch

    import mixture_experts_decode_gemv_amd as moe
    import workload as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(dev)
    spec = wl.SWEEP
    walk = {"dedup": moe.MOE_WALK_DEDUP, "per_route": moe.MOE_WALK_PER_ROUTE,
            "dedup_pass1": moe.MOE_WALK_DEDUP_PASS1}[args.walk]
    bpw = 2  # bf16
    expert_bytes = 3 * spec.H * spec.I * bpw

    t0 = time.time()
    layers = []
    host0 = None
    for l in range(args.layers):
        w = wl.make_layer(spec, layer=l)
        layers.append(moe.DeviceLayer(w, device=dev))
        if l == 0:
            host0 = w
        del w
    print("[bench] %d layers generated and resident (%.1f s)" % (args.layers, time.time() - t0), file=sys.stderr,
          flush=True)

    sizes = sorted(set([args.bs] + [int(s) for s in args.sweep.split(",") if s]))
    maxT = max(sizes)
    ws = layers[0].workspace(maxT)
    out = torch.empty((maxT, spec.H), dtype=torch.float32, device=dev)
    results = {}

    for T in sizes:
        xs = [torch.from_numpy(wl.make_x(T, spec.H, draw=d)).to(dev) for d in range(args.draws)]
        G = max(args.layers, args.draws)
        plan = [(s % args.layers, s % args.draws) for s in range(G)]

        def step(i, with_stats=False):
            li, di = plan[i % G]
            moe.moe_layer_fwd(layers[li].struct, xs[di], T, out, walk, ws, ws.numel(), stream)

        # unique experts of every planned step (read back outside the timed region)
        uniq = []
        with torch.cuda.stream(stream):
            for i in range(G):
                step(i)
                stream.synchronize()
                uniq.append(int(ws[:4].view(torch.int32).item()))
        mean_u = float(np.mean(uniq))

        graph = None
        if not args.no_graph:
            with torch.cuda.stream(stream):
                for i in range(3 * G):
                    step(i)
            stream.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                for i in range(G):
                    step(i)
            stream.synchronize()

        reps = max(1, (args.steps + G - 1) // G)
        nsteps = reps * G
        wreps = max(1, (args.warmup + G - 1) // G)
        with torch.cuda.stream(stream):
            for _ in range(wreps):
                if graph is not None:
                    graph.replay()
                else:
                    for i in range(G):
                        step(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(reps):
                if graph is not None:
                    graph.replay()
                else:
                    for i in range(G):
                        step(i)
            e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / nsteps
        gbs = mean_u * expert_bytes / (ms * 1e-3) / 1e9
        results[T] = dict(bs=T, ms_per_step=ms, steps_per_s=1e3 / ms, unique_experts=mean_u,
                          reuse=T * spec.top_k / mean_u, unique_expert_MiB=mean_u * expert_bytes / 2 ** 20,
                          hbm_GBps=gbs, hbm_frac=gbs / HBM_PEAK_GBS, timed_steps=nsteps)
        print("[bench] bs=%d  %.1f us/step  %.0f steps/s  U=%.1f  %.0f GB/s (%.1f%% of 8 TB/s)"
              % (T, ms * 1e3, 1e3 / ms, mean_u, gbs, 100 * gbs / HBM_PEAK_GBS), file=sys.stderr, flush=True)
        del graph, xs

    # ---- expert phase of the headline batch, timed on its own ----------------
    T = args.bs
    xs = [torch.from_numpy(wl.make_x(T, spec.H, draw=d)).to(dev) for d in range(args.draws)]
    routed = []
    for li in range(args.layers):
        wsl = layers[li].workspace(T)
        with torch.cuda.stream(stream):
            moe.moe_layer_fwd(layers[li].struct, xs[li % args.draws], T, out, walk, wsl, wsl.numel(), stream)
        stream.synchronize()
        r = moe.moe_layer_routing(layers[li].struct, T, wsl, wsl.numel())
        routed.append((li, li % args.draws, wsl, r, int(wsl[:4].view(torch.int32).item())))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    with torch.cuda.stream(stream):
        for i in range(args.warmup + args.steps):
            li, di, wsl, r, u = routed[i % len(routed)]
            if i >= args.warmup:
                ev[i - args.warmup][0].record(stream)
            moe.moe_expert_fwd(layers[li].struct, xs[di], T, r["topk_ids"], r["topk_w"], r["counts"],
                               r["offsets"], r["sorted_routes"], r["uniq"], r["n_uniq"], out, walk, wsl,
                               wsl.numel(), stream)
            if i >= args.warmup:
                ev[i - args.warmup][1].record(stream)
    torch.cuda.synchronize()
    exp_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    exp_bytes = float(np.mean([routed[(i + args.warmup) % len(routed)][4] for i in range(args.steps)])) * expert_bytes
    exp_gbs = exp_bytes / (exp_ms * 1e-3) / 1e9

    # ---- CPU oracle on a bounded sample ------------------------------------------
    cpu = None
    if not args.no_cpu:
        import oracle

        olayer = oracle.Layer(host0)
        nthreads = max(1, min(os.cpu_count() or 1, 16))
        done, t_start = 0, time.time()
        while True:
            oracle.moe_layer(olayer, wl.make_x(T, spec.H, draw=done), nthreads=nthreads)
            done += 1
            if time.time() - t_start >= args.cpu_seconds:
                break
        el = time.time() - t_start
        cpu = dict(value=done / el, unit="steps/s", cores=nthreads, kind="oracle",
                   sample="%d whole layer steps at bs=%d (E=256, k=8, H=2048, I=768, bf16), fp64 accumulation, "
                          "%.1f s" % (done, T, el))

    head = results[args.bs]
    line = {
        "metric": "MoE layer steps/s at bs=%d (uniform routing, E=256, top_k=8, H=2048, I=768, bf16); "
                  "achieved HBM GB/s on unique-expert bytes" % args.bs,
        "value": head["steps_per_s"],
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": head["timed_steps"],
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0, 1/sqrt(fan_in)) weights, N(0,1) activations)",
        "config": {"workload": "single MoE layer, uniform routing, E=256 top_k=8 H=2048 I=768 bf16 experts, "
                               "batch sweep", "bs": args.bs, "walk": args.walk, "resident_layers": args.layers,
                   "draws": args.draws, "graph": not args.no_graph, "parallelism": "none (1 GPU)"},
        "hbm_GBps_unique_expert_bytes": head["hbm_GBps"],
        "sweep": [results[t] for t in sizes],
        "roofline": {"bound": "hbm", "kernel": "expert phase (moe_expert_fwd: pass 1, pass 2, combine)",
                     "achieved": exp_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": exp_gbs / HBM_PEAK_GBS,
                     "traffic": None, "avg_launch_ms": exp_ms, "bytes_per_launch": exp_bytes},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


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
    Arm 1: all 30 moe_layer_fwd calls recorded in one HIP graph.  Arm 2: the
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
        gbs = mean_u * nl * expert_bytes / (graph_ms * 1e-3) / 1e9
        rows.append(dict(bs=T, graph_ms_per_step=graph_ms, host_sync_ms_per_step=sync_ms,
                         speedup=sync_ms / graph_ms, host_syncs_per_step_graph=0, host_syncs_per_step_sync_arm=nl,
                         unique_experts_per_layer=mean_u, hbm_GBps_unique_expert_bytes=gbs))
        print("[bench] stack bs=%d  graph %.1f us/step  host-sync %.1f us/step  U/layer=%.2f  %.0f GB/s"
              % (T, graph_ms * 1e3, sync_ms * 1e3, mean_u, gbs), file=sys.stderr, flush=True)
        del graph
    head = rows[0]
    print(json.dumps({
        "metric": "30-layer MoE decode stack ms/step (one HIP graph, zero host syncs) vs host-sync arm",
        "value": 1.0 / head["graph_ms_per_step"] * 1e3, "unit": "steps/s", "n_gpus": 1,
        "ms_per_step": head["graph_ms_per_step"], "higher_is_better": True, "dtype": "bf16",
        "data": "synthetic (seeded)",
        "config": {"workload": "30 layers, E=128, top_k=2, H=2048, I=1024, bf16, RMSNorm + residual",
                   "bs": head["bs"]},
        "stack": rows}), flush=True)


if __name__ == "__main__":
    main()
