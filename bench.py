#!/usr/bin/env python3
"""MoE decode layer benchmark on one MI355X.

A step is one whole MoE layer forward (router GEMV, top-k selection, counting
sort, pass 1, pass 2, combine) over one decode batch, all through
``moe_layer_fwd``.  The headline workload is the uniform-routing batch sweep
layer: E=256 experts, top_k=8, H=2048, I=768, bf16 experts (9 MiB each).
Steps rotate over several resident copies of the layer (distinct seeded
weights) and several seeded activation draws, so consecutive steps never
re-read the same expert bytes from the 256 MiB Infinity Cache; exactly K steps
are recorded into one HIP graph and replayed once inside the timed region.

Reported in one JSON line:
  * layer steps/s at the headline batch size, and for every batch size of the
    sweep the achieved HBM GB/s on unique-expert bytes (n_uniq * 3 * H * I *
    bytes per weight, n_uniq read back from each step's statistics);
  * the three walk arms (per route, pass 1 once per unique expert, both passes
    once per unique expert) on the same draws, beside the traffic model of the
    dedup page: speedup 1 / (2/3 / reuse + 1/3) for pass-1 dedup, reuse for
    both passes (uniform and Zipf-skewed routing);
  * the skewed sweep, the 30-layer stack (one graph, zero host syncs, against a
    host-synchronous arm) and the large-batch layer (bf16 and fp8 experts, MFMA
    segments) as extra keys, each with its own roofline fraction;
  * the roofline of the dominant kernel, and a read-stream probe's measured
    bandwidth as a second denominator;
  * the CPU oracle timed on bounded samples of the same workloads.
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
MFMA_PEAK_TFS = 2500.0  # dense bf16

# HBM traffic of pass1_kernel per launch at the headline configuration
# (uniform routing, bs=64), from rocprofv3 FETCH_SIZE / WRITE_SIZE runs
# scaled by a 1 GiB copy calibration: profiles/pass_kernels_uniform_bs64_hbm_counters.md.
# Reported only while the kernel source is the one that was measured.
PASS1_TRAFFIC_BS64 = {"read_bytes": 1.38555e+09, "write_bytes": 1.53456e+06, "source": "b5d718c057119eb6"}


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
    c = launch[launch.index("static int persistent_grid"):launch.index("// Segments with at least mfma_min_routes")]
    return hashlib.sha256((a + b + c).encode()).hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200, help="timed steps (exactly these, one graph replay)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--bs", type=int, default=64, help="headline batch size")
    ap.add_argument("--sweep", default="1,4,8,16,32,64", help="batch sizes reported besides the headline")
    ap.add_argument("--layers", type=int, default=4, help="resident layer copies rotated over")
    ap.add_argument("--draws", type=int, default=16, help="activation draws rotated over")
    ap.add_argument("--walk", default="dedup", choices=["dedup", "per_route", "dedup_pass1"])
    ap.add_argument("--cpu-seconds", type=float, default=6.0, help="budget of the headline CPU oracle sample")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-mfma", action="store_true", help="keep every segment on the GEMV kernels")
    ap.add_argument("--no-extras", action="store_true",
                    help="headline sweep only (no arms, skewed, stack, large, probe or extra CPU legs)")
    ap.add_argument("--workload", default="sweep", choices=["sweep", "skewed", "stack", "large"],
                    help="sweep: everything, headline = uniform batch sweep; "
                         "skewed: E=256 top_k=6 Zipf(1.1) routing, bs 1/8/32/64; "
                         "stack: 30-layer stack, one HIP graph vs a host-sync arm; "
                         "large: E=256 H=4096 I=1536 Zipf layer at bs 128/256/512 with MFMA segments")
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "fp8", "mxfp4", "q4_0"],
                    help="expert weights: bf16, mxfp4 or q4_0 (every workload but stack), fp8 (large workload)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a device-to-device copy of this many MiB, 3 times (reference for HBM counters)")
    return ap.parse_args()


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


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


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_threads():
    """Host threads for the oracle: the cores this process may use, at most
    16 (the GPU machine's share for one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


# ---- GPU timing ------------------------------------------------------------------

def time_layer(torch, moe, layers, xs, T, flags, steps, warmup, graph=True, stage=True, spread_reps=4):
    """Exactly `steps` layer steps, step i on (layer i % L, draw i % D),
    recorded into one HIP graph (after `warmup` untimed steps in a graph of
    their own) and replayed once between two events.  Then, outside the
    timed region, a few more replays with an event between each (spread of
    the per-step time), and optionally the planned steps run eagerly through
    moe_layer_fwd_events for per-stage times.  Returns a dict with ms/step,
    the per-step routing statistics and the stage times."""
    dev = xs[0].device
    stream = torch.cuda.Stream(dev)
    P = max(len(layers), len(xs))
    plan = [(i % len(layers), i % len(xs)) for i in range(P)]
    ws = layers[0].workspace(T, stream)
    out = torch.empty((T, layers[0].spec.H), dtype=torch.float32, device=dev)
    E = layers[0].spec.E

    def step(i):
        li, di = plan[i % P]
        moe.moe_layer_fwd(layers[li].struct, xs[di], T, out, flags, ws, ws.numel(), stream)

    # routing statistics of every planned step (read back outside the timed region)
    uniq, counts = [], []
    routing = moe.moe_layer_routing(layers[0].struct, T, ws, ws.numel())
    off = routing["counts"] - ws.data_ptr()
    with torch.cuda.stream(stream):
        for i in range(P):
            step(i)
            stream.synchronize()
            uniq.append(int(ws[:4].view(torch.int32).item()))
            counts.append(ws[off:off + 4 * E].view(torch.int32).cpu().numpy())
        for i in range(2 * P):
            step(i)
    stream.synchronize()
    gk = gw = None
    if graph:
        gk = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gk, stream=stream):
            for i in range(steps):
                step(i)
        if warmup > 0:
            gw = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gw, stream=stream):
                for i in range(warmup):
                    step(i)
        stream.synchronize()

    def run_timed():
        if gk is not None:
            gk.replay()
        else:
            for i in range(steps):
                step(i)

    with torch.cuda.stream(stream):
        if gw is not None:
            gw.replay()
        elif warmup > 0:
            for i in range(warmup):
                step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        run_timed()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # spread over separate replays, outside the timed region
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(spread_reps + 1)]
    with torch.cuda.stream(stream):
        evs[0].record(stream)
        for r in range(spread_reps):
            run_timed()
            evs[r + 1].record(stream)
    torch.cuda.synchronize()
    per = np.array([evs[r].elapsed_time(evs[r + 1]) / steps for r in range(spread_reps)])
    spread = {"p10": float(np.percentile(per, 10)), "p50": float(np.percentile(per, 50)),
              "p90": float(np.percentile(per, 90))}
    stage_ms, stage_idx = None, []
    if stage:
        sets = stage_events(torch, P)
        with torch.cuda.stream(stream):
            for i in range(P):
                step(i)
            for i in range(P):
                li, di = plan[i]
                moe.moe_layer_fwd_events(layers[li].struct, xs[di], T, out, flags, ws, ws.numel(), stream,
                                         [e.cuda_event for e in sets[i]])
        torch.cuda.synchronize()
        st = np.array([[sets[i][j].elapsed_time(sets[i][j + 1]) for j in range(moe.MOE_N_STAGES)]
                       for i in range(P)])
        stage_ms = dict(zip(moe.STAGES, st.mean(axis=0).tolist()))
        stage_idx = list(range(P))
    del gk, gw
    # n_uniq over exactly the timed steps
    u_timed = float(np.mean([uniq[i % P] for i in range(steps)]))
    return dict(ms=ms, timed_steps=steps, uniq=uniq, uniq_timed=u_timed, counts=counts, plan=plan,
                stage_ms=stage_ms, stage_steps=stage_idx, spread_ms=spread)


def sweep_rows(torch, moe, wl, layers, spec, sizes, flags, steps, warmup, draws, expert_bytes, graph=True,
               label="bs", stage=True):
    """One time_layer run per batch size; rows with steps/s and HBM GB/s on
    unique-expert bytes."""
    dev = torch.device("cuda:0")
    rows, runs = {}, {}
    for T in sizes:
        xs = [torch.from_numpy(wl.make_x(T, spec.H, draw=d)).to(dev) for d in range(draws)]
        run = time_layer(torch, moe, layers, xs, T, flags, steps, warmup, graph=graph, stage=stage)
        ms = run["ms"]
        u = run["uniq_timed"]
        gbs = u * expert_bytes / (ms * 1e-3) / 1e9
        row = dict(bs=T, ms_per_step=ms, steps_per_s=1e3 / ms, unique_experts=u, reuse=T * spec.top_k / u,
                   unique_expert_MiB=u * expert_bytes / 2 ** 20, hbm_GBps=gbs, hbm_frac=gbs / HBM_PEAK_GBS,
                   timed_steps=run["timed_steps"],
                   us_per_step_over_replays={k: v * 1e3 for k, v in run["spread_ms"].items()},
                   max_count=float(np.mean([c.max() for c in run["counts"]])))
        if run["stage_ms"] is not None:
            row["stage_us"] = {k: v * 1e3 for k, v in run["stage_ms"].items()}
        rows[T] = row
        runs[T] = run
        sp = run["spread_ms"]
        log("%s=%d  %.1f us/step (p10/p50/p90 %.1f/%.1f/%.1f)  %.0f steps/s  U=%.1f  %.0f GB/s (%.1f%% of 8 TB/s)%s"
            % (label, T, ms * 1e3, sp["p10"] * 1e3, sp["p50"] * 1e3, sp["p90"] * 1e3, 1e3 / ms, u, gbs,
               100 * gbs / HBM_PEAK_GBS,
               ("  stages(us) " + " ".join("%s=%.1f" % (k, v * 1e3) for k, v in run["stage_ms"].items()))
               if run["stage_ms"] else ""))
        del xs
    return rows, runs


def walk_arms(torch, moe, wl, layers, spec, sizes, steps, warmup, draws, expert_bytes, tag):
    """The three walk arms of the dedup page on the same draws: per route
    ("off"), pass 1 once per unique expert, both passes once per unique
    expert.  Speedups of the dedup arms over the per-route arm beside the
    page's traffic model."""
    arms = {"per_route": moe.MOE_WALK_PER_ROUTE, "dedup_pass1": moe.MOE_WALK_DEDUP_PASS1,
            "dedup": moe.MOE_WALK_DEDUP}
    res = {}
    for name, f in arms.items():
        res[name], _ = sweep_rows(torch, moe, wl, layers, spec, sizes, f, steps, warmup, draws, expert_bytes,
                                  label="%s %s bs" % (tag, name), stage=False)
    out = []
    for T in sizes:
        reuse = res["dedup"][T]["reuse"]
        pr, p1, dd = (res[a][T]["ms_per_step"] * 1e3 for a in ("per_route", "dedup_pass1", "dedup"))
        out.append(dict(bs=T, reuse=reuse, unique_experts=res["dedup"][T]["unique_experts"],
                        us_per_step={"per_route": pr, "dedup_pass1": p1, "dedup": dd},
                        speedup_dedup_pass1=pr / p1, model_dedup_pass1=1.0 / (2.0 / 3.0 / reuse + 1.0 / 3.0),
                        speedup_dedup=pr / dd, model_dedup=reuse))
        log("%s arms bs=%d  reuse %.2f  per-route %.1f  dedup-pass1 %.1f (x%.2f, model x%.2f)  dedup %.1f us "
            "(x%.2f, model x%.2f)" % (tag, T, reuse, pr, p1, pr / p1, out[-1]["model_dedup_pass1"], dd, pr / dd,
                                      reuse))
    return out


def mfma_experts(c, thr, hot):
    """Experts of one call's counts c on the matrix cores: those holding thr
    routes or more (moe_mfma_min_routes), if the largest holds hot or more
    (moe_mfma_hot_routes); none when thr is 0."""
    return int((c >= thr).sum()) if thr > 0 and c.max() >= hot else 0


def stage_roofline(head_run, spec, T, bpw, thr, hot):
    """Roofline of pass1_kernel (the dominant kernel of the uniform sweep) at
    the headline batch: algorithmic bytes = gate_up bytes of the experts the
    GEMV kernel streams (those not on the matrix cores, see mfma_experts),
    over its event-timed average launch."""
    counts = [head_run["counts"][i] for i in head_run["stage_steps"]]
    u_gemv = [int((c > 0).sum()) - mfma_experts(c, thr, hot) for c in counts]
    p1_ms = head_run["stage_ms"]["pass1_gemv"]
    p1_bytes = float(np.mean(u_gemv)) * 2 * spec.H * spec.I * bpw
    return p1_bytes / (p1_ms * 1e-3) / 1e9, p1_ms, p1_bytes


# ---- read-stream probe -------------------------------------------------------------

def read_stream_probe(torch, gib=4, reps=6):
    """Achievable HBM read bandwidth: a plain streaming read of a 4 GiB buffer
    (far beyond the 256 MiB Infinity Cache) with 16-byte streaming loads, at
    a few persistent grid sizes; the best is reported."""
    import ctypes

    path = os.path.join(ROOT, "mixture_experts_decode_gemv_amd", "libmoe_probe_gfx950.so")
    if not os.path.exists(path):
        return None
    L = ctypes.CDLL(path)
    L.moe_probe_read_stream.restype = ctypes.c_int
    L.moe_probe_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.c_void_p]
    dev = torch.device("cuda:0")
    nbytes = gib << 30
    buf = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    ncu = torch.cuda.get_device_properties(dev).multi_processor_count
    best = None
    stream = torch.cuda.current_stream(dev)
    for per_cu in (4, 8, 16):
        grid = ncu * per_cu
        sink = torch.zeros(grid, dtype=torch.int32, device=dev)
        rc = L.moe_probe_read_stream(buf.data_ptr(), nbytes, grid, sink.data_ptr(), stream.cuda_stream)
        if rc != 0:
            return None
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            L.moe_probe_read_stream(buf.data_ptr(), nbytes, grid, sink.data_ptr(), stream.cuda_stream)
        e1.record(stream)
        torch.cuda.synchronize()
        gbs = nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
        if best is None or gbs > best["GBps"]:
            best = {"GBps": gbs, "grid": grid, "bytes": nbytes, "reps": reps}
    del buf
    best["frac_of_peak"] = best["GBps"] / HBM_PEAK_GBS
    log("read-stream probe: %.0f GB/s (%.1f%% of 8 TB/s), grid %d" % (best["GBps"], 100 * best["frac_of_peak"],
                                                                     best["grid"]))
    return best


# ---- the 30-layer stack -----------------------------------------------------------

def host_topk(logits, k):
    """Host-side top-k of the host-sync arm: (logit desc, index asc), weights
    = softmax over the chosen logits (the pages' host selection)."""
    T, E = logits.shape
    order = np.lexsort((np.broadcast_to(np.arange(E), (T, E)), -logits), axis=1)[:, :k]
    chosen = np.take_along_axis(logits, order, axis=1).astype(np.float64)
    w = np.exp(chosen - chosen[:, :1])
    w /= w.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w.astype(np.float32)


def stack_rows(torch, moe, wl, reps):
    """30 layers (E=128, top_k=2, H=2048, I=1024, bf16, distinct weights per
    layer), RMSNorm before each router and a residual after each combine.
    Arm 1: one moe_stack_fwd call recorded in one HIP graph.  Arm 2: all 30
    moe_layer_fwd calls recorded in one HIP graph (bitwise the same output).
    Arm 3: the host-synchronous design of the pages: after each router the
    logits are copied to the host, the stream is synchronised and the top-k
    is taken on the host, then the experts run on the device."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(dev)
    spec = wl.STACK
    nl = wl.STACK_LAYERS
    t0 = time.time()
    layers = [moe.DeviceLayer(wl.make_layer(spec, layer=l), device=dev) for l in range(nl)]
    log("%d stack layers resident (%.1f s)" % (nl, time.time() - t0))
    flags = moe.MOE_RMSNORM_IN | moe.MOE_ACCUM_RESIDUAL
    expert_bytes = 3 * spec.H * spec.I * 2
    router_bytes = spec.E * spec.H * 2
    rows = []
    structs = [L.struct for L in layers]
    for T in wl.STACK_BS:
        x0 = torch.from_numpy(wl.make_x(T, spec.H)).to(dev)
        h = x0.clone()
        ws = layers[0].workspace(T, stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

        def timed_graph(g):
            with torch.cuda.stream(stream):
                for _ in range(3):
                    g.replay()
                h.copy_(x0)
                e0.record(stream)
                for _ in range(reps):
                    g.replay()
                e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        with torch.cuda.stream(stream):
            # unique experts per layer of one step (read outside the timed region)
            h.copy_(x0)
            uniq = []
            for L in layers:
                moe.moe_layer_fwd(L.struct, h, T, h, flags, ws, ws.numel(), stream)
                stream.synchronize()
                uniq.append(int(ws[:4].view(torch.int32).item()))
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                for L in layers:
                    moe.moe_layer_fwd(L.struct, h, T, h, flags, ws, ws.numel(), stream)
        graph_ms = timed_graph(graph)
        del graph
        sws_n = moe.moe_stack_workspace_bytes(layers[0].struct, T)
        sws = torch.empty(sws_n, dtype=torch.uint8, device=dev)
        with torch.cuda.stream(stream):
            moe.moe_stack_workspace_init(layers[0].struct, T, sws, sws_n, stream)
            moe.moe_stack_fwd(structs, h, T, h, 0, sws, sws_n, stream)
            stream.synchronize()
            fgraph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(fgraph, stream=stream):
                moe.moe_stack_fwd(structs, h, T, h, 0, sws, sws_n, stream)
        fused_ms = timed_graph(fgraph)
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
            hreps = max(2, reps // 4)
            t_start = time.perf_counter()
            for _ in range(hreps):
                host_sync_step()
            stream.synchronize()
            sync_ms = (time.perf_counter() - t_start) * 1e3 / hreps
        mean_u = float(np.mean(uniq))
        step_bytes = mean_u * nl * expert_bytes
        gbs = step_bytes / (fused_ms * 1e-3) / 1e9
        rows.append(dict(bs=T, fused_graph_ms_per_step=fused_ms, graph_ms_per_step=graph_ms,
                         host_sync_ms_per_step=sync_ms, speedup_vs_host_sync=sync_ms / fused_ms,
                         host_syncs_per_step_graph=0, host_syncs_per_step_sync_arm=nl,
                         unique_experts_per_layer=mean_u, unique_expert_bytes_per_step=step_bytes,
                         router_bytes_per_step=router_bytes * nl,
                         hbm_GBps_unique_expert_bytes=gbs, hbm_frac=gbs / HBM_PEAK_GBS, timed_steps=reps))
        log("stack bs=%d  fused graph %.1f us/step  layer-call graph %.1f us/step  host-sync %.1f us/step  "
            "U/layer=%.2f  %.0f GB/s (%.1f%%)" % (T, fused_ms * 1e3, graph_ms * 1e3, sync_ms * 1e3, mean_u, gbs,
                                                100 * gbs / HBM_PEAK_GBS))
    del layers
    torch.cuda.empty_cache()
    return rows


# ---- the large-batch layer ----------------------------------------------------------

def spec_name(dtype):
    return {"fp8": "fp8 e4m3 (128x128 block scales)", "mxfp4": "MXFP4 (E2M1, E8M0 scale per 32)",
            "q4_0": "q4_0 (4-bit codes, binary16 scale per 32)"}.get(dtype, "bf16")


def large_rows(torch, moe, wl, dtype, sizes, steps, warmup, draws):
    """E=256, top_k=8, H=4096, I=1536 with Zipf(1.1)-skewed routing; experts
    holding moe_mfma_min_routes() routes or more run on MFMA.  Per batch size: steps/s, HBM GB/s on
    unique-expert bytes, MFMA TFLOP/s on the MFMA stages, and the roofline of
    the stage that dominates."""
    dev = torch.device("cuda:0")
    spec = {"fp8": wl.LARGE_FP8, "mxfp4": wl.LARGE_MXFP4, "q4_0": wl.LARGE_Q4_0}.get(dtype, wl.LARGE)
    # bytes per weight, scales included: fp8 1 (+ 4 per 128x128 block), MXFP4
    # half a byte plus one scale byte per 32, q4_0 two scale bytes per 32
    bpw = {wl.FP8: 1 + 4 / (128 * 128), wl.MXFP4: 17 / 32, wl.Q4_0: 18 / 32}.get(spec.expert_dtype, 2)
    H, I = spec.H, spec.I
    expert_bytes = 3 * H * I * bpw
    bias = wl.zipf_bias(spec.E)
    t0 = time.time()
    host = wl.make_layer(spec)
    layer = moe.DeviceLayer(host, bias, device=dev)
    del host
    log("large %s layer resident (%.1f s)" % (dtype, time.time() - t0))
    rows = {}
    for T in sizes:
        xs = [torch.from_numpy(wl.make_x(T, H, draw=d)).to(dev) for d in range(draws)]
        run = time_layer(torch, moe, [layer], xs, T, moe.MOE_WALK_DEDUP, steps, warmup)
        ms = run["ms"]
        st = run["stage_ms"]
        cs = [run["counts"][i] for i in run["stage_steps"]]
        u_ev = float(np.mean([(c > 0).sum() for c in cs]))
        thr = moe.moe_mfma_min_routes(layer.struct, T, 0)
        hot = moe.moe_mfma_hot_routes(layer.struct, T, 0)
        big = [c[c >= thr] if c.max() >= hot else c[:0] for c in cs]
        n_big = float(np.mean([len(b) for b in big]))
        routes_big = float(np.mean([b.sum() for b in big]))
        tiles_big = float(np.mean([(np.ceil(b / 16) * 16).sum() for b in big]))
        flops_useful = 2 * routes_big * 3 * H * I
        flops_issued = 2 * tiles_big * 3 * H * I
        mfma_ms = st["pass1_mfma"] + st["pass2_mfma"]
        mfma_tf = flops_useful / (mfma_ms * 1e-3) / 1e12 if mfma_ms > 0 else 0.0
        u = run["uniq_timed"]
        gbs = u * expert_bytes / (ms * 1e-3) / 1e9
        # algorithmic bytes of each stage: weights of the experts it streams
        # (GEMV: below the threshold thr, MFMA: thr or more)
        n_gemv = u_ev - n_big
        per_expert = {"pass1": 2 * I * H * bpw, "pass2": H * I * bpw}
        stage_bytes = {"pass1_gemv": n_gemv * per_expert["pass1"], "pass1_mfma": n_big * per_expert["pass1"],
                       "pass2_gemv": n_gemv * per_expert["pass2"], "pass2_mfma": n_big * per_expert["pass2"],
                       "routing": spec.E * H * 2, "combine": 0}
        dom = max(st, key=st.get)
        dom_gbs = stage_bytes[dom] / (st[dom] * 1e-3) / 1e9 if st[dom] > 0 else 0.0
        kernel_of = {"pass1_gemv": "pass1_kernel", "pass1_mfma": "mfma_wide_kernel (pass 1)",
                     "pass2_gemv": "pass2_kernel", "pass2_mfma": "mfma_wide_kernel (pass 2)",
                     "routing": "route_kernel", "combine": "combine_kernel"}
        rows[T] = dict(bs=T, ms_per_step=ms, steps_per_s=1e3 / ms, unique_experts=u, mfma_experts=n_big,
                       mfma_route_frac=routes_big / (T * spec.top_k), hbm_GBps=gbs, hbm_frac=gbs / HBM_PEAK_GBS,
                       stage_us={k: v * 1e3 for k, v in st.items()},
                       mfma={"achieved_TFLOPs": mfma_tf, "peak_TFLOPs": MFMA_PEAK_TFS,
                             "frac": mfma_tf / MFMA_PEAK_TFS, "issued_over_useful": flops_issued / max(flops_useful, 1),
                             "rule": "2 x MFMA routes x 3HI over the pass 1 + pass 2 MFMA stage times (in order)"},
                       roofline={"bound": "hbm", "kernel": kernel_of[dom], "stage": dom, "achieved": dom_gbs,
                                 "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": dom_gbs / HBM_PEAK_GBS,
                                 "avg_launch_us": st[dom] * 1e3, "bytes_per_launch": stage_bytes[dom]},
                       timed_steps=run["timed_steps"],
                       us_per_step_over_replays={k: v * 1e3 for k, v in run["spread_ms"].items()})
        log("large %s bs=%d  %.1f us/step  U=%.1f (MFMA %.1f, %.0f%% of routes)  %.0f GB/s (%.1f%%)  "
            "MFMA %.0f TF/s useful  stages(us) %s" %
            (dtype, T, ms * 1e3, u, n_big, 100 * routes_big / (T * spec.top_k), gbs, 100 * gbs / HBM_PEAK_GBS,
             mfma_tf, " ".join("%s=%.1f" % (k, v * 1e3) for k, v in st.items())))
        del xs
    del layer
    torch.cuda.empty_cache()
    return rows, spec


# ---- CPU oracle legs ---------------------------------------------------------------

def cpu_legs(wl, host_sweep, T_head, budget_s, extras):
    """The oracle as it stands, on the host cores: the headline leg (whole
    bs=T_head layer steps of the uniform sweep, for about budget_s seconds),
    and, with extras, the oracle's per-route walk over the tiny layer, the
    uniform sweep and the skewed sweep (median of 3, one repetition at 64
    tokens), its grouped walk at the small batches, and single-thread bs=1
    and bs=64 legs."""
    import oracle

    nth = cpu_threads()
    expert_bytes = 3 * wl.SWEEP.H * wl.SWEEP.I * 2
    ol = oracle.Layer(host_sweep, None)
    done, t_start = 0, time.time()
    while True:
        oracle.moe_layer(ol, wl.make_x(T_head, wl.SWEEP.H, draw=done), nthreads=nth)
        done += 1
        if time.time() - t_start >= budget_s:
            break
    el = time.time() - t_start
    res = dict(value=done / el, unit="steps/s", cores=nth, kind="oracle", cpu_model=cpu_model(),
               sample="%d whole layer steps at bs=%d of the uniform sweep layer (E=256, k=8, H=2048, I=768, "
                      "bf16), per-route walk, fp64 accumulation, %d threads, %.1f s" % (done, T_head, nth, el))
    log("cpu oracle: %.3f steps/s at bs=%d (%d threads, %s)" % (res["value"], T_head, nth, res["cpu_model"]))
    if not extras:
        return res
    legs = []

    def leg(name, layer, spec, T, kind, threads, reps, bias=None):
        times, uniq = [], 0
        for r in range(reps):
            x = wl.make_x(T, spec.H, draw=r)
            t = time.perf_counter()
            o = oracle.moe_layer(layer, x, kind=kind, nthreads=threads)
            times.append(time.perf_counter() - t)
            uniq = len(np.unique(o["ids"]))
        ms = float(np.median(times)) * 1e3
        eb = 3 * spec.H * spec.I * (4 if spec.expert_dtype == wl.F32 else 2)
        legs.append(dict(workload=name, bs=T, walk="grouped" if kind == oracle.WALK_GROUPED else "per_route",
                         threads=threads, reps=reps, ms_per_step=ms, unique_experts_last=uniq,
                         GBps_unique_expert_bytes=uniq * eb / (ms * 1e-3) / 1e9))

    P, G = oracle.WALK_PER_ROUTE, oracle.WALK_GROUPED
    tiny_w = wl.make_layer(wl.TINY)
    for kind in (P, G):
        leg("tiny", oracle.Layer(tiny_w, None), wl.TINY, 4, kind, nth, 3)
        leg("tiny forced collision", oracle.Layer(tiny_w, wl.collision_bias(wl.TINY.E)), wl.TINY, 4, kind, nth, 3)
    # the per-route walk is threaded over routes; the grouped walk runs on one
    # thread (its loop nest is the definition's, reordered), so it is sampled
    # at the small batches only
    for T in wl.SWEEP_BS:
        leg("uniform sweep", ol, wl.SWEEP, T, P, nth, 3 if T < 64 else 1)
    for T in (1, 4, 8):
        leg("uniform sweep", ol, wl.SWEEP, T, G, nth, 1)
    skew_w = dict(host_sweep)
    skew_w["spec"] = wl.SKEWED
    sl = oracle.Layer(skew_w, wl.zipf_bias(wl.SKEWED.E))
    for T in wl.SKEWED_BS:
        leg("skewed", sl, wl.SKEWED, T, P, nth, 3 if T < 64 else 1)
    for T in (1, 8):
        leg("skewed", sl, wl.SKEWED, T, G, nth, 1)
    for T in (1, 64):
        leg("uniform sweep", ol, wl.SWEEP, T, P, 1, 1)
    res["legs"] = legs
    log("cpu oracle legs: %d (%.1f s in all)" % (len(legs), sum(l["ms_per_step"] * l["reps"] for l in legs) / 1e3))
    return res


# ---- main ---------------------------------------------------------------------------

def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the layer is built and timed on a single MI355X; "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)
        return

    import torch

    import mixture_experts_decode_gemv_amd as moe
    import workload as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.workload == "stack":
        rows = stack_rows(torch, moe, wl, max(5, args.steps // 10))
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
        return
    if args.workload == "large":
        sizes = [int(s) for s in args.sweep.split(",")] if args.sweep != "1,4,8,16,32,64" else list(wl.LARGE_BS)
        rows, spec = large_rows(torch, moe, wl, args.dtype, sizes, args.steps, args.warmup, args.draws)
        bs_head = args.bs if args.bs in sizes else max(sizes)
        head = rows[bs_head]
        print(json.dumps({
            "metric": "MoE layer steps/s at bs=%d (Zipf(1.1) routing, E=256, top_k=8, H=4096, I=1536, %s); "
                      "achieved HBM GB/s on unique-expert bytes; MFMA TFLOP/s" % (bs_head, spec_name(args.dtype)),
            "value": head["steps_per_s"], "unit": "steps/s", "n_gpus": 1, "steps": head["timed_steps"],
            "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None,
            "dtype": {"fp8": "fp8_e4m3 weights, bf16 MFMA operands",
                      "mxfp4": "mxfp4 weights, bf16 MFMA operands",
                      "q4_0": "q4_0 weights, bf16 MFMA operands"}.get(args.dtype, "bf16"),
            "data": "synthetic (seeded)",
            "config": {"workload": "large-batch single MoE layer, Zipf(1.1) routing, E=256 top_k=8 H=4096 I=1536 "
                                   "%s experts, MFMA for experts with >= 4 routes (moe_mfma_min_routes at 128+ tokens)" % spec_name(args.dtype),
                       "bs": bs_head, "draws": args.draws},
            "hbm_GBps_unique_expert_bytes": head["hbm_GBps"], "sweep": [rows[t] for t in sizes],
            "roofline": dict(head["roofline"], traffic=None), "mfma": head["mfma"], "cpu_baseline": None}),
            flush=True)
        return

    skewed = args.workload == "skewed"
    if args.dtype not in ("bf16", "mxfp4", "q4_0"):
        print("bench.py: the %s workload takes bf16, mxfp4 or q4_0 experts" % args.workload, file=sys.stderr)
        sys.exit(2)
    mx = args.dtype != "bf16"  # a 4-bit format
    base = wl.SKEWED if skewed else wl.SWEEP
    qdt = {"mxfp4": wl.MXFP4, "q4_0": wl.Q4_0}.get(args.dtype)
    spec = base if not mx else wl.LayerSpec(E=base.E, top_k=base.top_k, H=base.H, I=base.I, expert_dtype=qdt,
                                            router_dtype=base.router_dtype)
    wname = {"mxfp4": "MXFP4 (E2M1, E8M0 scale per 32)", "q4_0": "q4_0 (4-bit codes, binary16 scale per 32)"}.get(
        args.dtype, "bf16")
    bias = wl.zipf_bias(spec.E) if skewed else None
    walk = {"dedup": moe.MOE_WALK_DEDUP, "per_route": moe.MOE_WALK_PER_ROUTE,
            "dedup_pass1": moe.MOE_WALK_DEDUP_PASS1}[args.walk]
    flags = walk | (moe.MOE_NO_MFMA if args.no_mfma else 0)
    # bytes per weight: MXFP4 half a byte plus one scale byte per 32, q4_0 two scale bytes per 32
    bpw = {"mxfp4": 17 / 32, "q4_0": 18 / 32}.get(args.dtype, 2)
    expert_bytes = 3 * spec.H * spec.I * bpw

    t0 = time.time()
    layers, host0 = [], None
    for l in range(args.layers):
        w = wl.make_layer(spec, layer=l)
        layers.append(moe.DeviceLayer(w, bias, device=dev))
        if l == 0:
            host0 = w
        del w
    log("%d layers generated and resident (%.1f s)" % (args.layers, time.time() - t0))

    sweep = args.sweep
    if skewed and sweep == "1,4,8,16,32,64":
        sweep = ",".join(str(t) for t in wl.SKEWED_BS)
    sizes = sorted(set([args.bs] + [int(s) for s in sweep.split(",") if s]))
    rows, runs = sweep_rows(torch, moe, wl, layers, spec, sizes, flags, args.steps, args.warmup, args.draws,
                            expert_bytes, graph=not args.no_graph)
    head_run = runs[args.bs]
    p1_gbs, p1_ms, p1_bytes = stage_roofline(head_run, spec, args.bs, bpw,
                                             moe.moe_mfma_min_routes(layers[0].struct, args.bs, flags),
                                             moe.moe_mfma_hot_routes(layers[0].struct, args.bs, flags))

    # measured HBM bytes per pass-1 launch (headline configuration only, and
    # only for the kernel source the counters were taken on)
    traffic = None
    if (not skewed and not mx and args.bs == 64 and args.walk == "dedup" and not args.no_mfma
            and pass1_source_fingerprint() == PASS1_TRAFFIC_BS64["source"]):
        traffic = PASS1_TRAFFIC_BS64["read_bytes"] + PASS1_TRAFFIC_BS64["write_bytes"]

    extras = args.workload == "sweep" and not args.no_extras and not mx and args.walk == "dedup" and \
        not args.no_mfma and not args.no_graph
    xsteps = min(args.steps, 64)  # timed steps of the extra arms and workloads
    extra = {}
    if extras:
        extra["arms_uniform"] = walk_arms(torch, moe, wl, layers, spec, sizes, xsteps, args.warmup, args.draws,
                                          expert_bytes, "uniform")
        skl = [L.with_bias(wl.zipf_bias(wl.SKEWED.E), top_k=wl.SKEWED.top_k) for L in layers]
        sk_rows, _ = sweep_rows(torch, moe, wl, skl, wl.SKEWED, list(wl.SKEWED_BS), moe.MOE_WALK_DEDUP, xsteps,
                                args.warmup, args.draws, expert_bytes, label="skewed bs")
        extra["skewed"] = {"workload": "single MoE layer, Zipf(1.1) routing, E=256 top_k=6 H=2048 I=768 bf16",
                           "sweep": [sk_rows[t] for t in wl.SKEWED_BS]}
        extra["arms_skewed"] = walk_arms(torch, moe, wl, skl, wl.SKEWED, list(wl.SKEWED_BS), xsteps, args.warmup,
                                         args.draws, expert_bytes, "skewed")
        del skl
        del layers
        torch.cuda.empty_cache()
        extra["stack"] = {"workload": "30-layer stack, E=128 top_k=2 H=2048 I=1024 bf16, RMSNorm + residual, "
                                      "distinct weights per layer",
                          "rows": stack_rows(torch, moe, wl, 20)}
        large = {}
        for dt in ("bf16", "fp8"):
            r, _ = large_rows(torch, moe, wl, dt, [128], min(xsteps, 32), args.warmup, 4)
            large[dt] = r[128]
        extra["large"] = {"workload": "single MoE layer, Zipf(1.1) routing, E=256 top_k=8 H=4096 I=1536, MFMA for "
                                      "experts with >= 4 routes (fp8: W8A16 with 128x128 block scales)",
                          "bs128": large}
        extra["read_stream_probe"] = read_stream_probe(torch)
    else:
        del layers

    cpu = None
    if not args.no_cpu:
        cpu = cpu_legs(wl, host0 if not skewed and not mx else wl.make_layer(wl.SWEEP), args.bs,
                       args.cpu_seconds, extras)

    head = rows[args.bs]
    probe = extra.get("read_stream_probe")
    line = {
        "metric": "MoE layer steps/s at bs=%d (%s routing, E=256, top_k=%d, H=2048, I=768, %s); "
                  "achieved HBM GB/s on unique-expert bytes" % (args.bs, "Zipf(1.1)" if skewed else "uniform",
                                                              spec.top_k, args.dtype),
        "value": head["steps_per_s"],
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": head["timed_steps"],
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic (seeded N(0, 1/sqrt(fan_in)) weights, N(0,1) activations)",
        "config": {"workload": "single MoE layer, %s routing, E=256 top_k=%d H=2048 I=768 %s experts, batch "
                               "sweep" % ("Zipf(1.1)" if skewed else "uniform", spec.top_k, wname), "bs": args.bs,
                   "walk": args.walk, "mfma": not args.no_mfma, "resident_layers": args.layers,
                   "draws": args.draws, "graph": not args.no_graph, "parallelism": "none (1 GPU)"},
        "hbm_GBps_unique_expert_bytes": head["hbm_GBps"],
        "hbm_frac_of_read_stream_probe": head["hbm_GBps"] / probe["GBps"] if probe else None,
        "sweep": [rows[t] for t in sizes],
        "roofline": {"bound": "hbm", "kernel": "pass1_kernel (grouped GEMV, gate_up rows x routes)",
                     "achieved": p1_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": p1_gbs / HBM_PEAK_GBS,
                     "traffic": traffic, "avg_launch_us": p1_ms * 1e3, "bytes_per_launch": p1_bytes,
                     "frac_of_read_stream_probe": p1_gbs / probe["GBps"] if probe else None,
                     "bytes_rule": "unique experts on the GEMV path x 2I x H x %s (gate_up, %s)" %
                                   ({"mxfp4": "17/32 B (codes and E8M0 scales)",
                                     "q4_0": "18/32 B (codes and binary16 scales)"}.get(args.dtype, "2 B"),
                                    args.dtype)},
        "cpu_baseline": cpu,
    }
    line.update(extra)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
