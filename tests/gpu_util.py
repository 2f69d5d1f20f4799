"""Helpers of the GPU parity tests: run the C-ABI entry points on torch
device memory and compare with the CPU oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import mixture_experts_decode_gemv_amd as moe
import oracle
import workload as wl


def dev():
    return torch.device("cuda:0")


def stream():
    return torch.cuda.current_stream(dev())


def note(msg):
    """Name the case before a GPU step, flushed, so a crash log shows it."""
    sys.stdout.write("[gpu case] %s\n" % msg)
    sys.stdout.flush()


def to_dev(a, dtype=None):
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a)
    if dtype is not None:
        t = t.to(dtype)
    return t.to(dev())


def max_rel(got, ref):
    """max |got - ref| / max |ref| over the tensor (0 if ref is all zero and got matches)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max() if ref.size else 0.0
    num = np.abs(got - ref).max() if ref.size else 0.0
    if den == 0.0:
        return num
    return num / den


def gpu_route(layer: moe.DeviceLayer, x=None, logits_in=None, T=None):
    s = layer.spec
    T = T if T is not None else (x.shape[0] if x is not None else logits_in.shape[0])
    ids = torch.full((T, s.top_k), -7, dtype=torch.int32, device=dev())
    w = torch.full((T, s.top_k), -7.0, dtype=torch.float32, device=dev())
    lo = torch.full((T, s.E), -7.0, dtype=torch.float32, device=dev())
    xd = None if x is None else to_dev(x)
    li = None if logits_in is None else to_dev(logits_in)
    ws = layer.workspace(T)
    moe.moe_route(layer.struct, xd, li, T, lo, ids, w, ws, ws.numel(), stream())
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy(), lo.cpu().numpy()


def gpu_sort(ids: np.ndarray, E: int):
    T, k = ids.shape
    R = T * k
    d_ids = to_dev(ids.astype(np.int32))
    counts = torch.full((E,), -7, dtype=torch.int32, device=dev())
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device=dev())
    sorted_routes = torch.full((max(R, 1),), -7, dtype=torch.int32, device=dev())
    uniq = torch.full((E,), -7, dtype=torch.int32, device=dev())
    n = torch.full((1,), -7, dtype=torch.int32, device=dev())
    moe.moe_sort(d_ids, T, k, E, counts, offsets, sorted_routes, uniq, n, stream())
    torch.cuda.synchronize()
    nu = int(n.item())
    return dict(counts=counts.cpu().numpy(), offsets=offsets.cpu().numpy(),
                sorted_routes=sorted_routes.cpu().numpy()[:R], uniq=uniq.cpu().numpy()[:max(nu, 0)], n_uniq=nu)


def gpu_expert_fwd(layer: moe.DeviceLayer, x, ids, w, flags=0):
    """Experts + combine for a given routing (sorted on the GPU)."""
    s = layer.spec
    T = x.shape[0]
    R = T * s.top_k
    d_ids = to_dev(ids.astype(np.int32))
    d_w = to_dev(w.astype(np.float32))
    counts = torch.empty(s.E, dtype=torch.int32, device=dev())
    offsets = torch.empty(s.E + 1, dtype=torch.int32, device=dev())
    sorted_routes = torch.empty(max(R, 1), dtype=torch.int32, device=dev())
    uniq = torch.empty(s.E, dtype=torch.int32, device=dev())
    n = torch.empty(1, dtype=torch.int32, device=dev())
    moe.moe_sort(d_ids, T, s.top_k, s.E, counts, offsets, sorted_routes, uniq, n, stream())
    xd = to_dev(x.astype(np.float32))
    out = torch.full((T, s.H), float("nan"), dtype=torch.float32, device=dev())
    ws = layer.workspace(T)
    moe.moe_expert_fwd(layer.struct, xd, T, d_ids, d_w, counts, offsets, sorted_routes, uniq, n, out, flags, ws,
                       ws.numel(), stream())
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _ws_slice(ws, addr, n, dtype):
    off = addr - ws.data_ptr()
    nbytes = n * 4
    assert 0 <= off and off + nbytes <= ws.numel()
    return ws[off:off + nbytes].view(dtype).cpu().numpy()


def gpu_layer_fwd(layer: moe.DeviceLayer, x, flags=0, full=False):
    """moe_layer_fwd; with full=True also the routing it left in the workspace."""
    s = layer.spec
    T = x.shape[0]
    xd = to_dev(x.astype(np.float32))
    out = torch.full_like(xd, float("nan"))
    ws = layer.workspace(T)
    moe.moe_layer_fwd(layer.struct, xd, T, out, flags, ws, ws.numel(), stream())
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    if not full:
        return o
    r = moe.moe_layer_routing(layer.struct, T, ws, ws.numel())
    R = T * s.top_k
    res = dict(out=o, stats=ws[:16].view(torch.int32).cpu().numpy())
    res["ids"] = _ws_slice(ws, r["topk_ids"], R, torch.int32).reshape(T, s.top_k)
    res["w"] = _ws_slice(ws, r["topk_w"], R, torch.float32).reshape(T, s.top_k)
    res["counts"] = _ws_slice(ws, r["counts"], s.E, torch.int32)
    res["offsets"] = _ws_slice(ws, r["offsets"], s.E + 1, torch.int32)
    res["sorted_routes"] = _ws_slice(ws, r["sorted_routes"], R, torch.int32)
    res["n_uniq"] = int(_ws_slice(ws, r["n_uniq"], 1, torch.int32)[0])
    res["uniq"] = _ws_slice(ws, r["uniq"], s.E, torch.int32)[:res["n_uniq"]]
    return res


BF16_OPERAND_TOL = 2e-2  # bar for paths with bf16 operands: max abs error over max |ref|


def call_tol(layer: moe.DeviceLayer, x, flags=0, gemv_tol=1e-4):
    """The bar for one moe_layer_fwd call: the bf16-operand bar when some
    segment of it runs on the matrix cores (its largest expert holds
    moe_mfma_hot_routes() routes or more, which is at least
    moe_mfma_min_routes()), else the GEMV path's gemv_tol."""
    hot = moe.moe_mfma_hot_routes(layer.struct, x.shape[0], flags)
    if hot <= 0:
        return gemv_tol
    return BF16_OPERAND_TOL if gpu_layer_fwd(layer, x, flags, full=True)["counts"].max() >= hot else gemv_tol


def oracle_for_gpu_selection(olayer: oracle.Layer, x, oracle_logits, gpu_ids, rmsnorm_in=False, residual=False):
    """Oracle output when the routing is the GPU's ids: weights are the
    softmax of the oracle's logits over the GPU-chosen experts."""
    lg = np.take_along_axis(oracle_logits, gpu_ids.astype(np.int64), axis=1)
    w = np.exp(lg - lg.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    xin = oracle.rmsnorm(x) if rmsnorm_in else x.astype(np.float64)
    out = oracle.expert_fwd(olayer, xin, gpu_ids, w)
    if residual:
        out = out + x.astype(np.float64)
    return out


def ambiguous_tokens(oracle_logits, k, rel=1e-4):
    """Tokens with two of their k+1 largest oracle logits closer than
    rel * max|logit|: fp32 rounding may legitimately pick or order either."""
    T, E = oracle_logits.shape
    srt = -np.sort(-oracle_logits, axis=1)[:, :min(k + 1, E)]
    if srt.shape[1] < 2:
        return np.zeros(T, bool)
    gap = (srt[:, :-1] - srt[:, 1:]).min(axis=1)
    return gap < rel * np.abs(oracle_logits).max()


def check_layer_against_oracle(layer, olayer, x, flags=0, tol=1e-4, rmsnorm_in=False, residual=False):
    """GPU moe_layer_fwd vs the oracle.  The GPU's own selection must equal the
    oracle's except on near-tie tokens, which are compared against the oracle
    rerun with the GPU's ids.  Returns (max rel err, #tokens routed apart)."""
    g = gpu_layer_fwd(layer, x, flags, full=True)
    ref = oracle.moe_layer(olayer, x, rmsnorm_in=rmsnorm_in, residual=residual)
    amb = ambiguous_tokens(ref["logits"], layer.spec.top_k)
    same = (g["ids"] == ref["ids"]).all(1)
    assert (same | amb).all(), "selection differs on tokens with a clear gap: %s" % np.where(~(same | amb))[0]
    expect = ref["out"].copy()
    if (~same).any():
        alt = oracle_for_gpu_selection(olayer, x, ref["logits"], g["ids"], rmsnorm_in, residual)
        expect[~same] = alt[~same]
    assert np.isfinite(g["out"]).all()
    err = max_rel(g["out"], expect)
    assert err <= tol, "max rel err %g > %g" % (err, tol)
    return err, int((~same).sum())


def make_device_layer(spec: wl.LayerSpec, bias=None, layer_idx=0):
    w = wl.make_layer(spec, layer=layer_idx)
    return w, moe.DeviceLayer(w, bias, device=dev()), oracle.Layer(w, bias)


def oracle_weights_for(oracle_logits, ids):
    """Combine weights of the given expert ids: softmax of the oracle's logits
    over those experts."""
    lg = np.take_along_axis(oracle_logits, ids.astype(np.int64), axis=1)
    w = np.exp(lg - lg.max(axis=1, keepdims=True))
    return w / w.sum(axis=1, keepdims=True)


def check_layer_sampled(layer, olayer, x, sample, flags=0, tol=2e-2):
    """moe_layer_fwd at a size the oracle cannot finish whole: routing of
    every token against the oracle (ids bit-exact except near-ties, the sort
    bit-exact on the GPU's ids), outputs on the sampled tokens only.
    Returns (max rel err on the sample, GPU result dict)."""
    s = layer.spec
    g = gpu_layer_fwd(layer, x, flags, full=True)
    logits = oracle.router_logits(olayer, x)
    ids_ref, _ = oracle.select(logits, s.top_k)
    amb = ambiguous_tokens(logits, s.top_k)
    same = (g["ids"] == ids_ref).all(1)
    assert (same | amb).all(), "selection differs on tokens with a clear gap: %s" % np.where(~(same | amb))[0]
    r = oracle.sort(g["ids"], s.E)
    for key in ("counts", "offsets", "sorted_routes", "uniq"):
        assert np.array_equal(g[key], r[key]), key
    sample = np.asarray(sample)
    ids_s = g["ids"][sample]
    ref = oracle.expert_fwd(olayer, x[sample], ids_s, oracle_weights_for(logits[sample], ids_s))
    got = g["out"][sample]
    assert np.isfinite(g["out"]).all()
    err = max_rel(got, ref)
    assert err <= tol, "max rel err %g > %g on the sampled tokens" % (err, tol)
    return err, g
