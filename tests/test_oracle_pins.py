"""Pins of the CPU oracle to things other than itself.

Each test checks the oracle against brute force, a closed form, a library
routine on a special case, a value the pages print, or an invariant that the
mathematics fixes.  None of them retypes the oracle's own formula.
"""
import itertools
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import workload as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#") or line[0].isalpha():
                continue
            rows.append([float(v) for v in line.split()])
    return rows


def _spec(E, k, H, I, ed=wl.F32, rd=wl.F32):
    return wl.LayerSpec(E=E, top_k=k, H=H, I=I, expert_dtype=ed, router_dtype=rd)


def _f32_layer(E, k, H, I, gate_up, down, w_router=None, bias=None):
    w = dict(spec=_spec(E, k, H, I), w_gate_up=np.asarray(gate_up, np.float32),
             w_down=np.asarray(down, np.float32),
             w_router=np.zeros((E, H), np.float32) if w_router is None else np.asarray(w_router, np.float32))
    return oracle.Layer(w, bias)


def _torch_swiglu(x, gu, d):
    """Textbook SwiGLU FFN (library ops, float64): down(silu(gate x) * up x)."""
    x = torch.as_tensor(x, dtype=torch.float64)
    gu = torch.as_tensor(gu, dtype=torch.float64)
    d = torch.as_tensor(d, dtype=torch.float64)
    I = gu.shape[0] // 2
    g = torch.nn.functional.linear(x, gu[:I])
    u = torch.nn.functional.linear(x, gu[I:])
    return torch.nn.functional.linear(torch.nn.functional.silu(g) * u, d).numpy()


# ---------------------------------------------------------------- decoders --

def test_e4m3_decode_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(got[~nan], ref[~nan])
    assert oracle.e4m3_value(0x7E) == 448.0
    assert oracle.e4m3_value(0x08) == 2.0 ** -6
    assert oracle.e4m3_value(0x01) == 2.0 ** -9
    assert oracle.e4m3_value(0xFE) == -448.0


def test_bf16_decode_all_patterns_match_torch():
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_value(int(b)) for b in bits[::7]])
    r = ref[::7]
    nan = np.isnan(r)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], r[~nan])


# --------------------------------------------------------------- selection --

def _brute_topk(l, k):
    """All C(E, k) subsets; the answer is the one whose members beat every
    non-member under (logit descending, index ascending)."""
    E = len(l)

    def beats(a, b):
        return l[a] > l[b] or (l[a] == l[b] and a < b)

    winners = [s for s in itertools.combinations(range(E), k)
               if all(beats(a, b) for a in s for b in range(E) if b not in s)]
    assert len(winners) == 1
    s = list(winners[0])
    # slot order: the same total order
    s.sort(key=lambda e: (-l[e], e))
    return s


@pytest.mark.parametrize("mode", ["normal", "quarter", "equal", "zeros"])
def test_select_matches_brute_force(mode):
    rng = np.random.default_rng(7)
    E, T = 8, 40
    lg = rng.standard_normal((T, E))
    if mode == "quarter":
        lg = np.round(lg * 4) / 4  # many exact ties
    elif mode == "equal":
        lg = np.full((T, E), 0.5)
    elif mode == "zeros":
        lg = np.where(rng.random((T, E)) < 0.5, 0.0, -0.0)  # -0 == +0
    for k in (1, 2, 3, 8):
        ids, _ = oracle.select(lg, k)
        for t in range(T):
            assert list(ids[t]) == _brute_topk(lg[t], k), (mode, k, t)
    if mode in ("equal", "zeros"):
        ids, _ = oracle.select(lg, 3)
        assert (ids == np.array([0, 1, 2])).all()


def test_select_weights_are_softmax_over_selected():
    """Softmax over all E renormalised over the top k equals a softmax over the
    k selected logits alone (scipy), and sums to 1."""
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((50, 16)) * 3
    for k in (1, 2, 5, 16):
        ids, w = oracle.select(lg, k)
        sel = np.take_along_axis(lg, ids, axis=1)
        ref = scipy.special.softmax(sel, axis=1)
        assert np.allclose(w, ref, rtol=1e-13, atol=1e-15)
        assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-13)
        if k == 1:
            assert (w == 1.0).all()
        if k == 16:  # k = E: the dense softmax over all experts
            dense = scipy.special.softmax(lg, axis=1)
            assert np.allclose(np.take_along_axis(dense, ids, axis=1), w, rtol=1e-13, atol=1e-15)


def test_forced_collision_bias():
    """+64 on experts {0, 1}: every token picks them; the common bias cancels,
    so the weights are the 2-way logistic of the natural logits."""
    spec = wl.TINY
    w = wl.make_layer(spec)
    x = wl.make_x(4, spec.H)
    natural = oracle.router_logits(oracle.Layer(w), x)
    res = oracle.moe_layer(oracle.Layer(w, wl.collision_bias(spec.E)), x)
    assert set(np.unique(res["ids"])) == {0, 1}
    for t in range(4):
        a, b = res["ids"][t]
        assert natural[t, a] > natural[t, b] or (natural[t, a] == natural[t, b] and a < b)
        assert res["w"][t, 0] == pytest.approx(scipy.special.expit(natural[t, a] - natural[t, b]), abs=1e-12)


# -------------------------------------------------------------------- sort --

@pytest.mark.parametrize("T,k,E", [(1, 1, 1), (4, 2, 8), (64, 8, 256), (37, 6, 100), (5, 3, 3), (0, 2, 8)])
def test_sort_matches_library(T, k, E):
    rng = np.random.default_rng(T * 1000 + k * 10 + E)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]) if T else np.zeros((0, k), np.int32)
    s = oracle.sort(ids, E)
    flat = ids.reshape(-1)
    assert np.array_equal(s["counts"], np.bincount(flat, minlength=E))
    assert np.array_equal(s["offsets"], np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    assert np.array_equal(s["sorted_routes"], np.argsort(flat, kind="stable"))
    assert np.array_equal(s["uniq"], np.unique(flat))
    assert s["n_uniq"] == len(np.unique(flat))
    assert s["offsets"][E] == T * k


def test_unique_counts_match_printed_uniform_sweep():
    """The pages print one uniform-routing draw per batch size (E=256, k=8).
    The oracle's selection + sort over i.i.d. N(0,1) logits must give the
    expected count E(1 - (1 - k/E)^T) on average, and each printed count must
    sit inside the spread of the oracle's draws."""
    E, k = 256, 8
    rows = _read_golden("uniform_unique_experts.txt")
    for bs, routes, printed_unique, reuse in rows:
        bs = int(bs)
        assert routes == bs * k
        assert reuse == pytest.approx(routes / printed_unique, abs=0.006)
        us = []
        for d in range(300):
            lg = wl.make_logits(bs, E, draw=1000 + d)
            ids, _ = oracle.select(lg, k)
            us.append(oracle.sort(ids, E)["n_uniq"])
        us = np.array(us, dtype=np.float64)
        expect = E * (1 - (1 - k / E) ** bs)
        sem = us.std(ddof=1) / math.sqrt(len(us))
        assert abs(us.mean() - expect) < 4 * sem + 1e-9, (bs, us.mean(), expect)
        lo, hi = np.percentile(us, [0.5, 99.5])
        assert lo <= printed_unique <= hi, (bs, printed_unique, lo, hi)


# ------------------------------------------------------------ router, norm --

def test_router_logits_match_library_matmul():
    spec = _spec(6, 2, 33, 4)
    rng = np.random.default_rng(11)
    w = dict(spec=spec, w_router=rng.standard_normal((6, 33)).astype(np.float32),
             w_gate_up=np.zeros((6, 8, 33), np.float32), w_down=np.zeros((6, 33, 4), np.float32))
    bias = rng.standard_normal(6).astype(np.float32)
    x = rng.standard_normal((5, 33))
    got = oracle.router_logits(oracle.Layer(w, bias), x)
    ref = x @ w["w_router"].astype(np.float64).T + bias.astype(np.float64)
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-13)


def test_router_bf16_decodes_exactly():
    spec = wl.LayerSpec(E=8, top_k=2, H=64, I=32, expert_dtype=wl.BF16, router_dtype=wl.BF16)
    w = wl.make_layer(spec)
    x = wl.make_x(3, 64)
    got = oracle.router_logits(oracle.Layer(w), x)
    wr = torch.from_numpy(w["w_router"].view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.allclose(got, x.astype(np.float64) @ wr.T, rtol=1e-13, atol=1e-13)


def test_rmsnorm_matches_torch():
    x = np.random.default_rng(5).standard_normal((4, 2048)) * 3
    got = oracle.rmsnorm(x, 1e-6)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (2048,), eps=1e-6).numpy()
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------ expert math --

def test_closed_form_one_dimensional_expert():
    (xv, g, u, d, out), = _read_golden("swiglu_closed_form.txt")
    L = _f32_layer(1, 1, 1, 1, [[[g], [u]]], [[[d]]])
    res = oracle.moe_layer(L, np.array([[xv]], np.float32))
    assert res["w"][0, 0] == 1.0
    assert res["out"][0, 0] == pytest.approx(out, rel=1e-15)


def test_single_expert_is_textbook_swiglu():
    """E = 1, k = 1 reduces to one SwiGLU FFN (torch linear + silu)."""
    rng = np.random.default_rng(2)
    H, I = 24, 10
    gu = rng.standard_normal((1, 2 * I, H)).astype(np.float32)
    d = rng.standard_normal((1, H, I)).astype(np.float32)
    x = rng.standard_normal((7, H)).astype(np.float32)
    L = _f32_layer(1, 1, H, I, gu, d)
    got = oracle.moe_layer(L, x)["out"]
    ref = _torch_swiglu(x, gu[0], d[0])
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_permutation_experts_closed_form():
    """Experts built from permutation matrices have an elementwise closed form.
    gate rows = c_e * P_e, up rows = Q_e, down = d_e * S_e with
    P[i, p(i)] = 1 etc., so out[t, h] = sum_j w_tj d_e silu(c_e x[p(s(h))]) x[q(s(h))].
    A transposed operand (p^-1 for p), a swapped gate/up split or a wrong
    expert index changes the result."""
    rng = np.random.default_rng(9)
    E, k, n, T = 5, 2, 7, 6
    perms = {}
    gu = np.zeros((E, 2 * n, n), np.float32)
    dn = np.zeros((E, n, n), np.float32)
    c = np.array([0.5, 1.5, -1.0, 2.0, 0.75])
    d = np.array([1.0, -2.0, 0.5, 3.0, -0.25])
    for e in range(E):
        p, q, s = rng.permutation(n), rng.permutation(n), rng.permutation(n)
        perms[e] = (p, q, s)
        gu[e, np.arange(n), p] = c[e]
        gu[e, n + np.arange(n), q] = 1.0
        dn[e, np.arange(n), s] = d[e]
    wr = rng.standard_normal((E, n)).astype(np.float32)
    L = _f32_layer(E, k, n, n, gu, dn, w_router=wr)
    x = rng.standard_normal((T, n)).astype(np.float32)
    res = oracle.moe_layer(L, x)
    silu = lambda z: z / (1 + math.exp(-z))
    for t in range(T):
        for h in range(n):
            ref = 0.0
            for j in range(k):
                e = res["ids"][t, j]
                p, q, s = perms[e]
                i = s[h]
                ref += res["w"][t, j] * d[e] * silu(c[e] * float(x[t, p[i]])) * float(x[t, q[i]])
            assert res["out"][t, h] == pytest.approx(ref, rel=1e-13, abs=1e-14)


def test_dense_mixture_brute_force_tiny():
    """Brute force over all E experts (torch SwiGLU each) weighted by the
    selection (0 for experts not selected) equals the sparse layer."""
    spec = wl.TINY
    w = wl.make_layer(spec)
    x = wl.make_x(4, spec.H)
    for bias in (None, wl.collision_bias(spec.E)):
        res = oracle.moe_layer(oracle.Layer(w, bias), x)
        ref = np.zeros((4, spec.H))
        for e in range(spec.E):
            ffn = _torch_swiglu(x, w["w_gate_up"][e], w["w_down"][e])
            gate = np.zeros(4)
            for t in range(4):
                for j in range(spec.top_k):
                    if res["ids"][t, j] == e:
                        gate[t] = res["w"][t, j]
            ref += gate[:, None] * ffn
        assert np.allclose(res["out"], ref, rtol=1e-12, atol=1e-12)


def test_k_equals_E_is_dense_softmax_mixture():
    spec = _spec(4, 4, 16, 8)
    rng = np.random.default_rng(4)
    w = dict(spec=spec, w_router=rng.standard_normal((4, 16)).astype(np.float32),
             w_gate_up=rng.standard_normal((4, 16, 16)).astype(np.float32),
             w_down=rng.standard_normal((4, 16, 8)).astype(np.float32))
    x = rng.standard_normal((3, 16)).astype(np.float32)
    res = oracle.moe_layer(oracle.Layer(w), x)
    p = scipy.special.softmax(x.astype(np.float64) @ w["w_router"].astype(np.float64).T, axis=1)
    ref = sum(p[:, e:e + 1] * _torch_swiglu(x, w["w_gate_up"][e], w["w_down"][e]) for e in range(4))
    assert np.allclose(res["out"], ref, rtol=1e-12, atol=1e-12)


def test_identical_experts_ignore_routing():
    rng = np.random.default_rng(6)
    E, H, I = 6, 12, 5
    gu1 = rng.standard_normal((2 * I, H)).astype(np.float32)
    d1 = rng.standard_normal((H, I)).astype(np.float32)
    L = _f32_layer(E, 3, H, I, np.stack([gu1] * E), np.stack([d1] * E),
                   w_router=rng.standard_normal((E, H)).astype(np.float32))
    x = rng.standard_normal((5, H)).astype(np.float32)
    got = oracle.moe_layer(L, x)["out"]
    assert np.allclose(got, _torch_swiglu(x, gu1, d1), rtol=1e-12, atol=1e-12)


def test_fp8_expert_matches_library_decode():
    """fp8 e4m3 experts with 128x128 block scales: decode with torch's
    float8_e4m3fn, scale per block, run the textbook SwiGLU."""
    spec = wl.LayerSpec(E=2, top_k=1, H=128, I=128, expert_dtype=wl.FP8, router_dtype=wl.BF16)
    w = wl.make_layer(spec)
    x = wl.make_x(3, 128)
    L = oracle.Layer(w)
    ids = np.array([[1], [0], [1]], np.int32)
    got = oracle.expert_fwd(L, x, ids, np.ones((3, 1)))

    def dec(q, s):
        v = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        return v * np.kron(s.astype(np.float64), np.ones((128, 128)))

    for t in range(3):
        e = ids[t, 0]
        ref = _torch_swiglu(x[t:t + 1], dec(w["w_gate_up"][e], w["s_gate_up"][e]), dec(w["w_down"][e], w["s_down"][e]))
        assert np.allclose(got[t], ref[0], rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------- invariants --

@pytest.mark.parametrize("bias", [None, "collision", "zipf"])
def test_grouped_walk_equals_per_route_walk_bitwise(bias):
    spec = wl.TINY
    w = wl.make_layer(spec)
    b = {None: None, "collision": wl.collision_bias(spec.E), "zipf": wl.zipf_bias(spec.E)}[bias]
    L = oracle.Layer(w, b)
    x = wl.make_x(16, spec.H, draw=3)
    ids, _ = oracle.select(oracle.router_logits(L, x), spec.top_k)
    y0 = oracle.walk(L, x, ids, oracle.WALK_PER_ROUTE, nthreads=3)
    y1 = oracle.walk(L, x, ids, oracle.WALK_GROUPED)
    assert np.array_equal(y0, y1)
    a = oracle.moe_layer(L, x, kind=oracle.WALK_PER_ROUTE)["out"]
    b2 = oracle.moe_layer(L, x, kind=oracle.WALK_GROUPED)["out"]
    assert np.array_equal(a, b2)


def test_token_permutation_permutes_rows_bitwise():
    spec = wl.TINY
    L = oracle.Layer(wl.make_layer(spec))
    x = wl.make_x(9, spec.H, draw=5)
    perm = np.random.default_rng(1).permutation(9)
    a = oracle.moe_layer(L, x)["out"]
    b = oracle.moe_layer(L, x[perm])["out"]
    assert np.array_equal(a[perm], b)


def test_linearity_and_zero_cases():
    spec = wl.TINY
    w = wl.make_layer(spec)
    x = wl.make_x(4, spec.H)
    base = oracle.moe_layer(oracle.Layer(w), x)
    assert not np.isnan(base["out"]).any()
    w2 = dict(w, w_down=w["w_down"] * np.float32(2))
    assert np.array_equal(oracle.moe_layer(oracle.Layer(w2), x)["out"], 2 * base["out"])
    w0 = dict(w, w_gate_up=w["w_gate_up"].copy())
    w0["w_gate_up"][:, spec.I:, :] = 0  # up rows
    assert not oracle.moe_layer(oracle.Layer(w0), x)["out"].any()
    assert not oracle.moe_layer(oracle.Layer(w), np.zeros_like(x))["out"].any()


def test_residual_and_rmsnorm_flags():
    spec = wl.TINY
    L = oracle.Layer(wl.make_layer(spec))
    x = wl.make_x(4, spec.H)
    plain = oracle.moe_layer(L, x)["out"]
    res = oracle.moe_layer(L, x, residual=True)["out"]
    assert np.allclose(res, plain + x.astype(np.float64), rtol=0, atol=1e-14)
    normed = oracle.moe_layer(L, x, rmsnorm_in=True)
    xh = torch.nn.functional.rms_norm(torch.from_numpy(x.astype(np.float64)), (spec.H,), eps=1e-6).numpy()
    direct = oracle.expert_fwd(L, xh, normed["ids"], normed["w"])
    assert np.allclose(normed["out"], direct, rtol=1e-13, atol=1e-14)


def test_generator_is_thread_count_independent():
    k = wl.key(0, 3, wl.T_GATE_UP)
    a = wl.normal_bf16(k, 300001, 0.02, nthreads=1)
    b = wl.normal_bf16(k, 300001, 0.02, nthreads=7)
    assert np.array_equal(a, b)
    c = wl.normal_bf16(k, 1000, 0.02, start=123456, nthreads=2)
    assert np.array_equal(a[123456:124456], c)


def test_e4m3_encoder_is_nearest_code():
    vals = np.random.default_rng(0).standard_normal(2000) * 50
    mags = np.array([oracle.e4m3_value(c) for c in range(127)])
    for v in vals:
        c = wl.e4m3_encode(v)
        dv = oracle.e4m3_value(c)
        assert abs(min(abs(v), 448.0) - abs(dv)) <= np.min(np.abs(mags - min(abs(v), 448.0))) + 1e-15
        assert (dv < 0) == (v < 0) or dv == 0


# ------------------------------------------------------------------- MXFP4 --

def _e2m1_table():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "e2m1_values.txt")) if l.strip() and not l.startswith("#")]
    return {int(c): float(v) for c, v in rows[1:]}


def test_e2m1_decode_all_codes_match_the_specification_table():
    tab = _e2m1_table()
    assert sorted(tab) == list(range(16))
    for c, v in tab.items():
        got = oracle.e2m1_value(c)
        assert got == v and np.signbit(got) == np.signbit(v), c


def test_e8m0_decode_all_codes_match_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = np.array([oracle.e8m0_value(s) for s in range(256)])
    assert np.array_equal(got[:255], ref[:255])
    assert np.isnan(got[255]) and np.isnan(ref[255])


def _mx_decode(q, s):
    """MXFP4 [rows, cols/2] codes and [rows, cols/32] scale bytes to float64,
    from the specification table and torch's E8M0 decode."""
    tab = np.array([_e2m1_table()[c] for c in range(16)])
    codes = np.stack([q & 15, q >> 4], axis=-1).reshape(q.shape[0], -1)
    sc = torch.from_numpy(np.ascontiguousarray(s)).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    return tab[codes] * np.repeat(sc, 32, axis=1)


def test_mxfp4_expert_matches_table_decode():
    """MXFP4 experts (E2M1 codes, E8M0 scale per 32 elements along a row):
    decode with the specification table and torch's E8M0, run the textbook
    SwiGLU; a transposed or misaligned nibble or scale index fails this."""
    spec = wl.LayerSpec(E=2, top_k=1, H=96, I=64, expert_dtype=wl.MXFP4, router_dtype=wl.BF16)
    w = wl.make_layer(spec)
    x = wl.make_x(3, spec.H)
    L = oracle.Layer(w)
    ids = np.array([[1], [0], [1]], np.int32)
    got = oracle.expert_fwd(L, x, ids, np.ones((3, 1)))
    for t in range(3):
        e = ids[t, 0]
        ref = _torch_swiglu(x[t:t + 1], _mx_decode(w["w_gate_up"][e], w["s_gate_up"][e]),
                            _mx_decode(w["w_down"][e], w["s_down"][e]))
        assert np.allclose(got[t], ref[0], rtol=1e-12, atol=1e-12)


def test_mxfp4_generator_scales_and_codes():
    """The generator's blocks: scale 2^(floor(log2 amax) - 2), every code the
    nearest E2M1 value of w / scale (saturating at 6), ties to the even code."""
    k = wl.key(0, 0, 1)
    q, s = wl.mxfp4_matrices(k, 1, 8, 128, 0.1)
    src = wl.normal_f32(k, 8 * 128, 1.0).astype(np.float64).reshape(8, 128) * 0.1
    dec = _mx_decode(q[0], s[0])
    tab = np.array(sorted(set(abs(v) for v in _e2m1_table().values())))
    for r in range(8):
        for b in range(4):
            blk = src[r, 32 * b:32 * b + 32]
            scale = 2.0 ** (np.floor(np.log2(np.abs(blk).max())) - 2)
            assert int(s[0, r, b]) == int(np.log2(scale)) + 127
            for c in range(32):
                a = min(abs(blk[c]) / scale, 6.0)
                best = np.min(np.abs(tab - a))
                assert abs(abs(dec[r, 32 * b + c]) / scale - a) <= best + 1e-12
    for v in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0):  # exact ties go to the even code
        c = wl.e2m1_encode(v)
        assert c % 2 == 0, (v, c)


# -------------------------------------------------------------------- q4_0 --

def test_f16_decode_all_codes_match_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_value(int(h)) for h in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def _q4_decode(q, s):
    """q4_0 [rows, cols/2] code bytes and [rows, cols/32] binary16 scales to
    float64: per block of 16 bytes the low nibbles are elements 0..15 and the
    high nibbles elements 16..31; value (code - 8) * d, d from numpy's float16."""
    rows = q.shape[0]
    blk = q.reshape(rows, -1, 16).astype(np.int64)
    codes = np.concatenate([blk & 15, blk >> 4], axis=-1).reshape(rows, -1)
    d = np.ascontiguousarray(s).view(np.float16).astype(np.float64)
    return (codes - 8) * np.repeat(d, 32, axis=1)


def test_q4_0_expert_matches_reference_decode():
    """q4_0 experts: decode with numpy's binary16 and the block layout (low
    nibbles first), run the textbook SwiGLU; a swapped nibble half, a wrong
    code offset or a misaligned scale index fails this."""
    spec = wl.LayerSpec(E=2, top_k=1, H=96, I=64, expert_dtype=wl.Q4_0, router_dtype=wl.BF16)
    w = wl.make_layer(spec)
    x = wl.make_x(3, spec.H)
    L = oracle.Layer(w)
    ids = np.array([[1], [0], [1]], np.int32)
    got = oracle.expert_fwd(L, x, ids, np.ones((3, 1)))
    for t in range(3):
        e = ids[t, 0]
        ref = _torch_swiglu(x[t:t + 1], _q4_decode(w["w_gate_up"][e], w["s_gate_up"][e]),
                            _q4_decode(w["w_down"][e], w["s_down"][e]))
        assert np.allclose(got[t], ref[0], rtol=1e-12, atol=1e-12)


def test_q4_0_layer_equals_fp32_layer_of_its_values():
    """A q4_0 layer and the fp32 layer holding exactly its decoded weights
    (powers-of-two scales, so every value is exact in fp32) give the same
    output bit for bit: the element order of a block is that of the fp32 rows."""
    E, k, H, I = 3, 2, 64, 32
    rng = np.random.default_rng(7)
    gu_codes = rng.integers(0, 16, size=(E, 2 * I, H))
    dn_codes = rng.integers(0, 16, size=(E, H, I))
    gu_exp = rng.integers(-9, -5, size=(E, 2 * I, H // 32))
    dn_exp = rng.integers(-9, -5, size=(E, H, I // 32))

    def pack(codes, exps):
        r = codes.reshape(codes.shape[0], codes.shape[1], -1, 32)
        q = (r[..., :16] | (r[..., 16:] << 4)).astype(np.uint8).reshape(codes.shape[0], codes.shape[1], -1)
        s = np.ldexp(1.0, exps).astype(np.float16).view(np.uint16)
        vals = (codes - 8) * np.repeat(np.ldexp(1.0, exps), 32, axis=-1)
        return q, s, vals.astype(np.float32)

    qg, sg, vg = pack(gu_codes, gu_exp)
    qd, sd, vd = pack(dn_codes, dn_exp)
    wr = (rng.standard_normal((E, H)) * 0.2).astype(np.float32)
    x = rng.standard_normal((5, H)).astype(np.float32)
    Lq = oracle.Layer(dict(spec=_spec(E, k, H, I, wl.Q4_0, wl.F32), w_router=wr, w_gate_up=qg, w_down=qd,
                           s_gate_up=sg, s_down=sd))
    Lf = _f32_layer(E, k, H, I, vg, vd, w_router=wr)
    oq, of = oracle.moe_layer(Lq, x), oracle.moe_layer(Lf, x)
    for n in ("out", "ids", "w", "logits"):
        assert np.array_equal(oq[n], of[n]), n


def test_f16_encode_matches_numpy_rounding():
    rng = np.random.default_rng(3)
    vals = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-8, 4, 2000),
                           [0.0, -0.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 65504.0, 1.0 + 2.0 ** -11,
                            1.0 + 3 * 2.0 ** -11, 2.0 ** -14 - 2.0 ** -25]])
    for v in vals:
        assert wl.f16_encode(float(v)) == int(np.float16(v).view(np.uint16)), v


def test_q4_0_generator_scales_and_codes():
    """The generator's blocks: scale = binary16(amax / 7), every code the
    nearest integer to w / d plus 8 (ties to even), clamped to 0..15."""
    k = wl.key(0, 0, 1)
    q, s = wl.q4_0_matrices(k, 1, 8, 128, 0.1)
    src = wl.normal_f32(k, 8 * 128, 1.0).astype(np.float64).reshape(8, 128) * 0.1
    dec = _q4_decode(q[0], s[0])
    for r in range(8):
        for b in range(4):
            blk = src[r, 32 * b:32 * b + 32]
            d = float(np.float16(np.abs(blk).max() / 7.0))
            assert float(np.ascontiguousarray(s[0, r, b:b + 1]).view(np.float16)[0]) == d
            want = np.clip(np.rint(blk / d) + 8, 0, 15) - 8
            assert np.array_equal(dec[r, 32 * b:32 * b + 32] / d, want)
