"""Pins for the CPU oracle: each check compares it with something other than itself.

Sources: closed forms and hand-worked examples (``tests/golden``), brute force on tiny
inputs, exactly-representable inputs, textbook special cases computed with library
routines (torch CPU float64 matmul, numpy einsum), and the structural invariants of
padding-free buffers (X-MoE review, section 三: PFT complexity analysis and training
pipeline steps 1-6; FlashDMoE blog, section 5: only routed tokens are carried).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from gemm_gate_softmax_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _distinct_routing(rng, T, k, E):
    return np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)


# ----------------------------------------------------------------------- bf16 rounding

def test_round_bf16_matches_library_conversion(orc):
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        [0.0, -0.0, 1e-40, -1e-40, 3e38, -3e38]]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = orc.round_bf16(v.astype(np.float64))
    assert np.array_equal(got, ref)


def test_round_bf16_direct_from_double(orc):
    # Halfway cases that a detour through fp32 would round differently (worked by hand):
    # 1 + 2^-8 is the midpoint between bf16 1.0 and 1 + 2^-7; a hair above it must go up.
    v = np.array([1 + 2 ** -8 + 2 ** -40, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8 + 2 ** -40),
                  float.fromhex("0x1.fe8p127"), float.fromhex("0x1.ff8p127"), 2.0 ** -133, 2.0 ** -134, 2.0 ** -134 * 1.5])
    want = [0x3F81, 0x3F80, 0x3F82, 0xBF81, 0x7F7F, 0x7F80, 0x0001, 0x0000, 0x0001]
    assert list(orc.round_bf16(v)) == want


# ------------------------------------------------------------------------------- gate

def _rank_select(l, k):
    """Brute force: e is picked iff fewer than k experts come before it; its slot is that count."""
    T, E = l.shape
    te = np.full((T, k), -1, np.int32)
    for t in range(T):
        for e in range(E):
            before = sum(1 for f in range(E) if l[t, f] > l[t, e] or (l[t, f] == l[t, e] and f < e))
            if before < k:
                te[t, before] = e
    return te


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("E,k", [(8, 1), (8, 2), (16, 5), (12, 12)])
def test_gate_selection_brute_force(orc, dt, E, k):
    rng = np.random.default_rng(E * 100 + k)
    T, H = 48, 40
    x = W._store(rng.standard_normal((T, H)), dt)
    wg = W._store(rng.standard_normal((E, H)) / math.sqrt(H), dt)
    bias = rng.standard_normal(E).astype(np.float32)
    te, tw, l32, l64 = orc.gate_topk(dt, x, wg, bias, k, want_logits=True)
    assert np.array_equal(te, _rank_select(l32, k))
    # the stored logits are the double sums rounded once to fp32
    xs = x if dt == "f32" else W.bf16_bits_to_f32(x)
    gs = wg if dt == "f32" else W.bf16_bits_to_f32(wg)
    ref = xs.astype(np.float64) @ gs.astype(np.float64).T + bias.astype(np.float64)
    assert np.allclose(l64, ref, rtol=0, atol=1e-12)
    assert np.array_equal(l32, l64.astype(np.float32))


@pytest.mark.parametrize("k", [1, 3, 8])
def test_gate_all_ties(orc, k):
    T, H, E = 10, 16, 8
    x = np.random.default_rng(0).standard_normal((T, H)).astype(np.float32)
    te, tw = orc.gate_topk("f32", x, np.zeros((E, H), np.float32), None, k)
    assert np.array_equal(te, np.tile(np.arange(k, dtype=np.int32), (T, 1)))
    assert np.array_equal(tw, np.full((T, k), 1.0 / k, np.float32))


def test_gate_one_hot_rows_give_weight_rows(orc):
    H, E = 24, 10
    rng = np.random.default_rng(3)
    wg = rng.standard_normal((E, H)).astype(np.float32)
    x = np.eye(H, dtype=np.float32)
    _, _, l32, _ = orc.gate_topk("f32", x, wg, None, 2, want_logits=True)
    assert np.array_equal(l32, wg.T)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_gate_integer_grid_exact(orc, dt):
    # Every product and partial sum is a multiple of 2^-11 below 2^8: exact in any order.
    rng = np.random.default_rng(7)
    T, H, E, k = 64, 32, 16, 4
    xi = rng.integers(-2, 3, (T, H))
    gi = rng.integers(-8, 9, (E, H))
    bi = rng.integers(-4, 5, E)
    x = W._store(xi * 2.0 ** -3, dt)
    wg = W._store(gi * 2.0 ** -8, dt)
    bias = (bi * 2.0 ** -11).astype(np.float32)
    te, tw, l32, _ = orc.gate_topk(dt, x, wg, bias, k, want_logits=True)
    exact = [[Fraction(int(xi[t] @ gi[e]), 2 ** 11) + Fraction(int(bi[e]), 2 ** 11) for e in range(E)]
             for t in range(T)]
    assert all(Fraction(float(l32[t, e])) == exact[t][e] for t in range(T) for e in range(E))
    ex = np.array([[float(v) for v in row] for row in exact])
    assert np.array_equal(te, _rank_select(ex, k))
    n_ties = sum(len(set(r)) < E for r in exact)
    assert n_ties > 0          # the grid really produces ties


def test_gate_hand_example(orc):
    g = _golden("gate_hand_example.json")
    x = np.array([[1.0, 0.0]], np.float32)
    wg = np.zeros((g["E"], g["H"]), np.float32)
    te, tw = orc.gate_topk("f32", x, wg, np.array(g["bias"], np.float32), g["k"])
    assert te.tolist() == g["top_experts"]
    assert np.allclose(tw, g["top_weights"], rtol=1e-7, atol=0)


@pytest.mark.parametrize("k", [1, 2, 6])
def test_gate_weights_closed_form(orc, k):
    rng = np.random.default_rng(11 + k)
    T, H, E = 200, 64, 32
    x = rng.standard_normal((T, H)).astype(np.float32)
    wg = (rng.standard_normal((E, H)) / 8).astype(np.float32)
    te, tw, l32, _ = orc.gate_topk("f32", x, wg, None, k, want_logits=True)
    assert np.all(np.abs(tw.astype(np.float64).sum(1) - 1.0) <= k * 2.0 ** -24)
    assert np.all(np.diff(tw, axis=1) <= 0)
    for t in range(T):                # k-only form: the full-E denominator cancels
        l0 = float(l32[t, te[t, 0]])
        num = [math.exp(float(l32[t, e]) - l0) for e in te[t]]
        ref = np.array([v / sum(num) for v in num])
        assert np.allclose(tw[t], ref, rtol=2 ** -23, atol=0)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_sigmoid_routing_selects_like_softmax(orc, dt):
    # both scores increase with the logit, so the picks (and their order) are the same
    rng = np.random.default_rng(23)
    T, H, E, k = 300, 64, 48, 5
    x = W._store(rng.standard_normal((T, H)), dt)
    wg = W._store(rng.standard_normal((E, H)) / 8, dt)
    bias = rng.standard_normal(E).astype(np.float32)
    te_soft, tw_soft = orc.gate_topk(dt, x, wg, bias, k)
    te_sig, tw_sig = orc.gate_topk(dt, x, wg, bias, k, routing="sigmoid")
    assert np.array_equal(te_soft, te_sig)
    assert np.all(np.abs(tw_sig.astype(np.float64).sum(1) - 1.0) <= k * 2.0 ** -24)
    assert np.all(np.diff(tw_sig, axis=1) <= 0)
    assert not np.allclose(tw_soft, tw_sig)          # a different routing function


def test_sigmoid_routing_closed_forms(orc):
    # Wg = 0 makes the logits equal the bias exactly; sigmoid(ln 3) = 3/4, sigmoid(0) = 1/2,
    # sigmoid(-ln 3) = 1/4, so the renormalised picks are plain fractions.
    ln3 = math.log(3.0)
    x = np.ones((1, 64), np.float32)
    wg = np.zeros((4, 64), np.float32)
    bias = np.array([0.0, -ln3, ln3, -5.0], np.float32)
    cases = {1: [2], 2: [2, 0], 3: [2, 0, 1]}
    want = {1: [1.0], 2: [0.6, 0.4], 3: [0.5, 1 / 3, 1 / 6]}
    for k, picks in cases.items():
        te, tw = orc.gate_topk("f32", x, wg, bias, k, routing="sigmoid")
        assert te[0].tolist() == picks
        assert np.allclose(tw[0], want[k], rtol=0, atol=1e-6)
    # a symmetric pair keeps the raw sigmoid values (they already sum to 1); softmax routing
    # of the same logits gives 9/10 and 1/10 instead
    te, tw = orc.gate_topk("f32", x[:, :64], np.zeros((2, 64), np.float32),
                           np.array([ln3, -ln3], np.float32), 2, routing="sigmoid")
    assert np.allclose(tw[0], [0.75, 0.25], rtol=0, atol=1e-6)
    te, tw = orc.gate_topk("f32", x[:, :64], np.zeros((2, 64), np.float32),
                           np.array([ln3, -ln3], np.float32), 2)
    assert np.allclose(tw[0], [0.9, 0.1], rtol=0, atol=1e-6)


# ------------------------------------------------------------------ padding-free buffers

def test_pft_hand_example(orc):
    g = _golden("pft_hand_example.json")
    got = orc.pft_build(np.array(g["top_experts"], np.int32), g["E"])
    for name in ("counts", "offsets", "token_ids", "expert_ids", "dest_pos"):
        assert got[name].tolist() == g[name], name


@pytest.mark.parametrize("T,k,E", [(1, 1, 1), (50, 3, 7), (37, 5, 5), (64, 2, 64)])
def test_pft_brute_force(orc, T, k, E):
    te = _distinct_routing(np.random.default_rng(T * k + E), T, k, E)
    got = orc.pft_build(te, E)
    flat = te.reshape(-1)
    counts = [int(sum(1 for v in flat if v == e)) for e in range(E)]
    assert got["counts"].tolist() == counts
    assert got["offsets"].tolist() == [sum(counts[:e]) for e in range(E + 1)]
    for i, e in enumerate(flat):
        p = sum(counts[:e]) + sum(1 for i2 in range(i) if flat[i2] == e)
        assert got["dest_pos"].reshape(-1)[i] == p
        assert got["token_ids"][p] == i // k and got["expert_ids"][p] == e


def pft_invariants(te, E, b):
    """Structural facts of padding-free buffers that hold at any size."""
    T, k = te.shape
    N = T * k
    counts, offsets = b["counts"], b["offsets"]
    assert counts.sum() == N and offsets[0] == 0 and offsets[E] == N
    assert np.array_equal(np.diff(offsets), counts)
    eid, tok, dp = b["expert_ids"], b["token_ids"], b["dest_pos"]
    assert np.all(np.diff(eid) >= 0)
    assert np.array_equal(np.repeat(np.arange(E), counts), eid)
    for e in range(E):
        seg = tok[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)
    assert np.array_equal(np.sort(dp.reshape(-1)), np.arange(N))      # a permutation: no pad rows
    assert np.array_equal(tok[dp], np.repeat(np.arange(T), k).reshape(T, k))
    assert np.array_equal(eid[dp], te)


@pytest.mark.parametrize("T,k,E", [(256, 2, 8), (4096, 8, 256), (3000, 6, 1024)])
def test_pft_invariants(orc, T, k, E):
    rng = np.random.default_rng(5)
    # skewed routing including experts that receive nothing (every 7th one is never drawn)
    p = 1.0 / np.arange(1, E + 1) ** 1.5
    p[3::7] = 0.0
    te = np.stack([rng.choice(E, size=k, replace=False, p=p / p.sum()) for _ in range(T)]).astype(np.int32)
    b = orc.pft_build(te, E)
    pft_invariants(te, E, b)
    assert np.all(b["counts"][3::7] == 0)


def test_pft_rejects_out_of_range(orc):
    te = np.array([[0, 1], [2, 5]], np.int32)
    with pytest.raises(RuntimeError):
        orc.pft_build(te, 4)


# ----------------------------------------------------------------- dispatch + combine

@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_dispatch_combine_round_trip(orc, dt):
    # With the identity as every expert (y = xd), combining the dispatched rows gives
    # x * sum_j w_j = x for any routing.
    rng = np.random.default_rng(2)
    T, H, E, k = 96, 64, 12, 4
    x = W._store(rng.standard_normal((T, H)), dt)
    te = _distinct_routing(rng, T, k, E)
    w = rng.random((T, k)) + 0.1
    w = (w / w.sum(1, keepdims=True)).astype(np.float32)
    b = orc.pft_build(te, E)
    xd = orc.dispatch(dt, x, b["dest_pos"])
    assert np.array_equal(xd[b["dest_pos"].reshape(-1)], np.repeat(x, k, axis=0))
    assert np.array_equal(xd, x[b["token_ids"]])
    out = orc.combine(dt, xd, b["dest_pos"], w)
    if dt == "bf16":
        assert np.array_equal(out, x)
    else:
        assert np.allclose(out, x, rtol=k * 2.0 ** -23, atol=0)


# ------------------------------------------------------------------------ experts

def _swiglu_ffn_f64(x, w1, w3, w2):
    """Dense SwiGLU FFN with torch CPU float64 (library matmul + silu)."""
    xt = torch.from_numpy(np.asarray(x, np.float64))
    a = xt @ torch.from_numpy(np.asarray(w1, np.float64)).T
    g = xt @ torch.from_numpy(np.asarray(w3, np.float64)).T
    h = torch.nn.functional.silu(a) * g
    return h.numpy(), (h @ torch.from_numpy(np.asarray(w2, np.float64)).T).numpy()


def test_single_expert_top1_is_dense_ffn(orc):
    cfg = W.LayerConfig("e1", T=40, H=64, E=1, F=32, k=1, dtype="f32")
    d = W.make_host(cfg, seed=4)
    out = orc.layer_forward("f32", d["x"], d["wg"], None, d["w1"], d["w3"], d["w2"], 1)
    _, ref = _swiglu_ffn_f64(d["x"], d["w1"][0], d["w3"][0], d["w2"][0])
    assert np.max(np.abs(out - ref)) <= 1e-6 * np.max(np.abs(ref))
    te, tw = orc.gate_topk("f32", d["x"], d["wg"], None, 1)
    assert np.all(te == 0) and np.all(tw == 1.0)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_identical_experts_ignore_routing(orc, dt):
    cfg = W.LayerConfig("same", T=64, H=64, E=6, F=32, k=3, dtype=dt)
    d = W.make_host(cfg, seed=9)
    w1 = np.repeat(d["w1"][:1], 6, 0)
    w3 = np.repeat(d["w3"][:1], 6, 0)
    w2 = np.repeat(d["w2"][:1], 6, 0)
    out = orc.layer_forward(dt, d["x"], d["wg"], None, w1, w3, w2, 3)
    f = (lambda a: a) if dt == "f32" else W.bf16_bits_to_f32
    _, ref = _swiglu_ffn_f64(f(d["x"]), f(w1[0]), f(w3[0]), f(w2[0]))
    tol = 1e-6 if dt == "f32" else 2e-2
    assert np.max(np.abs(f(out) - ref)) <= tol * np.max(np.abs(ref))


def test_expert_rows_python_loops(orc):
    # Per-row loops in plain Python for a few rows of each expert.
    rng = np.random.default_rng(21)
    E, H, F = 3, 12, 8
    counts = [4, 0, 3]
    offsets = np.array([0, 4, 4, 7], np.int32)
    N = 7
    xd = rng.standard_normal((N, H)).astype(np.float32)
    w1 = rng.standard_normal((E, F, H)).astype(np.float32)
    w3 = rng.standard_normal((E, F, H)).astype(np.float32)
    w2 = rng.standard_normal((E, H, F)).astype(np.float32)
    h, y = orc.grouped_gemm_swiglu("f32", xd, offsets, w1, w3, w2)
    for p in range(N):
        e = 0 if p < 4 else 2
        hrow = []
        for f in range(F):
            a = sum(float(xd[p, c]) * float(w1[e, f, c]) for c in range(H))
            g = sum(float(xd[p, c]) * float(w3[e, f, c]) for c in range(H))
            hrow.append(float(np.float32(a / (1.0 + math.exp(-a)) * g)))
        assert np.allclose(h[p], hrow, rtol=1e-7, atol=1e-30)
        for c in range(H):
            s = sum(hrow[f] * float(w2[e, c, f]) for f in range(F))
            assert math.isclose(float(y[p, c]), s, rel_tol=1e-6, abs_tol=1e-30)
    assert counts[1] == 0


# ------------------------------------------------------- dense (GShard-style) formulation

@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_layer_matches_dense_capacity_formulation(orc, dt):
    # The capacity-padded formulation the X-MoE review contrasts with (O(E*C*H) memory),
    # with capacity C = T so nothing is dropped: one-hot dispatch mask [T,E,C], einsum
    # dispatch, per-expert FFN on the padded [C,H] block, weighted einsum combine.
    cfg = W.CONFIGS["tiny_f32"].scaled(dtype=dt, T=64, H=64, E=8, F=32)
    d = W.make_host(cfg, seed=0)
    f = (lambda a: np.asarray(a, np.float64)) if dt == "f32" else \
        (lambda a: W.bf16_bits_to_f32(a).astype(np.float64))
    rnd = (lambda a: a.astype(np.float32).astype(np.float64)) if dt == "f32" else \
        (lambda a: f(orc.round_bf16(a)))
    te, tw = orc.gate_topk(dt, d["x"], d["wg"], d["bias"], cfg.k)
    T, E, C = cfg.T, cfg.E, cfg.T
    mask = np.zeros((T, E, C))
    fill = np.zeros(E, int)
    for t in range(T):                       # positions in token order
        for j in range(cfg.k):
            e = te[t, j]
            mask[t, e, fill[e]] = 1.0
            fill[e] += 1
    xe = np.einsum("tec,th->ech", mask, f(d["x"]))
    ye = np.zeros_like(xe)
    for e in range(E):
        a = xe[e] @ f(d["w1"][e]).T
        g = xe[e] @ f(d["w3"][e]).T
        h = rnd(a / (1 + np.exp(-a)) * g)
        ye[e] = rnd(h @ f(d["w2"][e]).T)
    cw = np.zeros((T, E, C))
    for t in range(T):
        for j in range(cfg.k):
            cw[t] += tw[t, j] * (np.arange(E)[:, None] == te[t, j]) * mask[t]
    ref = rnd(np.einsum("tec,ech->th", cw, ye))
    out = f(orc.layer_forward(dt, d["x"], d["wg"], d["bias"], d["w1"], d["w3"], d["w2"], cfg.k))
    # Same rounding points on both sides: only double summation order differs, so the
    # stored outputs agree except where that order straddles a rounding boundary.
    assert np.mean(out != ref) < 1e-3
    assert np.max(np.abs(out - ref)) <= 2.0 ** -7 * np.max(np.abs(ref))
    # the padded buffer holds exactly the padding-free rows, in the same order
    b = orc.pft_build(te, E)
    xd = f(orc.dispatch(dt, d["x"], b["dest_pos"]))
    for e in range(E):
        c = b["counts"][e]
        assert np.array_equal(xe[e, :c], xd[b["offsets"][e]:b["offsets"][e + 1]])
        assert not xe[e, c:].any()


# ----------------------------------------------------------------------- error paths

def test_oracle_rejects_bad_arguments(orc):
    x = np.zeros((4, 8), np.float32)
    with pytest.raises(KeyError):
        orc.gate_topk("f32", x, np.zeros((3, 8), np.float32), None, 2, routing="relu")
    # an unknown routing id is rejected before any pointer is touched
    assert orc.lib().oracle_gate_topk(0, 4, 8, 3, 2, 5, *([None] * 7)) != 0
    with pytest.raises(RuntimeError):
        orc.gate_topk("f32", x, np.zeros((3, 8), np.float32), None, 4)     # k > E
    with pytest.raises(RuntimeError):
        orc.grouped_gemm_swiglu("f32", np.zeros((3, 8), np.float32), np.array([0, 2], np.int32),
                                np.zeros((1, 4, 8), np.float32), np.zeros((1, 4, 8), np.float32),
                                np.zeros((1, 8, 4), np.float32))            # offsets[E] != N
