"""GPU parity: every stage of the HIP path against the CPU oracle on identical inputs.

Routing and buffer indices are compared bit-exactly (routing mismatches are allowed only
for near-tie tokens, counted and reported); floating-point outputs within the max-abs-
relative tolerances in ``parity.TOL``.  Inputs are seeded and synthetic.  Every call goes
through the C ABI via ``gemm_gate_softmax_amd.ops``.
"""
import os
import sys

import numpy as np
import pytest
import torch

from gemm_gate_softmax_amd import ops
from gemm_gate_softmax_amd import workloads as W

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from parity import (TOL, WEIGHT_ATOL, compare_routing, max_abs_rel, rms_rel,  # noqa: E402
                    routing_note, skewed_routing)

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _native():
    ops.lib()                       # raises if libmoe.so is missing: no fallback exists
    assert torch.cuda.is_available()


def dev(a, dt=None):
    return W.to_device(a, dt, DEV)


def host(t, dt=None):
    return W.to_host(t, dt)


def _log(msg):
    print(msg, flush=True)


def ws_word(ws, i):
    """The i-th int32 of a workspace: 0 = out-of-range routing ids (buffer build), 1 =
    tokens the gate re-decided from exactly rounded logits."""
    return int(host(ws[4 * i:4 * i + 4].view(torch.int32))[0])


# --------------------------------------------------------------------------- buffers

PFT_SHAPES = [(0, 2, 8), (1, 1, 1), (5, 3, 7), (256, 2, 8), (1000, 8, 256), (4096, 2, 64),
              (8192, 6, 64), (4096, 6, 128), (4096, 8, 256), (777, 5, 1000), (3, 64, 64),
              (1500, 4, 1024)]


@pytest.mark.parametrize("T,k,E", PFT_SHAPES)
def test_pft_parity(orc, T, k, E):
    rng = np.random.default_rng(T + 7 * k + E)
    te = skewed_routing(rng, T, k, E, alpha=1.2, empty_every=5 if E >= 5 * k else 0)
    ref = orc.pft_build(te, E)
    got = ops.moe_pft_build(dev(te), E)
    torch.cuda.synchronize()
    assert int(host(got["ws"][:4].view(torch.int32))[0]) == 0
    for n in ("counts", "offsets", "token_ids", "expert_ids", "dest_pos"):
        assert np.array_equal(host(got[n]), ref[n]), n


def test_pft_deterministic_and_out_of_range(orc):
    rng = np.random.default_rng(3)
    T, k, E = 3000, 8, 256
    te = skewed_routing(rng, T, k, E)
    runs = [ops.moe_pft_build(dev(te), E) for _ in range(3)]
    torch.cuda.synchronize()
    for r in runs[1:]:
        for n in ("counts", "offsets", "token_ids", "expert_ids", "dest_pos"):
            assert torch.equal(r[n], runs[0][n])
    bad = te.copy()
    bad[10, 3], bad[2000, 0], bad[2999, 7] = E, -1, 10 ** 6
    got = ops.moe_pft_build(dev(bad), E)
    torch.cuda.synchronize()
    assert int(host(got["ws"][:4].view(torch.int32))[0]) == 3
    dp = host(got["dest_pos"])
    assert dp[10, 3] == -1 and dp[2000, 0] == -1 and dp[2999, 7] == -1


def test_pft_many_segments(orc):
    # more routing entries than the scan's block has threads x 512 (one segment per wave of
    # 512 entries): the per-expert running sums and the error count each take more than
    # one segment per thread
    rng = np.random.default_rng(11)
    T, k, E = 140000, 4, 64
    te = skewed_routing(rng, T, k, E, alpha=1.2)
    assert (T * k + 511) // 512 > 1024
    ref = orc.pft_build(te, E)
    got = ops.moe_pft_build(dev(te), E)
    torch.cuda.synchronize()
    assert int(host(got["ws"][:4].view(torch.int32))[0]) == 0
    for n in ("counts", "offsets", "token_ids", "expert_ids", "dest_pos"):
        assert np.array_equal(host(got[n]), ref[n]), n
    # out-of-range ids in the first segment and around and past segment 1024
    bad = te.copy()
    flat = [7, 1023 * 512 + 100, 1024 * 512 + 5, T * k - 1]
    for i in flat:
        bad[i // k, i % k] = E + i % 3
    got = ops.moe_pft_build(dev(bad), E)
    torch.cuda.synchronize()
    assert int(host(got["ws"][:4].view(torch.int32))[0]) == len(flat)
    dp = host(got["dest_pos"])
    assert all(dp[i // k, i % k] == -1 for i in flat)
    assert int(host(got["counts"]).sum()) == T * k - len(flat)


# ---------------------------------------------------------------- dispatch / combine

MOVE_SHAPES = [(1, 1, 64), (300, 3, 192), (4096, 8, 7168), (513, 6, 2048)]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("T,k,H", MOVE_SHAPES)
def test_dispatch_parity(orc, dt, T, k, H):
    rng = np.random.default_rng(T * k + H)
    x = W._store(rng.standard_normal((T, H)), dt)
    E = max(2 * k, 16)
    b = orc.pft_build(skewed_routing(rng, T, k, E), E)
    ref = orc.dispatch(dt, x, b["dest_pos"])
    got = ops.moe_dispatch(dev(x, dt), dev(b["dest_pos"]))
    assert np.array_equal(host(got, dt), ref)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("T,k,H", MOVE_SHAPES)
def test_combine_parity(orc, dt, T, k, H):
    rng = np.random.default_rng(T * k + H + 1)
    N = T * k
    y = W._store(rng.standard_normal((N, H)), dt)
    dpos = rng.permutation(N).astype(np.int32).reshape(T, k)
    w = rng.random((T, k)).astype(np.float32) + 0.05
    w /= w.sum(1, keepdims=True)
    ref = orc.combine(dt, y, dpos, w)
    got = host(ops.moe_combine(dev(y, dt), dev(dpos), dev(w)), dt)
    # fp32 FMA chain vs double sum: a few fp32 ulps; bf16: at most one bf16 ulp apart
    assert max_abs_rel(got, ref, dt) <= (1e-6 if dt == "f32" else 2.0 ** -7)
    if dt == "bf16":
        assert np.mean(got != ref) < 0.01


# ------------------------------------------------------------------------------ gate

GATE_SHAPES = [(1, 64, 8, 1), (200, 256, 8, 2), (333, 512, 64, 6), (256, 1024, 256, 8),
               (64, 128, 1000, 8), (130, 192, 6, 6), (64, 64, 64, 64),
               # k = 64 < E: the first expert left out is the 65th pick, beyond the wave's lanes
               (96, 256, 200, 64)]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("T,H,E,k", GATE_SHAPES)
def test_gate_parity(orc, dt, T, H, E, k):
    cfg = W.LayerConfig("g", T=T, H=H, E=E, F=64, k=k, dtype=dt, bias=("zipf", 1.0))
    g = W.make_gate_inputs(cfg, seed=T + E)
    te_ref, tw_ref, _, l64 = orc.gate_topk(dt, g["x"], g["wg"], g["bias"], k, want_logits=True)
    ws = ops.workspace(ops.MOE_WS_GATE, T, H, E, 64, k, ops.dtype_code(W.torch_dtype(dt)), DEV)
    te, tw = ops.moe_gate_topk(dev(g["x"], dt), dev(g["wg"], dt), dev(g["bias"]), k, ws=ws)
    te, tw = host(te), host(tw)
    r = compare_routing(te, te_ref, l64, k)
    _log(f"gate {dt} T={T} H={H} E={E} k={k}: {routing_note(r, ws_word(ws, 1))}")
    assert len(r["mismatch"]) == 0
    dw = float(np.max(np.abs(tw - tw_ref)))
    _log(f"    max |dw| {dw:.2e}")
    assert dw <= WEIGHT_ATOL


def _near_tie_gate_inputs(dt, T, H, E, seed):
    """Exact and near ties by construction.  Every token row of x repeats with period 64
    along H, and expert 2i + 1's gate row is expert 2i's row rotated by a multiple of 64:
    each token's two logits are sums of the same products in different orders, so they tie
    exactly, while fp32 accumulation in any blocked order separates them by rounding noise.
    The bias then splits some pairs by one to three fp32 ulps of the logit, far below that
    noise."""
    rng = np.random.default_rng(seed)
    base = rng.standard_normal((T, 64))
    x = W._store(np.tile(base, (1, H // 64)), dt)
    wg = W._store(rng.standard_normal((E, H)) / np.sqrt(H), dt)
    for i in range(0, E - 1, 2):
        wg[i + 1] = np.roll(wg[i], 64 * (1 + i % (H // 64 - 1)))
    bias = (rng.standard_normal(E) * 0.5).astype(np.float32)
    for i in range(0, E - 1, 2):
        bias[i + 1] = bias[i]
        if i % 4 == 2:       # 1-3 ulps of a logit near 2 (ulp 2^-22) apart
            bias[i + 1] = np.float32(bias[i] + (1 + i % 3) * 2.0 ** -22 * (1 if i % 8 == 2 else -1))
    return x, wg, bias


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("T,H,E,k", [(512, 2048, 16, 4), (256, 7168, 64, 6)])
def test_gate_near_ties_decided_exactly(orc, dt, T, H, E, k):
    x, wg, bias = _near_tie_gate_inputs(dt, T, H, E, seed=H + E)
    te_ref, tw_ref, _, l64 = orc.gate_topk(dt, x, wg, bias, k, want_logits=True)
    ws = ops.workspace(ops.MOE_WS_GATE, T, H, E, 64, k, ops.dtype_code(W.torch_dtype(dt)), DEV)
    te, tw = ops.moe_gate_topk(dev(x, dt), dev(wg, dt), dev(bias), k, ws=ws)
    te, tw = host(te), host(tw)
    r = compare_routing(te, te_ref, l64, k)
    refined = ws_word(ws, 1)
    _log(f"gate near ties {dt} T={T} H={H} E={E} k={k}: {routing_note(r, refined)}")
    assert r["near_tie"] > T // 2          # the construction does make near ties
    assert refined >= r["near_tie"]         # and the gate saw every one of them
    assert len(r["mismatch"]) == 0
    assert np.max(np.abs(tw - tw_ref)) <= WEIGHT_ATOL


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_gate_exact_logits_bit_exact(orc, dt):
    # Integer-grid inputs: every partial sum is exact in fp32, so routing must agree with
    # no exemption at all, ties (broken toward the lower id) included.
    rng = np.random.default_rng(17)
    T, H, E, k = 512, 256, 64, 6
    x = W._store(rng.integers(-2, 3, (T, H)) * 2.0 ** -3, dt)
    wg = W._store(rng.integers(-2, 3, (E, H)) * 2.0 ** -8, dt)
    bias = (rng.integers(-4, 5, E) * 2.0 ** -11).astype(np.float32)
    te_ref, tw_ref = orc.gate_topk(dt, x, wg, bias, k)
    te, tw = ops.moe_gate_topk(dev(x, dt), dev(wg, dt), dev(bias), k)
    assert np.array_equal(host(te), te_ref)
    # exact logits: only exp and the division round, a few fp32 ulps
    assert np.allclose(host(tw), tw_ref, rtol=1e-6, atol=1e-7)
    # all-equal logits: experts 0..k-1 with weight 1/k
    te, tw = ops.moe_gate_topk(dev(x, dt), torch.zeros_like(dev(wg, dt)), None, k)
    assert np.array_equal(host(te), np.tile(np.arange(k, dtype=np.int32), (T, 1)))
    assert np.allclose(host(tw), 1.0 / k, rtol=1e-6)


# ------------------------------------------------------------------------ experts

def _segments(rng, E, N, empties=True):
    """Uneven per-expert row counts summing to N, with empty experts and ragged tails."""
    w = rng.pareto(1.0, E) + 0.05
    if empties:
        w[rng.choice(E, size=max(1, E // 4), replace=False)] = 0.0
    c = np.floor(w / w.sum() * N).astype(np.int64)
    c[np.argmax(w)] += N - c.sum()
    return np.concatenate([[0], np.cumsum(c)]).astype(np.int32)


GEMM_SHAPES = [  # (N, E, H, F)
    (1, 1, 64, 64), (37, 3, 64, 128), (600, 12, 256, 192), (1000, 5, 192, 320),
    (700, 1, 128, 256), (2000, 40, 128, 128), (3000, 1024, 64, 128)]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("N,E,H,F", GEMM_SHAPES)
def test_grouped_gemm_parity(orc, dt, N, E, H, F):
    rng = np.random.default_rng(N + E + H + F)
    offsets = _segments(rng, E, N, empties=E > 2)
    xd = W._store(rng.standard_normal((N, H)), dt)
    w1 = W._store(rng.standard_normal((E, F, H)) / np.sqrt(H), dt)
    w3 = W._store(rng.standard_normal((E, F, H)) / np.sqrt(H), dt)
    w2 = W._store(rng.standard_normal((E, H, F)) / np.sqrt(F), dt)
    h_ref, y_ref = orc.grouped_gemm_swiglu(dt, xd, offsets, w1, w3, w2)
    h, y = ops.moe_grouped_gemm_swiglu(dev(xd, dt), dev(offsets), dev(w1, dt), dev(w3, dt),
                                       dev(w2, dt))
    h, y = host(h, dt), host(y, dt)
    eh, ey = max_abs_rel(h, h_ref, dt), max_abs_rel(y, y_ref, dt)
    _log(f"gemm {dt} N={N} E={E} H={H} F={F}: h err {eh:.2e} y err {ey:.2e} "
         f"(rms {rms_rel(y, y_ref, dt):.2e})")
    assert eh <= TOL[dt] and ey <= TOL[dt]
    # the up product alone (w2 = y = NULL) runs the same kernel: identical h
    h_up, y_up = ops.moe_grouped_gemm_swiglu(dev(xd, dt), dev(offsets), dev(w1, dt),
                                             dev(w3, dt), None)
    assert y_up is None
    assert np.array_equal(host(h_up, dt), h)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("pad", [0, 8192])
def test_grouped_gemm_tile_boundaries(orc, dt, pad):
    """Segments on both sides of every tile-size boundary: experts of up to 64 rows take
    one 64-token tile, larger ones 128-token tiles with a ragged last tile (64-token tiles
    when the call has fewer 128-token tiles than CUs: pad adds an expert that lifts it over
    that line); empty experts take none."""
    counts = [64, 65, 1, 0, 63, 128, 129, 0, 192, 64, 2, 255, 256, 257, 0, 33] + ([pad] if pad else [])
    E, H, F = len(counts), 128, 320
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    N = int(offsets[-1])
    rng = np.random.default_rng(64)
    xd = W._store(rng.standard_normal((N, H)), dt)
    w1 = W._store(rng.standard_normal((E, F, H)) / np.sqrt(H), dt)
    w3 = W._store(rng.standard_normal((E, F, H)) / np.sqrt(H), dt)
    w2 = W._store(rng.standard_normal((E, H, F)) / np.sqrt(F), dt)
    h_ref, y_ref = orc.grouped_gemm_swiglu(dt, xd, offsets, w1, w3, w2)
    h, y = ops.moe_grouped_gemm_swiglu(dev(xd, dt), dev(offsets), dev(w1, dt), dev(w3, dt),
                                       dev(w2, dt))
    h, y = host(h, dt), host(y, dt)
    eh, ey = max_abs_rel(h, h_ref, dt), max_abs_rel(y, y_ref, dt)
    _log(f"gemm tile boundaries {dt}: h err {eh:.2e} y err {ey:.2e}")
    assert eh <= TOL[dt] and ey <= TOL[dt]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_grouped_gemm_gathered_rows(orc, dt):
    """token_ids given: product row p reads x[token_ids[p]] (the dispatch fused into the up
    product).  h and y equal the call on the dispatched rows xd = x[token_ids] bit for bit,
    and the oracle within tolerance; the up product alone gives the same h.  Segments cross
    every tile-size boundary; token ids repeat and come in any order."""
    counts = [64, 65, 1, 0, 63, 128, 129, 0, 192, 2, 257, 33]
    E, H, F, T = len(counts), 128, 192, 97
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    N = int(offsets[-1])
    rng = np.random.default_rng(97)
    x = W._store(rng.standard_normal((T, H)), dt)
    tok = rng.integers(0, T, N).astype(np.int32)
    w1 = W._store(rng.standard_normal((E, F, H)) / np.sqrt(H), dt)
    w3 = W._store(rng.standard_normal((E, F, H)) / np.sqrt(H), dt)
    w2 = W._store(rng.standard_normal((E, H, F)) / np.sqrt(F), dt)
    xd = x[tok]
    h_ref, y_ref = orc.grouped_gemm_swiglu(dt, xd, offsets, w1, w3, w2)
    args = (dev(offsets), dev(w1, dt), dev(w3, dt))
    h_g, y_g = ops.moe_grouped_gemm_swiglu(dev(x, dt), *args, dev(w2, dt), token_ids=dev(tok))
    h_d, y_d = ops.moe_grouped_gemm_swiglu(dev(xd, dt), *args, dev(w2, dt))
    h_g, y_g, h_d, y_d = (host(t, dt) for t in (h_g, y_g, h_d, y_d))
    assert np.array_equal(h_g, h_d) and np.array_equal(y_g, y_d)
    eh, ey = max_abs_rel(h_g, h_ref, dt), max_abs_rel(y_g, y_ref, dt)
    _log(f"gemm gathered rows {dt}: h err {eh:.2e} y err {ey:.2e}")
    assert eh <= TOL[dt] and ey <= TOL[dt]
    h_up, y_up = ops.moe_grouped_gemm_swiglu(dev(x, dt), *args, None, token_ids=dev(tok))
    assert y_up is None and np.array_equal(host(h_up, dt), h_g)


# ----------------------------------------------------------------------- whole layer

SMALL_LAYERS = [
    W.CONFIGS["tiny_f32"],
    W.LayerConfig("small_bf16", T=300, H=256, E=16, F=192, k=4, dtype="bf16", bias=("zipf", 1.2)),
    W.LayerConfig("small_f32", T=200, H=128, E=24, F=320, k=6, dtype="f32", bias=("zipf", 1.0)),
    # the most experts the ABI takes: nearly every expert has a handful of rows
    W.LayerConfig("wide_bf16", T=256, H=128, E=1024, F=128, k=8, dtype="bf16", bias=("zipf", 1.2)),
    # the most picks per token the ABI takes, with experts left out
    W.LayerConfig("max_k_bf16", T=96, H=128, E=128, F=64, k=64, dtype="bf16", bias=("zipf", 1.0)),
    # the smallest H and F: every product is a single k-slice
    W.LayerConfig("min_dims_bf16", T=500, H=64, E=16, F=64, k=4, dtype="bf16", bias=("zipf", 1.2)),
]


@pytest.mark.parametrize("cfg", SMALL_LAYERS, ids=lambda c: c.name)
def test_layer_parity_small(orc, cfg):
    d = W.make_host(cfg, seed=0)
    dt = cfg.dtype
    ref = orc.layer_forward(dt, d["x"], d["wg"], d["bias"], d["w1"], d["w3"], d["w2"], cfg.k)
    te_ref, _, _, l64 = orc.gate_topk(dt, d["x"], d["wg"], d["bias"], cfg.k, want_logits=True)
    out, bufs, ws = ops.moe_layer_forward(dev(d["x"], dt), dev(d["wg"], dt), dev(d["bias"]),
                                          dev(d["w1"], dt), dev(d["w3"], dt), dev(d["w2"], dt),
                                          cfg.k)
    out = host(out, dt)
    r = compare_routing(host(bufs["top_experts"]), te_ref, l64, cfg.k)
    assert len(r["mismatch"]) == 0
    err = max_abs_rel(out, ref, dt)
    _log(f"layer {cfg.name}: err {err:.2e}; {routing_note(r, ws_word(ws, 1))}")
    assert err <= TOL[dt]
    # buffers of the GPU routing are exactly the oracle's buffers of that routing
    b_ref = orc.pft_build(host(bufs["top_experts"]), cfg.E)
    for n in ("counts", "offsets", "token_ids", "expert_ids", "dest_pos"):
        assert np.array_equal(host(bufs[n]), b_ref[n]), n
    assert int(host(ws[:4].view(torch.int32))[0]) == 0


# Layers with more tiles than the chip has CUs in both bf16 expert products, so their
# persistent tile loop runs several tiles per workgroup, claimed from the per-XCD counters,
# with the 64-token tiles of small experts mixed among the 128-token tiles.  The second draw
# runs on the first call's workspace, whose counters the first call left at their final
# values: the kernel that writes the tile tables has to clear them.  The first draw gathers
# its rows from x (dispatch fused), the second reads them from xd.
RUN_LAYERS = [
    W.LayerConfig("runs_bf16", T=2048, H=1024, E=48, F=1024, k=4, dtype="bf16", bias=("zipf", 1.2)),
    W.LayerConfig("runs_skew_bf16", T=1536, H=512, E=40, F=768, k=3, dtype="bf16", bias=("zipf", 1.2)),
]


@pytest.mark.parametrize("cfg", RUN_LAYERS, ids=lambda c: c.name)
def test_layer_persistent_runs(orc, cfg):
    dt = cfg.dtype
    ws = None
    for seed in (0, 1):
        d = W.make_host(cfg, seed=seed)
        out, bufs, ws = ops.moe_layer_forward(dev(d["x"], dt), dev(d["wg"], dt), dev(d["bias"]),
                                              dev(d["w1"], dt), dev(d["w3"], dt), dev(d["w2"], dt),
                                              cfg.k, ws=ws, fuse_dispatch=seed == 0)
        assert (bufs["xd"] is None) == (seed == 0)
        te_ref, tw_ref, _, l64 = orc.gate_topk(dt, d["x"], d["wg"], d["bias"], cfg.k, want_logits=True)
        r = compare_routing(host(bufs["top_experts"]), te_ref, l64, cfg.k)
        assert len(r["mismatch"]) == 0
        b_ref = orc.pft_build(te_ref, cfg.E)
        for n in ("counts", "offsets", "token_ids", "expert_ids", "dest_pos"):
            assert np.array_equal(host(bufs[n]), b_ref[n]), n
        c = b_ref["counts"]
        tiles = int(sum((n + 127) // 128 for n in c if n > 64) + np.count_nonzero((c > 0) & (c <= 64)))
        # more up-product tiles than CUs (runs_bf16: the down product's too), small experts among them
        assert tiles * (cfg.F // 128) > 256 and np.any((c > 0) & (c <= 64))
        xd_ref = orc.dispatch(dt, d["x"], b_ref["dest_pos"])
        h_ref, y_ref = orc.grouped_gemm_swiglu(dt, xd_ref, b_ref["offsets"], d["w1"], d["w3"], d["w2"])
        out_ref = orc.combine(dt, y_ref, b_ref["dest_pos"], tw_ref)
        eh = max_abs_rel(host(bufs["h"], dt), h_ref, dt)
        ey = max_abs_rel(host(bufs["y"], dt), y_ref, dt)
        eo = max_abs_rel(host(out, dt), out_ref, dt)
        _log(f"persistent runs {cfg.name} seed {seed}: {tiles} token tiles x {cfg.F // 128} up / "
             f"{cfg.H // 256} down feature tiles; err h {eh:.2e} y {ey:.2e} out {eo:.2e}")
        assert eh <= TOL[dt] and ey <= TOL[dt] and eo <= TOL[dt]
        assert ws_word(ws, 0) == 0


# The method's degenerate layers: one expert (every token to it with weight 1: a dense
# SwiGLU FFN), every expert chosen by every token (k = E), and a single token.
DEGENERATE_LAYERS = [
    W.LayerConfig("one_expert_f32", T=130, H=128, E=1, F=192, k=1, dtype="f32"),
    W.LayerConfig("one_expert_bf16", T=300, H=192, E=1, F=128, k=1, dtype="bf16"),
    W.LayerConfig("k_equals_e_bf16", T=100, H=192, E=8, F=128, k=8, dtype="bf16", bias=("zipf", 1.0)),
    W.LayerConfig("one_token_bf16", T=1, H=256, E=64, F=128, k=6, dtype="bf16", bias=("zipf", 1.2)),
]


@pytest.mark.parametrize("cfg", DEGENERATE_LAYERS, ids=lambda c: c.name)
def test_layer_degenerate_cases(orc, cfg):
    d = W.make_host(cfg, seed=4)
    dt = cfg.dtype
    ref = orc.layer_forward(dt, d["x"], d["wg"], d["bias"], d["w1"], d["w3"], d["w2"], cfg.k)
    outs = []
    for fuse in (False, True):
        out, bufs, ws = ops.moe_layer_forward(dev(d["x"], dt), dev(d["wg"], dt), dev(d["bias"]),
                                              dev(d["w1"], dt), dev(d["w3"], dt), dev(d["w2"], dt),
                                              cfg.k, fuse_dispatch=fuse)
        outs.append(out)
        assert int(host(ws[:4].view(torch.int32))[0]) == 0
        counts = host(bufs["counts"])
        assert int(counts.sum()) == cfg.T * cfg.k
        if cfg.k == cfg.E:             # every token picks every expert exactly once
            assert np.array_equal(counts, np.full(cfg.E, cfg.T))
            assert np.array_equal(np.sort(host(bufs["top_experts"]), axis=1),
                                  np.tile(np.arange(cfg.E), (cfg.T, 1)))
        if cfg.E == 1:                 # the renormalised weight of a single pick is exactly 1
            assert np.all(host(bufs["top_weights"]) == 1.0)
    assert torch.equal(outs[0], outs[1])
    got = host(outs[0], dt)
    err = max_abs_rel(got, ref, dt)
    _log(f"layer {cfg.name}: err {err:.2e}")
    assert err <= TOL[dt]
    if cfg.E == 1 and dt == "f32":
        # pinned apart from the oracle: the dense SwiGLU FFN by torch on the CPU (float64)
        x = torch.from_numpy(np.asarray(d["x"], dtype=np.float64))
        w1, w3, w2 = (torch.from_numpy(np.asarray(d[n][0], dtype=np.float64)) for n in ("w1", "w3", "w2"))
        ffn = (torch.nn.functional.silu(x @ w1.T) * (x @ w3.T)) @ w2.T
        assert max_abs_rel(got, ffn.numpy(), dt) <= TOL[dt]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("T,H,E,k", [(200, 256, 8, 2), (333, 512, 64, 6), (256, 1024, 256, 8)])
def test_gate_sigmoid_parity(orc, dt, T, H, E, k):
    cfg = W.LayerConfig("g", T=T, H=H, E=E, F=64, k=k, dtype=dt, bias=("zipf", 1.0))
    g = W.make_gate_inputs(cfg, seed=T + E + 1)
    te_ref, tw_ref, _, l64 = orc.gate_topk(dt, g["x"], g["wg"], g["bias"], k, want_logits=True,
                                           routing="sigmoid")
    te, tw = ops.moe_gate_topk(dev(g["x"], dt), dev(g["wg"], dt), dev(g["bias"]), k,
                               routing="sigmoid")
    te, tw = host(te), host(tw)
    r = compare_routing(te, te_ref, l64, k)
    _log(f"gate sigmoid {dt} T={T} H={H} E={E} k={k}: {routing_note(r)}")
    assert len(r["mismatch"]) == 0
    assert np.max(np.abs(tw - tw_ref)) <= WEIGHT_ATOL


@pytest.mark.parametrize("cfg", SMALL_LAYERS[1:], ids=lambda c: c.name)
def test_layer_sigmoid_routing_small(orc, cfg):
    d = W.make_host(cfg, seed=3)
    dt = cfg.dtype
    ref = orc.layer_forward(dt, d["x"], d["wg"], d["bias"], d["w1"], d["w3"], d["w2"], cfg.k,
                            routing="sigmoid")
    te_ref, _, _, l64 = orc.gate_topk(dt, d["x"], d["wg"], d["bias"], cfg.k, want_logits=True,
                                      routing="sigmoid")
    out, bufs, _ = ops.moe_layer_forward(dev(d["x"], dt), dev(d["wg"], dt), dev(d["bias"]),
                                         dev(d["w1"], dt), dev(d["w3"], dt), dev(d["w2"], dt),
                                         cfg.k, routing="sigmoid", fuse_dispatch=True)
    r = compare_routing(host(bufs["top_experts"]), te_ref, l64, cfg.k)
    assert len(r["mismatch"]) == 0
    err = max_abs_rel(host(out, dt), ref, dt)
    _log(f"layer sigmoid {cfg.name}: out err {err:.2e}; {routing_note(r)}")
    assert err <= TOL[dt]


def test_layer_deterministic():
    cfg = SMALL_LAYERS[1]
    d = W.make_device(cfg, seed=1, device=DEV)
    a = ops.moe_layer_forward(d["x"], d["wg"], d["bias"], d["w1"], d["w3"], d["w2"], cfg.k)[0]
    b = ops.moe_layer_forward(d["x"], d["wg"], d["bias"], d["w1"], d["w3"], d["w2"], cfg.k)[0]
    assert torch.equal(a, b)


FUSED_CASES = SMALL_LAYERS + [W.CONFIGS["xmoe_small"], W.CONFIGS["xmoe_large"]]


@pytest.mark.parametrize("cfg", FUSED_CASES, ids=lambda c: c.name)
def test_layer_fused_dispatch_identical(orc, cfg):
    # bufs.xd = NULL gathers the expert rows from x through token_ids on load: the same
    # values reach the same MFMAs in the same order, so every output is bit-identical to
    # the staged path, and the oracle pins the staged path elsewhere.
    d = W.make_device(cfg, seed=2, device=DEV)
    args = (d["x"], d["wg"], d["bias"], d["w1"], d["w3"], d["w2"], cfg.k)
    out_s, b_s, _ = ops.moe_layer_forward(*args)
    out_f, b_f, _ = ops.moe_layer_forward(*args, fuse_dispatch=True)
    torch.cuda.synchronize()
    assert b_f["xd"] is None
    for n in ("top_experts", "counts", "offsets", "token_ids", "dest_pos", "h", "y"):
        assert torch.equal(b_s[n], b_f[n]), n
    assert torch.equal(out_s, out_f)
    _log(f"[fused] {cfg.name}: staged and fused-dispatch layers agree bit for bit")


def test_layer_zero_tokens():
    cfg = SMALL_LAYERS[0].scaled(T=0)
    d = W.make_device(cfg, seed=0, device=DEV)
    out, _, _ = ops.moe_layer_forward(d["x"], d["wg"], d["bias"], d["w1"], d["w3"], d["w2"], cfg.k)
    assert out.shape == (0, cfg.H)


def test_rejects_bad_arguments_on_device():
    x = torch.zeros((8, 64), device=DEV)
    wg = torch.zeros((4, 64), device=DEV)
    with pytest.raises(ops.MoeError):
        ops.moe_gate_topk(x, wg, None, 5)                     # k > E
    with pytest.raises(ops.MoeError):
        ops.moe_dispatch(torch.zeros((8, 96), device=DEV), torch.zeros((8, 2), dtype=torch.int32, device=DEV))
    ws = torch.zeros(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(ops.MoeError):
        ops.moe_gate_topk(x, wg, None, 2, ws=ws)              # workspace too small


# ----------------------------------------------------------------------- full sizes

def _expert_host(d, e, dt):
    return tuple(host(d[n][e], dt) for n in ("w1", "w3", "w2"))


def _weights_host(d, experts, dt):
    """Host copies of the expert weights at full shape; only the listed experts' rows are
    filled (the oracle reads no other expert's weights, so the rest of the pages are never
    touched)."""
    out = {}
    for n in ("w1", "w3", "w2"):
        a = np.empty(tuple(d[n].shape), np.float32 if dt == "f32" else np.uint16)
        for e in experts:
            a[e] = host(d[n][e], dt)
        out[n] = a
    return out


@pytest.mark.timeout(600)
@pytest.mark.parametrize("seed", [1, 2])
@pytest.mark.parametrize("name", ["xmoe_small", "xmoe_medium", "xmoe_large", "xmoe_super"])
def test_routing_full_size_more_seeds(orc, name, seed):
    """Other draws of the full-size layers (near ties fall elsewhere): the fused layer's
    routing on every token and every buffer array bit-exact against the oracle, routing
    weights within tolerance."""
    cfg = W.CONFIGS[name]
    dt = cfg.dtype
    _log(f"[routing] {name} seed {seed}: generating inputs")
    d = W.make_device(cfg, seed=seed, device=DEV)
    out, bufs, ws = ops.moe_layer_forward(d["x"], d["wg"], d["bias"], d["w1"], d["w3"], d["w2"],
                                          cfg.k, fuse_dispatch=True)
    torch.cuda.synchronize()
    x_h, wg_h = host(d["x"], dt), host(d["wg"], dt)
    bias_h = None if d["bias"] is None else host(d["bias"])
    del d, out
    te_ref, tw_ref, _, l64 = orc.gate_topk(dt, x_h, wg_h, bias_h, cfg.k, want_logits=True)
    te, tw = host(bufs["top_experts"]), host(bufs["top_weights"])
    r = compare_routing(te, te_ref, l64, cfg.k)
    _log(f"[routing] {name} seed {seed}: {routing_note(r, ws_word(ws, 1))}")
    assert len(r["mismatch"]) == 0
    assert float(np.max(np.abs(tw - tw_ref))) <= WEIGHT_ATOL
    b_ref = orc.pft_build(te_ref, cfg.E)
    for n in ("counts", "offsets", "token_ids", "expert_ids", "dest_pos"):
        assert np.array_equal(host(bufs[n]), b_ref[n]), n
    _log(f"[routing] {name} seed {seed}: {W.routing_summary(b_ref['counts'])}")


EVERY_ROW = [("top2_f32", 0), ("xmoe_small", 0), ("xmoe_medium", 0), ("xmoe_large", 0),
             ("top2_f32", 1), ("xmoe_small", 1), ("xmoe_medium", 1)]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,seed", EVERY_ROW)
def test_layer_full_size_every_row(orc, name, seed):
    """The layer as the benchmark times it (seed 0; also a second draw of the smaller
    configurations; dispatch fused into the up product), compared with the oracle on every
    token and every buffer row: routing and all buffer arrays bit-exact, routing weights, h
    and y of all N rows, and out of all T tokens."""
    cfg = W.CONFIGS[name]
    dt = cfg.dtype
    _log(f"[every row] {name} seed {seed}: generating inputs")
    d = W.make_device(cfg, seed=seed, device=DEV)
    out, bufs, ws = ops.moe_layer_forward(d["x"], d["wg"], d["bias"], d["w1"], d["w3"], d["w2"],
                                          cfg.k, fuse_dispatch=True)
    torch.cuda.synchronize()
    assert bufs["xd"] is None
    assert ws_word(ws, 0) == 0
    x_h, wg_h = host(d["x"], dt), host(d["wg"], dt)
    bias_h = None if d["bias"] is None else host(d["bias"])
    te_ref, tw_ref, _, l64 = orc.gate_topk(dt, x_h, wg_h, bias_h, cfg.k, want_logits=True)
    te, tw = host(bufs["top_experts"]), host(bufs["top_weights"])
    r = compare_routing(te, te_ref, l64, cfg.k)
    _log(f"[every row] {name} seed {seed}: {routing_note(r, ws_word(ws, 1))}")
    assert len(r["mismatch"]) == 0
    dw = float(np.max(np.abs(tw - tw_ref)))
    assert dw <= WEIGHT_ATOL, dw
    b_ref = orc.pft_build(te_ref, cfg.E)
    for n in ("counts", "offsets", "token_ids", "expert_ids", "dest_pos"):
        assert np.array_equal(host(bufs[n]), b_ref[n]), n
    _log(f"[every row] {name} seed {seed}: routing {W.routing_summary(b_ref['counts'])}; "
         f"max |dw| {dw:.2e}; oracle experts over all {cfg.N} rows")
    active = np.flatnonzero(b_ref["counts"])
    w = _weights_host(d, active, dt)
    xd_ref = orc.dispatch(dt, x_h, b_ref["dest_pos"])
    h_ref, y_ref = orc.grouped_gemm_swiglu(dt, xd_ref, b_ref["offsets"], w["w1"], w["w3"], w["w2"])
    del w
    out_ref = orc.combine(dt, y_ref, b_ref["dest_pos"], tw_ref)
    h, y, o = host(bufs["h"], dt), host(bufs["y"], dt), host(out, dt)
    eh, ey, eo = max_abs_rel(h, h_ref, dt), max_abs_rel(y, y_ref, dt), max_abs_rel(o, out_ref, dt)
    _log(f"[every row] {name} seed {seed}: max-abs-rel err h {eh:.2e} y {ey:.2e} out {eo:.2e} "
         f"(rms {rms_rel(h, h_ref, dt):.2e} / {rms_rel(y, y_ref, dt):.2e} / "
         f"{rms_rel(o, out_ref, dt):.2e}); tolerance {TOL[dt]:g}")
    assert eh <= TOL[dt] and ey <= TOL[dt] and eo <= TOL[dt]


@pytest.mark.parametrize("name", ["xmoe_super"])
def test_layer_full_size_sampled(orc, name):
    """The X-MoE Super shape (a parity case beyond the benchmark set): routing of every
    token and all buffer arrays exact; sampled expert rows and tokens against the oracle."""
    cfg = W.CONFIGS[name]
    dt = cfg.dtype
    _log(f"[full] {name}: generating inputs")
    d = W.make_device(cfg, seed=0, device=DEV)
    out, bufs, ws = ops.moe_layer_forward(d["x"], d["wg"], d["bias"], d["w1"], d["w3"], d["w2"], cfg.k)
    torch.cuda.synchronize()
    assert ws_word(ws, 0) == 0
    x_h, wg_h = host(d["x"], dt), host(d["wg"], dt)
    bias_h = None if d["bias"] is None else host(d["bias"])
    te_ref, tw_ref, _, l64 = orc.gate_topk(dt, x_h, wg_h, bias_h, cfg.k, want_logits=True)
    te, tw = host(bufs["top_experts"]), host(bufs["top_weights"])
    r = compare_routing(te, te_ref, l64, cfg.k)
    _log(f"[full] {name}: {routing_note(r, ws_word(ws, 1))}")
    assert len(r["mismatch"]) == 0
    assert np.max(np.abs(tw - tw_ref)) <= WEIGHT_ATOL
    b_ref = orc.pft_build(te, cfg.E)
    for n in ("counts", "offsets", "token_ids", "expert_ids", "dest_pos"):
        assert np.array_equal(host(bufs[n]), b_ref[n]), n
    # dispatch: every buffer row is its token's row (property, all rows)
    assert torch.equal(bufs["xd"], d["x"][bufs["token_ids"].long()])
    counts, offs = b_ref["counts"], b_ref["offsets"]
    big = int(np.argmax(counts))
    nz = np.flatnonzero(counts)
    small = int(nz[np.argmin(counts[nz])])
    rng = np.random.default_rng(0)
    rows = {offs[big], offs[big + 1] - 1, (offs[big] + offs[big + 1]) // 2, offs[small],
            offs[small + 1] - 1, *rng.integers(0, cfg.N, 10).tolist()}
    rows = sorted(int(p) for p in rows)
    xd_rows = host(bufs["xd"][rows], dt)
    h_rows, y_rows = host(bufs["h"][rows], dt), host(bufs["y"][rows], dt)
    cache = {}
    for i, p in enumerate(rows):
        e = int(b_ref["expert_ids"][p])
        if e not in cache:
            cache[e] = _expert_host(d, e, dt)
        w1, w3, w2 = cache[e]
        h1, y1 = orc.grouped_gemm_swiglu(dt, xd_rows[i:i + 1], np.array([0, 1], np.int32),
                                         w1[None], w3[None], w2[None])
        assert max_abs_rel(h_rows[i:i + 1], h1, dt) <= TOL[dt], (p, e)
        assert max_abs_rel(y_rows[i:i + 1], y1, dt) <= TOL[dt], (p, e)
    toks = sorted(set(rng.choice(cfg.T, size=12, replace=False).tolist()))
    out_h = host(out, dt)
    for t in toks:
        ys = []
        for j in range(cfg.k):
            e = int(te_ref[t, j])
            if e not in cache:
                cache[e] = _expert_host(d, e, dt)
            w1, w3, w2 = cache[e]
            ys.append(orc.grouped_gemm_swiglu(dt, x_h[t:t + 1], np.array([0, 1], np.int32),
                                              w1[None], w3[None], w2[None], want_h=False)[1])
        chain = orc.combine(dt, np.concatenate(ys), np.arange(cfg.k, dtype=np.int32)[None],
                            tw_ref[t:t + 1])
        assert max_abs_rel(out_h[t:t + 1], chain, dt) <= TOL[dt], t
    _log(f"[full] {name}: {len(rows)} sampled expert rows and {len(toks)} tokens match")
