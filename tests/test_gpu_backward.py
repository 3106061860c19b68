"""GPU parity of the layer backward (moe_layer_backward through the C ABI) against the
CPU oracle's backward on identical inputs.

Every gradient is compared as max |gpu - oracle| / max |oracle| over the tensor.  The
oracle differentiates in double from the forward's stored h and y; the HIP path
accumulates in fp32 and stores its intermediates (dy, dh, a, g, da|dg, dxd) in the storage
type, so bf16 gradients carry a few bf16 roundings along each chain (BWD_TOL).
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from gemm_gate_softmax_amd import ops
from gemm_gate_softmax_amd import workloads as W

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from parity import as_f64  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"
GRADS = ("dx", "dwg", "dbias", "dw1", "dw3", "dw2", "dtw")
FP32_GRADS = ("dbias", "dtw")
# f32: fp32 accumulation over at most a few thousand terms (measured <= 1e-6); bf16: a
# chain of up to three bf16 roundings of intermediates (2^-9 relative each) ahead of an fp32
# product (measured <= 7e-3); the fp32 outputs dtw and dbias see only the stored y and the
# fp32 logits (measured <= 2e-4 at bf16)
BWD_TOL = {"f32": 2e-5, "bf16": 1.5e-2}
FP32_GRAD_TOL = {"f32": 2e-5, "bf16": 2e-3}

CASES = [
    (W.CONFIGS["tiny_f32"], "softmax"),
    (W.LayerConfig("small_bf16", T=300, H=256, E=16, F=192, k=4, dtype="bf16",
                   bias=("zipf", 1.2)), "softmax"),
    (W.LayerConfig("small_f32", T=200, H=128, E=24, F=320, k=6, dtype="f32",
                   bias=("zipf", 1.0)), "softmax"),
    (W.LayerConfig("small_bf16", T=300, H=256, E=16, F=192, k=4, dtype="bf16",
                   bias=("zipf", 1.2)), "sigmoid"),
    (W.LayerConfig("one_expert_f32", T=96, H=128, E=1, F=128, k=1, dtype="f32"), "softmax"),
    # every expert above 64 rows: all weight gradients on the tile GEMM reading the row-major
    # operands, expert offsets not multiples of 64, ragged last k-slices
    (W.LayerConfig("rows_f32", T=333, H=192, E=5, F=128, k=2, dtype="f32"), "softmax"),
    (W.LayerConfig("rows_bf16", T=333, H=192, E=5, F=128, k=2, dtype="bf16"), "softmax"),
    # the smallest H and F: every K-major product is one k-slice (dxd reads W1 for its first
    # slice and W3 for its second)
    (W.LayerConfig("min_dims_bf16", T=500, H=64, E=16, F=64, k=4, dtype="bf16",
                   bias=("zipf", 1.2)), "softmax"),
    # the most picks per token, with experts left out
    (W.LayerConfig("max_k_bf16", T=96, H=128, E=128, F=64, k=64, dtype="bf16",
                   bias=("zipf", 1.0)), "softmax"),
]


@pytest.fixture(scope="module", autouse=True)
def _native():
    ops.lib()                       # raises if libmoe.so is missing: no fallback exists
    assert torch.cuda.is_available()


def _run(cfg, routing, fuse, seed=0):
    d = W.make_device(cfg, seed=seed, device=DEV)
    rng = np.random.default_rng(seed + 100)
    dout_h = W._store(rng.standard_normal((cfg.T, cfg.H)), cfg.dtype)
    dout = W.to_device(dout_h, cfg.dtype, DEV)
    args = (d["x"], d["wg"], d["bias"], d["w1"], d["w3"], d["w2"], cfg.k)
    out, bufs, _ = ops.moe_layer_forward(*args, fuse_dispatch=fuse, routing=routing)
    grads, _ = ops.moe_layer_backward(*args, bufs, dout, routing=routing)
    torch.cuda.synchronize()
    return d, dout_h, bufs, grads


@pytest.mark.parametrize("cfg,routing", CASES, ids=lambda c: getattr(c, "name", c))
def test_layer_backward_parity(cfg, routing):
    d, dout_h, bufs, grads = _run(cfg, routing, fuse=True)
    h = {n: W.to_host(d[n], cfg.dtype if n != "bias" else None) for n in
         ("x", "wg", "w1", "w3", "w2")}
    bias = None if d["bias"] is None else W.to_host(d["bias"], None)
    te_ref, _ = oracle.gate_topk(cfg.dtype, h["x"], h["wg"], bias, cfg.k, routing=routing)
    assert np.array_equal(W.to_host(bufs["top_experts"], None), te_ref), "routing differs"
    if cfg.name.startswith("rows_"):
        counts = W.to_host(bufs["counts"], None)
        assert counts.min() > 64 and any(int(o) % 64 for o in W.to_host(bufs["offsets"], None)), counts
    ref = oracle.layer_backward(cfg.dtype, h["x"], h["wg"], bias, h["w1"], h["w3"], h["w2"],
                                cfg.k, dout_h, routing=routing)
    for n in GRADS:
        got = grads[n].cpu().numpy() if n in FP32_GRADS else as_f64(W.to_host(grads[n], cfg.dtype), cfg.dtype)
        r = ref[n]
        scale = float(np.max(np.abs(r)))
        err = float(np.max(np.abs(got.astype(np.float64) - r)))
        tol = (FP32_GRAD_TOL if n in FP32_GRADS else BWD_TOL)[cfg.dtype] * scale
        print(f"{cfg.name} {routing} {n}: max err {err:.3e} scale {scale:.3e} ({err / max(scale, 1e-30):.2e})",
              flush=True)
        if scale == 0.0:
            assert err == 0.0, n
        else:
            assert err <= tol, (n, err, scale)


def test_single_expert_gate_gradients_are_zero():
    cfg = W.LayerConfig("one_expert_f32", T=96, H=128, E=1, F=128, k=1, dtype="f32")
    _, _, _, grads = _run(cfg, "softmax", fuse=False)
    assert torch.count_nonzero(grads["dwg"]).item() == 0
    assert torch.count_nonzero(grads["dbias"]).item() == 0


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_backward_fused_and_staged_identical_and_deterministic(dt):
    cfg = W.LayerConfig("small", T=300, H=256, E=16, F=192, k=4, dtype=dt, bias=("zipf", 1.2))
    _, _, _, g1 = _run(cfg, "softmax", fuse=True)
    _, _, _, g2 = _run(cfg, "softmax", fuse=False)
    _, _, _, g3 = _run(cfg, "softmax", fuse=True)
    for n in GRADS:
        assert torch.equal(g1[n], g2[n]), n
        assert torch.equal(g1[n], g3[n]), n


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("fuse", [True, False])
def test_backward_with_stored_up_halves_identical(dt, fuse):
    """The forward can store a = x.W1^T and g = x.W3^T beside h (bufs a and g); the backward
    then uses them instead of recomputing them on the same tiles in the same order, so the
    forward's outputs and every gradient are bit-identical either way."""
    cfg = W.LayerConfig("small", T=300, H=256, E=16, F=192, k=4, dtype=dt, bias=("zipf", 1.2))
    d = W.make_device(cfg, seed=0, device=DEV)
    rng = np.random.default_rng(100)
    dout = W.to_device(W._store(rng.standard_normal((cfg.T, cfg.H)), cfg.dtype), cfg.dtype, DEV)
    args = (d["x"], d["wg"], d["bias"], d["w1"], d["w3"], d["w2"], cfg.k)
    results = []
    for store in (False, True):
        bufs = ops.alloc_layer_bufs(cfg.T, cfg.H, cfg.E, cfg.F, cfg.k, d["x"].dtype, DEV,
                                    fuse_dispatch=fuse, store_ag=store)
        out, bufs, _ = ops.moe_layer_forward(*args, bufs=bufs)
        grads, _ = ops.moe_layer_backward(*args, bufs, dout)
        torch.cuda.synchronize()
        results.append((out, bufs, grads))
    (o0, b0, g0), (o1, b1, g1) = results
    assert torch.equal(o0, o1)
    for n in ("h", "y", "top_experts", "top_weights", "token_ids", "dest_pos"):
        assert torch.equal(b0[n], b1[n]), n
    for n in GRADS:
        assert torch.equal(g0[n], g1[n]), n
    # the stored halves give back h: silu(a) * g rounded like h (tolerance: GPU exp and
    # reciprocal against torch's)
    a, g = b1["a"].double(), b1["g"].double()
    h_ref = (a / (1.0 + torch.exp(-a)) * g)
    err = ((b1["h"].double() - h_ref).abs().max() / h_ref.abs().max()).item()
    assert err <= (1e-5 if dt == "f32" else 1e-2), err


def test_experts_without_rows_get_zero_weight_gradients():
    cfg = W.LayerConfig("skewed", T=64, H=128, E=32, F=128, k=2, dtype="bf16", bias=("zipf", 2.0))
    _, _, bufs, grads = _run(cfg, "softmax", fuse=True)
    counts = W.to_host(bufs["counts"], None)
    empty = np.where(counts == 0)[0]
    assert len(empty) > 0
    for n in ("dw1", "dw3", "dw2"):
        assert torch.count_nonzero(grads[n][torch.tensor(empty, device=DEV)]).item() == 0, n


def _sub_offsets(experts_of_rows):
    """Compact expert segments for rows already sorted by expert: (unique experts, offsets)."""
    uniq, counts = np.unique(experts_of_rows, return_counts=True)
    return uniq, np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["xmoe_small", "xmoe_large"])
def test_backward_full_size_sampled(name):
    """At the benchmark shapes, on the launch the benchmark times: dtw and dx of sampled
    tokens, all weight gradients of the expert with the fewest rows (outer-product route)
    and of the expert with the most rows (tile-GEMM route, K ranges of thousands of rows),
    dWg and dbias of the first, and the zero sum of dbias, each against the oracle's stage
    functions on just the rows involved."""
    cfg = W.CONFIGS[name]
    d, dout_h, bufs, grads = _run(cfg, "softmax", fuse=True)
    dt, k = cfg.dtype, cfg.k
    te = W.to_host(bufs["top_experts"], None)
    tw = W.to_host(bufs["top_weights"], None)
    dp = W.to_host(bufs["dest_pos"], None)
    off = W.to_host(bufs["offsets"], None)
    counts = W.to_host(bufs["counts"], None)
    tok = W.to_host(bufs["token_ids"], None)
    x_h = W.to_host(d["x"], dt)
    wg_h = W.to_host(d["wg"], dt)
    bias_h = W.to_host(d["bias"], None)
    rng = np.random.default_rng(5)

    def expert_w(e_list):
        idx = torch.tensor(np.asarray(e_list, np.int64), device=DEV)
        return [W.to_host(d[n][idx], dt) for n in ("w1", "w3", "w2")]

    def check(got, ref, what, fp32=False):
        scale = float(np.max(np.abs(ref)))
        err = float(np.max(np.abs(np.asarray(got, np.float64) - ref)))
        tol = (FP32_GRAD_TOL if fp32 else BWD_TOL)[dt] * scale
        print(f"{name} {what}: max err {err:.3e} scale {scale:.3e}", flush=True)
        assert err <= tol, (what, err, scale)

    # 1. dtw and dx of sampled tokens
    ts = np.sort(rng.choice(cfg.T, size=4, replace=False))
    rows = dp[ts].reshape(-1)                                   # their buffer rows
    y_sub = W.to_host(bufs["y"][torch.tensor(rows.astype(np.int64), device=DEV)], dt)
    dy_ref, dtw_ref = oracle.combine_backward(dt, dout_h[ts], y_sub,
                                              np.arange(len(rows), dtype=np.int32).reshape(len(ts), k),
                                              tw[ts])
    check(grads["dtw"].cpu().numpy()[ts], dtw_ref, "dtw (sampled tokens)", fp32=True)
    order = np.argsort(te[ts].reshape(-1), kind="stable")      # group the rows by expert
    e_rows = te[ts].reshape(-1)[order]
    uniq, soff = _sub_offsets(e_rows)
    w1s, w3s, w2s = expert_w(uniq)
    xd_sub = x_h[np.repeat(ts, k)[order]]
    h_sub = W.to_host(bufs["h"][torch.tensor(rows[order].astype(np.int64), device=DEV)], dt)
    eb = oracle.expert_backward(dt, xd_sub, soff, w1s, w3s, w2s, dy_ref[order], h=h_sub)
    dxd = np.empty_like(eb["dxd"])
    dxd[order] = eb["dxd"]
    dx_ref = dxd.reshape(len(ts), k, cfg.H).sum(axis=1)
    gb = oracle.gate_backward(dt, x_h[ts], wg_h, bias_h, te[ts], dtw_ref, dx=dx_ref)
    check(as_f64(W.to_host(grads["dx"], dt)[ts], dt), gb["dx"], "dx (sampled tokens)")

    # 2. every weight gradient of the expert with the fewest rows and of the one with the
    # most, each from all of its rows
    active = np.where(counts > 0)[0]
    slot = {}
    for t_ in range(cfg.T):
        for j_ in range(k):
            slot[int(dp[t_, j_])] = (t_, j_)
    for e in (int(active[np.argmin(counts[active])]), int(active[np.argmax(counts[active])])):
        prow = np.arange(off[e], off[e + 1])
        tj = [slot[int(p)] for p in prow]
        assert all(int(tok[p]) == t for p, (t, _) in zip(prow, tj))
        dy_e = np.stack([tw[t, j] * as_f64(dout_h[t], dt) for t, j in tj])
        w1s, w3s, w2s = expert_w([e])
        h_e = W.to_host(bufs["h"][int(off[e]):int(off[e + 1])], dt)
        eb = oracle.expert_backward(dt, x_h[[t for t, _ in tj]],
                                    np.array([0, len(prow)], np.int32), w1s, w3s, w2s, dy_e, h=h_e)
        for n in ("dw1", "dw3", "dw2"):
            check(as_f64(W.to_host(grads[n][e], dt), dt), eb[n][0], f"{n}[{e}] ({len(prow)} rows)")
    e = int(active[np.argmin(counts[active])])
    prow = np.arange(off[e], off[e + 1])
    tj = [slot[int(p)] for p in prow]

    # 3. dWg and dbias of that expert, from every token that picked it
    tpick = np.array(sorted({t for t, _ in tj}))
    dtw_t = np.zeros((len(tpick), k))
    for i, t in enumerate(tpick):
        rows_t = dp[t]
        yt = W.to_host(bufs["y"][torch.tensor(rows_t.astype(np.int64), device=DEV)], dt)
        _, dtw_t[i] = oracle.combine_backward(dt, dout_h[[t]], yt,
                                              np.arange(k, dtype=np.int32).reshape(1, k), tw[[t]])
    gb = oracle.gate_backward(dt, x_h[tpick], wg_h, bias_h, te[tpick], dtw_t)
    check(as_f64(W.to_host(grads["dwg"][e], dt), dt), gb["dwg"][e], f"dwg[{e}]")
    check(grads["dbias"].cpu().numpy()[[e]], gb["dbias"][[e]], f"dbias[{e}]", fp32=True)

    # 4. softmax logit gradients of a token sum to zero, so dbias does too
    db = grads["dbias"].double().cpu().numpy()
    assert abs(db.sum()) <= 1e-4 * np.abs(db).sum()
