"""Pins of the oracle's layer backward (CPU only).

The backward formulas in the oracle are checked against things other than themselves:
central finite differences of the oracle's forward, an independent float64 autograd of the
same mixture written here with plain torch CPU ops, the zero sum of softmax-routing logit
gradients, exact linearity in dout, and the single-expert case where routing weights are
constant.
"""
import numpy as np
import pytest
import torch

import oracle
from gemm_gate_softmax_amd import workloads as W

GRADS = ("dx", "dwg", "dbias", "dw1", "dw3", "dw2")


def _fd_inputs():
    """T=3, H=4, E=4, F=3, k=2 with logit gaps near 1, so perturbations of 1e-2 keep the
    picks (checked below) while the routing weights stay away from 0 and 1."""
    rng = np.random.default_rng(11)
    T, H, E, F = 3, 4, 4, 3
    base = np.array([[1.0, 0.5, -0.5, -1.0], [-1.0, 1.0, 0.5, -0.5], [0.5, -1.0, 1.0, -0.5]])
    x = (base + 0.05 * rng.standard_normal((T, H))).astype(np.float32)
    wg = (2.0 * np.eye(E, H) + 0.1 * rng.standard_normal((E, H))).astype(np.float32)
    bias = (0.1 * rng.standard_normal(E)).astype(np.float32)
    w1 = (0.5 * rng.standard_normal((E, F, H))).astype(np.float32)
    w3 = (0.5 * rng.standard_normal((E, F, H))).astype(np.float32)
    w2 = (0.5 * rng.standard_normal((E, H, F))).astype(np.float32)
    dout = rng.standard_normal((T, H)).astype(np.float32)
    return dict(x=x, wg=wg, bias=bias, w1=w1, w3=w3, w2=w2), dout


def _loss(p, dout, k, routing):
    out = oracle.layer_forward("f32", p["x"], p["wg"], p["bias"], p["w1"], p["w3"], p["w2"], k,
                               routing=routing)
    return float(np.sum(dout.astype(np.float64) * out.astype(np.float64)))


@pytest.mark.parametrize("routing", ["softmax", "sigmoid"])
def test_backward_matches_finite_differences(routing):
    p, dout = _fd_inputs()
    k, eps = 2, 1e-2
    te0, _ = oracle.gate_topk("f32", p["x"], p["wg"], p["bias"], k, routing=routing)
    g = oracle.layer_backward("f32", p["x"], p["wg"], p["bias"], p["w1"], p["w3"], p["w2"], k,
                              dout, routing=routing)
    names = dict(x="dx", wg="dwg", bias="dbias", w1="dw1", w3="dw3", w2="dw2")
    for pname, gname in names.items():
        fd = np.empty(p[pname].shape)
        for idx in np.ndindex(p[pname].shape):
            vals = []
            for sgn in (1.0, -1.0):
                q = {n: a.copy() for n, a in p.items()}
                q[pname][idx] += np.float32(sgn * eps)
                te, _ = oracle.gate_topk("f32", q["x"], q["wg"], q["bias"], k, routing=routing)
                assert np.array_equal(te, te0), "perturbation changed the picks"
                vals.append(_loss(q, dout, k, routing))
            # the stored perturbation is what was applied
            step = float(np.float32(p[pname][idx] + np.float32(eps))) - float(np.float32(p[pname][idx] - np.float32(eps)))
            fd[idx] = (vals[0] - vals[1]) / step
        err = np.max(np.abs(fd - g[gname]))
        scale = max(1.0, float(np.max(np.abs(g[gname]))))
        assert err <= 2e-3 * scale, (gname, err, scale)


def _torch_reference(dt, p, dout, te, routing):
    """float64 autograd of out[t] = sum_j w_tj * SwiGLU_{e_tj}(x[t]), picks te fixed."""
    def f64(a):
        a = np.asarray(a)
        if a.dtype == np.uint16:
            a = W.bf16_bits_to_f32(a)
        return torch.tensor(np.asarray(a, np.float64), requires_grad=True)
    x, wg, b = f64(p["x"]), f64(p["wg"]), f64(p["bias"])
    w1, w3, w2 = f64(p["w1"]), f64(p["w3"]), f64(p["w2"])
    picks = torch.tensor(te.astype(np.int64))
    lsel = (x @ wg.T + b).gather(1, picks)
    if routing == "softmax":
        w = torch.softmax(lsel, dim=1)
    else:
        s = torch.sigmoid(lsel)
        w = s / s.sum(dim=1, keepdim=True)
    out = torch.zeros_like(x)
    for j in range(te.shape[1]):
        e = picks[:, j]
        a = torch.einsum("th,tfh->tf", x, w1[e])
        gg = torch.einsum("th,tfh->tf", x, w3[e])
        hh = torch.nn.functional.silu(a) * gg
        out = out + w[:, j:j + 1] * torch.einsum("tf,thf->th", hh, w2[e])
    d = np.asarray(dout)
    if d.dtype == np.uint16:
        d = W.bf16_bits_to_f32(d)
    (out * torch.tensor(np.asarray(d, np.float64))).sum().backward()
    return dict(dx=x.grad.numpy(), dwg=wg.grad.numpy(), dbias=b.grad.numpy(),
                dw1=w1.grad.numpy(), dw3=w3.grad.numpy(), dw2=w2.grad.numpy())


@pytest.mark.parametrize("routing", ["softmax", "sigmoid"])
@pytest.mark.parametrize("dt,rtol", [("f32", 1e-5), ("bf16", 2e-2)])
def test_backward_matches_float64_autograd(dt, rtol, routing):
    cfg = W.LayerConfig("bwd", T=24, H=32, E=8, F=24, k=3, dtype=dt, bias=("zipf", 1.0))
    p = W.make_host(cfg, seed=4)
    rng = np.random.default_rng(9)
    dout = W._store(rng.standard_normal((cfg.T, cfg.H)), dt)
    te, _ = oracle.gate_topk(dt, p["x"], p["wg"], p["bias"], cfg.k, routing=routing)
    g = oracle.layer_backward(dt, p["x"], p["wg"], p["bias"], p["w1"], p["w3"], p["w2"], cfg.k,
                              dout, routing=routing)
    ref = _torch_reference(dt, p, dout, te, routing)
    for n in GRADS:
        scale = float(np.max(np.abs(ref[n])))
        err = float(np.max(np.abs(g[n] - ref[n])))
        # the oracle uses the stored (rounded) h and y where the forward does; the float64
        # reference does not round: the difference is a few storage ulps of those values
        assert err <= rtol * scale, (n, err, scale)


def test_softmax_logit_gradients_sum_to_zero():
    cfg = W.LayerConfig("bwd", T=40, H=32, E=16, F=16, k=4, dtype="f32", bias=("zipf", 1.2))
    p = W.make_host(cfg, seed=2)
    dout = np.random.default_rng(1).standard_normal((cfg.T, cfg.H)).astype(np.float32)
    g = oracle.layer_backward("f32", p["x"], p["wg"], p["bias"], p["w1"], p["w3"], p["w2"],
                              cfg.k, dout)
    # per token the renormalised softmax weights sum to 1, so their logit gradients sum to 0
    assert abs(float(np.sum(g["dbias"]))) <= 1e-12 * float(np.sum(np.abs(g["dbias"])))
    assert np.any(g["dbias"] != 0.0)


@pytest.mark.parametrize("routing", ["softmax", "sigmoid"])
def test_backward_is_linear_in_dout(routing):
    cfg = W.LayerConfig("bwd", T=16, H=32, E=8, F=16, k=2, dtype="f32", bias=("zipf", 1.0))
    p = W.make_host(cfg, seed=3)
    dout = np.random.default_rng(2).standard_normal((cfg.T, cfg.H)).astype(np.float32)
    args = ("f32", p["x"], p["wg"], p["bias"], p["w1"], p["w3"], p["w2"], cfg.k)
    g1 = oracle.layer_backward(*args, dout, routing=routing)
    g2 = oracle.layer_backward(*args, 2.0 * dout, routing=routing)
    for n in GRADS + ("dtw",):
        assert np.array_equal(g2[n], 2.0 * g1[n]), n


def test_single_expert_has_no_gate_gradient():
    cfg = W.LayerConfig("bwd", T=8, H=16, E=1, F=8, k=1, dtype="f32")
    p = W.make_host(cfg, seed=6)
    dout = np.random.default_rng(3).standard_normal((cfg.T, cfg.H)).astype(np.float32)
    g = oracle.layer_backward("f32", p["x"], p["wg"], p["bias"], p["w1"], p["w3"], p["w2"], 1, dout)
    assert np.all(g["dwg"] == 0.0) and np.all(g["dbias"] == 0.0)
    assert np.any(g["dx"] != 0.0) and np.any(g["dw1"] != 0.0)


def test_backward_stages_reject_bad_input():
    with pytest.raises(RuntimeError):
        oracle.dispatch_backward(np.zeros((4, 8)), np.array([[0, 9], [1, 2]], np.int32))
    with pytest.raises(RuntimeError):
        oracle.gate_backward("f32", np.zeros((2, 4), np.float32), np.zeros((3, 4), np.float32),
                             None, np.array([[0], [5]], np.int32), np.zeros((2, 1)))


def test_stage_wrappers_compose_to_the_layer_backward():
    """The per-stage entry points (used by the sampled full-size GPU checks) chained by hand
    give the whole-layer backward."""
    cfg = W.LayerConfig("bwd", T=20, H=32, E=6, F=16, k=2, dtype="bf16", bias=("zipf", 1.0))
    p = W.make_host(cfg, seed=8)
    dout = W._store(np.random.default_rng(4).standard_normal((cfg.T, cfg.H)), "bf16")
    te, tw = oracle.gate_topk("bf16", p["x"], p["wg"], p["bias"], cfg.k)
    b = oracle.pft_build(te, cfg.E)
    xd = oracle.dispatch("bf16", p["x"], b["dest_pos"])
    h, y = oracle.grouped_gemm_swiglu("bf16", xd, b["offsets"], p["w1"], p["w3"], p["w2"])
    dy, dw = oracle.combine_backward("bf16", dout, y, b["dest_pos"], tw)
    eb = oracle.expert_backward("bf16", xd, b["offsets"], p["w1"], p["w3"], p["w2"], dy, h=h)
    dx = oracle.dispatch_backward(eb["dxd"], b["dest_pos"])
    gb = oracle.gate_backward("bf16", p["x"], p["wg"], p["bias"], te, dw, dx=dx)
    ref = oracle.layer_backward("bf16", p["x"], p["wg"], p["bias"], p["w1"], p["w3"], p["w2"],
                                cfg.k, dout)
    assert np.array_equal(gb["dx"], ref["dx"]) and np.array_equal(dw, ref["dtw"])
    assert np.array_equal(gb["dwg"], ref["dwg"]) and np.array_equal(gb["dbias"], ref["dbias"])
    for n in ("dw1", "dw3", "dw2"):
        assert np.array_equal(eb[n], ref[n]), n
