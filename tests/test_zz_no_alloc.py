"""The layer forward that allocates nothing (moe_layer_forward_noalloc, static device
scratch) against moe_layer_forward on the same inputs, through the C ABI: every output
and intermediate bit-identical, on two calls in a row whose second is smaller, with the
dispatch fused and staged; and within the layer tolerance of the oracle."""
import os
import sys

import numpy as np
import pytest
import torch

from gemm_gate_softmax_amd import ops
from gemm_gate_softmax_amd import workloads as W

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from parity import TOL, max_abs_rel  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"
NAMES = ("top_experts", "top_weights", "counts", "offsets", "token_ids", "expert_ids",
         "dest_pos", "h", "y")


@pytest.fixture(scope="module", autouse=True)
def _native():
    ops.lib()
    assert torch.cuda.is_available()


def _check_call(orc, cfg, seed, fuse):
    d = W.make_host(cfg, seed=seed)
    dt = cfg.dtype
    dv = {n: W.to_device(d[n], dt if n != "bias" else None, DEV) for n in d}
    args = (dv["x"], dv["wg"], dv["bias"], dv["w1"], dv["w3"], dv["w2"], cfg.k)
    ref_out, ref_bufs, _ = ops.moe_layer_forward(*args, fuse_dispatch=fuse)
    bufs = ops.alloc_layer_bufs(cfg.T, cfg.H, cfg.E, cfg.F, cfg.k, dv["x"].dtype, DEV,
                                fuse_dispatch=fuse)
    out = torch.empty_like(ref_out)
    ops.moe_layer_forward_noalloc(*args, out=out, bufs=bufs)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out)
    for n in NAMES:
        assert torch.equal(bufs[n], ref_bufs[n]), n
    if not fuse:
        assert torch.equal(bufs["xd"], ref_bufs["xd"])
    ref = orc.layer_forward(dt, d["x"], d["wg"], d["bias"], d["w1"], d["w3"], d["w2"], cfg.k)
    err = max_abs_rel(W.to_host(out, dt), ref, dt)
    print(f"noalloc {cfg.name} T={cfg.T} fuse={fuse}: identical to moe_layer_forward; "
          f"oracle err {err:.2e}", flush=True)
    assert err <= TOL[dt]


@pytest.mark.parametrize("fuse", [True, False])
def test_noalloc_matches_layer_forward_twice(orc, fuse):
    big = W.LayerConfig("noalloc_big", T=300, H=256, E=16, F=192, k=4, dtype="bf16",
                        bias=("zipf", 1.2))
    small = big.scaled(name="noalloc_small", T=77)
    _check_call(orc, big, seed=5, fuse=fuse)
    _check_call(orc, small, seed=6, fuse=fuse)


def test_noalloc_fp32_then_smaller():
    cfg = W.CONFIGS["tiny_f32"]
    for T, seed in ((cfg.T, 1), (31, 2)):
        c = cfg.scaled(T=T)
        d = W.make_device(c, seed=seed, device=DEV)
        args = (d["x"], d["wg"], d["bias"], d["w1"], d["w3"], d["w2"], c.k)
        ref_out, _, _ = ops.moe_layer_forward(*args, fuse_dispatch=True)
        bufs = ops.alloc_layer_bufs(c.T, c.H, c.E, c.F, c.k, d["x"].dtype, DEV,
                                    fuse_dispatch=True)
        out = torch.empty_like(ref_out)
        ops.moe_layer_forward_noalloc(*args, out=out, bufs=bufs)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out)
