"""The layer forward captured into a HIP graph (through torch.cuda.graph) and replayed:
the library enqueues kernels only (no memset nodes, no host reads of device data), so a
captured call replays as is.  Each replay runs after unrelated eager work and a
synchronisation, and its outputs are compared with the eager call's, bit for bit."""
import pytest
import torch

from gemm_gate_softmax_amd import ops
from gemm_gate_softmax_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _native():
    ops.lib()
    assert torch.cuda.is_available()


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(g):
        fn()
    return g


@pytest.mark.parametrize("noalloc", [False, True])
@pytest.mark.parametrize("fuse", [True, False])
@pytest.mark.parametrize("cfg", [W.CONFIGS["tiny_f32"],
                                 W.LayerConfig("graph_bf16", T=300, H=256, E=16, F=192, k=4,
                                               dtype="bf16", bias=("zipf", 1.2))],
                         ids=lambda c: c.name)
def test_layer_graph_replays_match_eager(cfg, fuse, noalloc):
    d = W.make_device(cfg, seed=7, device=DEV)
    args = (d["x"], d["wg"], d["bias"], d["w1"], d["w3"], d["w2"], cfg.k)
    ref_out, ref_bufs, _ = ops.moe_layer_forward(*args, fuse_dispatch=fuse)
    bufs = ops.alloc_layer_bufs(cfg.T, cfg.H, cfg.E, cfg.F, cfg.k, d["x"].dtype, DEV,
                                fuse_dispatch=fuse)
    out = torch.empty_like(ref_out)
    dt = ops.dtype_code(d["x"].dtype)
    ws = ops.workspace(ops.MOE_WS_LAYER, cfg.T, cfg.H, cfg.E, cfg.F, cfg.k, dt, DEV)
    if noalloc:
        step = lambda: ops.moe_layer_forward_noalloc(*args, out=out, bufs=bufs)
    else:
        step = lambda: ops.moe_layer_forward(*args, out=out, bufs=bufs, ws=ws)
    g = _capture(step)
    other = W.make_device(cfg.scaled(T=max(1, cfg.T // 3)), seed=8, device=DEV)
    for _ in range(3):
        out.zero_()
        bufs["h"].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out)
        for n in ("top_experts", "top_weights", "counts", "offsets", "token_ids", "dest_pos", "h", "y"):
            assert torch.equal(bufs[n], ref_bufs[n]), n
        # unrelated eager work between replays
        ops.moe_layer_forward(other["x"], other["wg"], other["bias"], other["w1"], other["w3"],
                              other["w2"], cfg.k, fuse_dispatch=fuse)
        torch.cuda.synchronize()
