#!/usr/bin/env python3
"""Benchmark: forward pass of one MoE layer on one MI355X, through the C ABI.

One step = one ``moe_layer_forward`` call (gate -> padding-free buffers -> dispatch ->
grouped SwiGLU experts -> combine) over one batch of synthetic, device-resident input,
with the dispatch fused into the expert up product (bufs.xd = NULL: rows gathered from x
on load; results identical to the staged layer, whose time is reported beside it).
Default workload: the X-MoE Large layer (T=4096, H=7168, E=256, F=2048, top-8, bf16,
Zipf(1.2) gate bias).  Prints ONE JSON line (see the keys below); with --verbose a
per-stage table goes to stderr first.

  python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config xmoe_large]
                  [--no-cpu-baseline] [--cpu-seconds 15]
  python bench.py --calibrate-copy     # plain 1 GiB device copies, for HBM byte counters
  python bench.py --up-kernel-only     # one staged layer, then only the up-product calls
                                       # (the launches the traffic counters are read on)
  python bench.py --expert-kernels-only  # the same with both products (up, then down)
  python bench.py --dense              # the tile engine vs torch.matmul on dense products
  python bench.py --memory-ceilings    # how fast one workgroup per CU can read 16 bytes a
                                       # lane from the L2s, the Infinity Cache and HBM
  python bench.py --ab LIB,LIB,...     # the layer with each library (variants built by
                                       # gemm_gate_softmax_amd.build --variant), alternating;
                                       # --ab-backward times moe_layer_backward as well

The roofline object covers the dominant kernel, the expert gate/up product with its
SwiGLU epilogue (two thirds of the layer's flops), timed on its own through the same
entry point with w2 = y = NULL.  Its bound is chosen by arithmetic intensity: algorithmic
flop per algorithmic byte (each active expert's W1 and W3 read once, xd read once, h
written once) against the ridge point 2500 TFLOP/s / 8 TB/s; with skewed routing most
experts see a few rows, so at X-MoE Large the kernel sits below the ridge (HBM-bound).
Its "traffic" (bytes per launch between the L2 and the memory fabric, from FETCH_SIZE and
WRITE_SIZE counters scaled by a plain copy's reading; Infinity Cache hits included) comes
from the committed counter summary and is reported only while the kernel sources still
hash to what was profiled.  Step times are the median of per-step event intervals.  The
"parity" object compares the timed step's routing (every token) and output (the CPU
baseline's sample) with the oracle.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer fwd tokens/s + grouped-GEMM % MFMA peak, X-MoE Large, 1 GPU"
HBM_PEAK_GBS = 8000.0                       # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # dense MFMA, published
UP_KERNEL = "expert_gemm_kernel<moe::bf16_t, 2, 1"   # name prefix in profiler output
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "xmoe_large_expert_up_traffic.md")
COPY_BYTES = 1 << 30      # counter calibration copy


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="xmoe_large")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip timing moe_layer_backward (reported beside the forward)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run plain device copies of 1 GiB (counter calibration)")
    ap.add_argument("--expert-kernels-only", action="store_true",
                    help="like --up-kernel-only with both expert products per call (counter "
                         "runs of the down product)")
    ap.add_argument("--up-kernel-only", action="store_true",
                    help="one staged layer, then --steps calls of the up product alone")
    ap.add_argument("--dense", action="store_true",
                    help="the tile engine on dense single-expert products against torch.matmul "
                         "(hipBLASLt) on the same shapes, as a ceiling reference")
    ap.add_argument("--ab", default=None,
                    help="comma-separated libmoe builds (variants from gemm_gate_softmax_amd.build "
                         "--variant): the fused layer, its up product and both expert products "
                         "timed with each, alternating, outputs compared with the first's")
    ap.add_argument("--ab-reps", type=int, default=3)
    ap.add_argument("--ab-backward", action="store_true",
                    help="with --ab: also time moe_layer_backward with each build and compare its "
                         "gradients with the first build's")
    ap.add_argument("--memory-ceilings", action="store_true",
                    help="read rates of the loads the tile engine issues (libmoe_probe.so): "
                         "direct-to-LDS and plain, 4 and 8 issuing waves per CU, from regions "
                         "held in the L2s, in the Infinity Cache and in HBM")
    ap.add_argument("--weight-stream", action="store_true",
                    help="the up product on a routing of one row per expert for every expert of "
                         "the workload: a pure stream of the expert weights (for counter runs)")
    return ap.parse_args()


def kernel_digest():
    """sha256 over the expert kernel's code: counter readings are tied to it."""
    from gemm_gate_softmax_amd.profile_summary import kernel_digest as digest
    return digest()


def recorded_traffic(workload):
    """HBM bytes per launch of the up kernel from the committed counter summary, or None
    when it is missing, for another workload, or taken from other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
    except OSError:
        return None
    fields = dict(re.findall(r"^- (\w+): `([^`]*)`", text, re.M))
    if fields.get("workload") != workload or fields.get("source_sha256") != kernel_digest():
        return None
    return int(fields["fabric_bytes_per_launch"])


def calibrate_copy():
    import torch
    src = torch.full((COPY_BYTES,), 7, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read": COPY_BYTES,
                      "bytes_written": COPY_BYTES, "launches": 3}), flush=True)
    return 0


def algorithmic(cfg, counts):
    """Algorithmic bytes / flops per stage (what the method itself must move/compute)."""
    b = 4 if cfg.dtype == "f32" else 2
    T, H, E, F, k, N = cfg.T, cfg.H, cfg.E, cfg.F, cfg.k, cfg.N
    active = int((counts > 0).sum())
    return dict(
        active_experts=active,
        gemm_flops=6.0 * N * H * F,
        up_flops=4.0 * N * H * F,
        # the up kernel with the dispatch fused (as in the timed step) reads each active
        # expert's W1 and W3 once and the token rows x once, and writes h once
        up_bytes=active * 2.0 * F * H * b + b * (T * H + N * F),
        gemm_bytes=active * 3.0 * H * F * b + b * (2.0 * N * H + 2.0 * N * F),
        dispatch_bytes=b * (T * H + N * H) + 4.0 * N,
        combine_bytes=b * (N * H + T * H) + 8.0 * N,
        gate_bytes=b * (T * H + E * H) + 8.0 * T * k,
        gate_flops=2.0 * T * E * H,
    )


def time_calls(fn, iters, stream):
    """Median ms per call over `iters` back-to-back calls, each bracketed by its own pair of
    events on `stream` (an interval also holds the launch gaps inside the call)."""
    return time_steps(fn, iters, stream)["median"]


def time_steps(fn, iters, stream):
    """Per-call ms of `iters` back-to-back calls: dict(median, mean, min, max, all)."""
    import statistics

    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
    ev[0].record(stream)
    for i in range(iters):
        fn()
        ev[i + 1].record(stream)
    ev[-1].synchronize()
    ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(iters)]
    return {"median": statistics.median(ms), "mean": sum(ms) / len(ms), "min": min(ms),
            "max": max(ms), "all": ms}


def cpu_baseline(cfg, d, seed, target_s, gpu_out, gpu_te, gpu_tw, refined):
    """The oracle, as it is, on the first tokens of the same workload (bounded sample).
    Returns (cpu_baseline record, parity record): the sample's oracle output is compared
    with the GPU's output for the same tokens, and the oracle's routing of every token of
    the batch with the GPU's."""
    import numpy as np

    import oracle
    from gemm_gate_softmax_amd import workloads as W

    dt = cfg.dtype
    x_all, wg = W.to_host(d["x"], dt), W.to_host(d["wg"], dt)
    bias = None if d["bias"] is None else W.to_host(d["bias"], None)
    w_host = {n: np.empty(tuple(d[n].shape), np.float32 if dt == "f32" else np.uint16)
              for n in ("w1", "w3", "w2")}      # pages of unused experts are never touched
    loaded = set()

    def run(ntok):
        te, _ = oracle.gate_topk(dt, x_all[:ntok], wg, bias, cfg.k)
        for e in sorted(set(te.reshape(-1).tolist()) - loaded):
            for n in ("w1", "w3", "w2"):
                w_host[n][e] = W.to_host(d[n][e], dt)
            loaded.add(e)
        t0 = time.perf_counter()
        out, secs = oracle.layer_forward(dt, x_all[:ntok], wg, bias, w_host["w1"], w_host["w3"],
                                         w_host["w2"], cfg.k, stage_seconds=True)
        return time.perf_counter() - t0, secs, out

    # The oracle parallelises over the rows of each expert, so tokens/s grows with the
    # sample; grow it until one run takes about target_s (or the whole batch is used).
    ntok = 16
    while True:
        wall, secs, out_ref = run(ntok)
        if wall >= 0.7 * target_s or ntok >= cfg.T:
            break
        ntok = int(min(cfg.T, ntok * min(8.0, max(2.0, target_s / max(wall, 1e-3)))))
    base = {"value": ntok / wall, "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"first {ntok} of {cfg.T} tokens of the same {cfg.name} layer (same weights), "
                      f"oracle_layer_forward end to end, {wall:.1f} s; stage seconds gate/buffers/"
                      f"dispatch/experts/combine = {', '.join(f'{s:.2f}' for s in secs)}"}
    # parity: routing of the whole batch (oracle gate on every token), output of the sample
    te_ref, tw_ref, _, l64 = oracle.gate_topk(dt, x_all, wg, bias, cfg.k, want_logits=True)
    m = min(cfg.k + 1, cfg.E)
    top = -np.sort(-l64, axis=1)[:, :m]
    gaps = ((top[:, :-1] - top[:, 1:]) / np.maximum(1.0, np.abs(top[:, :-1]))).min(axis=1) \
        if m > 1 else np.full(cfg.T, np.inf)
    g = W.bf16_bits_to_f32(gpu_out[:ntok]) if dt == "bf16" else gpu_out[:ntok]
    r = W.bf16_bits_to_f32(out_ref) if dt == "bf16" else out_ref
    g, r = g.astype(np.float64), r.astype(np.float64)
    scale = float(np.max(np.abs(r))) or 1.0
    parity = {
        "routing_tokens": cfg.T,
        "routing_mismatches": int(np.any(gpu_te != te_ref, axis=1).sum()),
        "near_tie_tokens": int((gaps <= 1e-6).sum()),
        "band_tokens_1e-6_1e-5": int(((gaps > 1e-6) & (gaps <= 1e-5)).sum()),
        "tokens_decided_from_exact_logits": refined,
        "top_weights_max_abs_err": float(np.max(np.abs(gpu_tw - tw_ref))),
        "out_tokens_compared": ntok,
        "out_max_abs_rel": float(np.max(np.abs(g - r))) / scale,
        "out_rms_rel": float(np.sqrt(np.mean((g - r) ** 2)) / (np.sqrt(np.mean(r * r)) or 1.0)),
        "tolerance": 1e-4 if dt == "f32" else 2e-2,
        "note": "oracle gate on every token of the batch; oracle layer output on the "
                "cpu_baseline sample, against the GPU output of the timed step",
    }
    return base, parity


def weight_stream(cfg, args, dev):
    """The up product with every expert given exactly one row: each expert's W1 and W3 are
    read once and almost nothing else moves, so the launch is a pure weight stream through
    the small-expert tiles.  Prints the streamed bytes per launch and the rate."""
    import torch

    from gemm_gate_softmax_amd import ops
    from gemm_gate_softmax_amd import workloads as W

    d = W.make_device(cfg, seed=args.seed, device=dev)
    E, H, F = cfg.E, cfg.H, cfg.F
    xd = d["x"][:E].contiguous()
    offsets = torch.arange(0, E + 1, dtype=torch.int32, device=dev)
    h = torch.empty((E, F), dtype=xd.dtype, device=dev)
    ws = ops.workspace(ops.MOE_WS_GEMM, E, H, E, F, 1, ops.dtype_code(xd.dtype), dev)
    call = lambda: ops.moe_grouped_gemm_swiglu(xd, offsets, d["w1"], d["w3"], None, h=h, ws=ws)
    call()
    torch.cuda.synchronize()
    ms = time_calls(call, max(1, args.steps), torch.cuda.current_stream())
    nbytes = E * 2.0 * F * H * xd.element_size()
    print(json.dumps({"weight_stream": cfg.name, "experts": E, "bytes_per_launch": nbytes,
                      "us": round(ms * 1e3, 1), "GBs": round(nbytes / (ms * 1e-3) / 1e9, 1)}),
          flush=True)
    return 0


DENSE_SHAPES = (   # (rows, H, F): one expert of the X-MoE Large and Small layers
    (4096, 7168, 2048), (8192, 7168, 2048), (16384, 7168, 2048), (8192, 2048, 1408),
    (32768, 2048, 1408))


def dense(args, dev):
    """Dense products (one expert holding every row) through moe_grouped_gemm_swiglu against
    torch.matmul on the same operands: the up product x.[W1; W3]^T (the engine adds its SwiGLU
    epilogue) and the down product h.W2^T.  bf16, fp32 accumulate.  torch.matmul is used only
    as a reference ceiling here; nothing on the library's path calls it."""
    import torch

    from gemm_gate_softmax_amd import ops
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)
    rows = []
    iters = max(4, args.steps)
    for N, H, F in DENSE_SHAPES:
        x = torch.randn(N, H, device=dev, generator=gen).to(torch.bfloat16)
        w1 = (torch.randn(1, F, H, device=dev, generator=gen) / H ** 0.5).to(torch.bfloat16)
        w3 = (torch.randn(1, F, H, device=dev, generator=gen) / H ** 0.5).to(torch.bfloat16)
        w2 = (torch.randn(1, H, F, device=dev, generator=gen) / F ** 0.5).to(torch.bfloat16)
        offs = torch.tensor([0, N], dtype=torch.int32, device=dev)
        h = torch.empty(N, F, dtype=torch.bfloat16, device=dev)
        y = torch.empty(N, H, dtype=torch.bfloat16, device=dev)
        ws = ops.workspace(ops.MOE_WS_GEMM, N, H, 1, F, 1, ops.MOE_BF16, dev)
        wcat = torch.cat([w1[0], w3[0]], 0).t().contiguous()        # [H, 2F]
        w2t = w2[0].t().contiguous()                                # [F, H]
        calls = {
            "engine_up": lambda: ops.moe_grouped_gemm_swiglu(x, offs, w1, w3, None, h=h, ws=ws),
            "engine_up_down": lambda: ops.moe_grouped_gemm_swiglu(x, offs, w1, w3, w2, h=h, y=y,
                                                                  ws=ws),
            "matmul_up": lambda: torch.matmul(x, wcat),
            "matmul_down": lambda: torch.matmul(h, w2t),
        }
        ms = {}
        for name, fn in calls.items():
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            ms[name] = time_steps(fn, iters, torch.cuda.current_stream())["median"]
        ms["engine_down"] = ms["engine_up_down"] - ms["engine_up"]
        fu, fd = 4.0 * N * H * F, 2.0 * N * H * F
        tf = lambda f, m: round(f / (m * 1e-3) / 1e12, 1)
        rows.append({"rows": N, "H": H, "F": F,
                     "up_tflops": {"engine": tf(fu, ms["engine_up"]), "matmul": tf(fu, ms["matmul_up"])},
                     "down_tflops": {"engine": tf(fd, ms["engine_down"]),
                                     "matmul": tf(fd, ms["matmul_down"])},
                     "us": {k_: round(v * 1e3, 1) for k_, v in ms.items()}})
        log(f"dense {N}x{H}x{F}: up engine {rows[-1]['up_tflops']['engine']} vs matmul "
            f"{rows[-1]['up_tflops']['matmul']} TFLOP/s; down engine "
            f"{rows[-1]['down_tflops']['engine']} vs matmul {rows[-1]['down_tflops']['matmul']}")
        del x, w1, w3, w2, h, y, ws, wcat, w2t
        torch.cuda.empty_cache()
    print(json.dumps({"dense": rows, "peak_tflops": MFMA_PEAK_TFLOPS["bf16"],
                      "note": "median of per-call event intervals; matmul = torch.matmul "
                              "(hipBLASLt) on the same operands, reference only"}), flush=True)
    return 0


CEILING_REGIONS = ((1 << 20, "1 MiB (L2)"), (64 << 20, "64 MiB (Infinity Cache)"),
                   (1 << 30, "1 GiB (HBM)"))


def memory_ceilings(args):
    """moe_probe_stream from libmoe_probe.so (a measurement library, not part of libmoe.so):
    256 workgroups, one per CU, each reading 1500 slices of 48 KiB round-robin from a region,
    16 bytes per lane, either as direct-to-LDS transfers into a 3-slot ring (the engine's
    loaders) or as plain loads into registers, or writing them with plain stores.  Median of
    5 timed launches after one warm-up."""
    import ctypes

    import torch

    from gemm_gate_softmax_amd import build as B
    if not os.path.exists(B.PROBE_LIB):
        raise RuntimeError(f"{B.PROBE_LIB} is missing: run the build first")
    probe = ctypes.CDLL(B.PROBE_LIB)
    probe.moe_probe_stream.restype = ctypes.c_int
    probe.moe_probe_stream.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_longlong, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_void_p]
    grid, iters, slice_bytes = 256, 1500, 48 * 1024
    buf = torch.full((1 << 30,), 1, dtype=torch.uint8, device="cuda")
    sink = torch.empty(grid * 8 * 64, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    rows = []
    for region, label in CEILING_REGIONS:
        for kind, kname in ((0, "direct-to-LDS"), (1, "plain loads"), (2, "plain stores")):
            for waves in (4, 8):
                call = lambda: probe.moe_probe_stream(kind, waves, buf.data_ptr(), region, grid,
                                                      iters, sink.data_ptr(), stream.cuda_stream)
                if call() != 0:
                    raise RuntimeError("moe_probe_stream refused its arguments")
                torch.cuda.synchronize()
                ms = time_steps(call, 5, stream)["median"]
                total = grid * iters * slice_bytes / (ms * 1e-3)
                rows.append({"region": label, "kind": kname, "waves_per_cu": waves,
                             "TBs": round(total / 1e12, 2),
                             "GBs_per_cu": round(total / grid / 1e9, 1),
                             "GBs_per_wave": round(total / grid / waves / 1e9, 1)})
                log(f"{label:24s} {kname:14s} {waves} waves/CU: {rows[-1]['TBs']:.2f} TB/s, "
                    f"{rows[-1]['GBs_per_cu']:.1f} GB/s per CU")
    print(json.dumps({"memory_ceilings": rows, "grid": grid, "bytes_per_workgroup":
                      iters * slice_bytes}), flush=True)
    return 0


def ab_compare(cfg, args, dev):
    """The fused layer, the up product as the layer runs it, and both expert products, with
    each library in turn (rounds alternate between them); each library's h, y and out are
    compared with the first library's: bit-identical, or the max-abs-rel error."""
    import torch

    from gemm_gate_softmax_amd import ops
    from gemm_gate_softmax_amd import workloads as W
    libs = [os.path.abspath(p) for p in args.ab.split(",") if p]
    for p in libs:
        if not os.path.exists(p):
            raise RuntimeError(f"{p} is missing")

    def use(path):
        ops._lib = None
        ops.LIB_PATH = path
        ops.lib()

    d = W.make_device(cfg, seed=args.seed, device=dev)
    use(libs[0])
    bufs = ops.alloc_layer_bufs(cfg.T, cfg.H, cfg.E, cfg.F, cfg.k, d["x"].dtype, dev,
                                fuse_dispatch=True)
    dtc = ops.dtype_code(d["x"].dtype)
    ws = gws = gate_ws = None
    for p in libs:                   # workspaces large enough for every variant
        use(p)
        w = ops.workspace(ops.MOE_WS_LAYER, cfg.T, cfg.H, cfg.E, cfg.F, cfg.k, dtc, dev)
        g = ops.workspace(ops.MOE_WS_GEMM, cfg.N, cfg.H, cfg.E, cfg.F, 1, dtc, dev)
        a = ops.workspace(ops.MOE_WS_GATE, cfg.T, cfg.H, cfg.E, cfg.F, cfg.k, dtc, dev)
        ws = w if ws is None or w.numel() > ws.numel() else ws
        gws = g if gws is None or g.numel() > gws.numel() else gws
        gate_ws = a if gate_ws is None or a.numel() > gate_ws.numel() else gate_ws
    out = torch.empty_like(d["x"])
    stream = torch.cuda.current_stream()
    layer = lambda: ops.moe_layer_forward(d["x"], d["wg"], d["bias"], d["w1"], d["w3"], d["w2"],
                                          cfg.k, out=out, bufs=bufs, ws=ws)
    up = lambda: ops.moe_grouped_gemm_swiglu(d["x"], bufs["offsets"], d["w1"], d["w3"], None,
                                             h=bufs["h"], ws=gws, token_ids=bufs["token_ids"])
    both = lambda: ops.moe_grouped_gemm_swiglu(d["x"], bufs["offsets"], d["w1"], d["w3"], d["w2"],
                                               h=bufs["h"], y=bufs["y"], ws=gws,
                                               token_ids=bufs["token_ids"])
    te = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=dev)
    tw = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=dev)
    gate = lambda: ops.moe_gate_topk(d["x"], d["wg"], d["bias"], cfg.k, top_experts=te,
                                     top_weights=tw, ws=gate_ws)
    ref, res = None, {p: {"layer": [], "up": [], "experts": [], "gate": []} for p in libs}
    agree = {}
    bwd = {"grads": None, "ws": None, "ref": None, "dout": None, "agree": {}}
    if args.ab_backward:
        gen = torch.Generator(device=dev)
        gen.manual_seed(args.seed + 1)
        bwd["dout"] = torch.randn((cfg.T, cfg.H), generator=gen, device=dev).to(d["x"].dtype)
        for p in libs:
            res[p]["backward"] = []

    def backward():
        bwd["grads"], bwd["ws"] = ops.moe_layer_backward(
            d["x"], d["wg"], d["bias"], d["w1"], d["w3"], d["w2"], cfg.k, bufs, bwd["dout"],
            grads=bwd["grads"], ws=bwd["ws"])
    for _ in range(max(1, args.ab_reps)):
        for p in libs:
            use(p)
            layer()
            torch.cuda.synchronize()
            got = {n: t.float().clone() for n, t in (("h", bufs["h"]), ("y", bufs["y"]), ("out", out))}
            if ref is None:
                ref = got
            if p not in agree:
                same = all(torch.equal(got[n], ref[n]) for n in got)
                err = max(float((got[n] - ref[n]).abs().max() / ref[n].abs().max()) for n in got)
                agree[p] = "bit-identical" if same else f"max-abs-rel {err:.2e}"
            if args.ab_backward and p not in bwd["agree"]:
                backward()                       # on this build's forward intermediates
                torch.cuda.synchronize()
                g = {n: t.clone() for n, t in bwd["grads"].items() if t is not None}
                if bwd["ref"] is None:
                    bwd["ref"] = g
                bwd["agree"][p] = "bit-identical" if all(
                    torch.equal(g[n], bwd["ref"][n]) for n in g) else "differs"
                del g
            for name, fn in (("layer", layer), ("up", up), ("experts", both), ("gate", gate)):
                fn()
                torch.cuda.synchronize()
                res[p][name].append(time_steps(fn, 10, stream)["median"])
            if args.ab_backward:
                layer()                          # the intermediates the backward reads
                backward()
                torch.cuda.synchronize()
                res[p]["backward"].append(time_steps(backward, 3, stream)["median"])
            log(f"ab {cfg.name} {os.path.basename(p)}: layer {res[p]['layer'][-1]:.3f} ms, up "
                f"{res[p]['up'][-1]:.3f} ms, both products {res[p]['experts'][-1]:.3f} ms, gate "
                f"{res[p]['gate'][-1] * 1e3:.1f} us")
    print(json.dumps({"ab": cfg.name, "libs": [
        {"lib": os.path.relpath(p, ROOT), "outputs_vs_first": agree[p],
         **({"gradients_vs_first": bwd["agree"][p]} if args.ab_backward else {}),
         **{f"{n}_ms_min": round(min(v), 4) for n, v in res[p].items()}} for p in libs]}),
        flush=True)
    return 0


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        log("bench.py: only --gpus 1 is supported (single-GPU layer forward)")
        return 2

    if args.calibrate_copy:
        return calibrate_copy()
    if args.memory_ceilings:
        return memory_ceilings(args)

    import torch

    from gemm_gate_softmax_amd import ops
    from gemm_gate_softmax_amd import workloads as W

    cfg = W.CONFIGS[args.config]
    dev = "cuda"
    ops.lib()                                   # the HIP library or nothing
    if args.weight_stream:
        return weight_stream(cfg, args, dev)
    if args.ab:
        return ab_compare(cfg, args, dev)
    if args.dense:
        return dense(args, dev)
    log(f"bench: {cfg.name} T={cfg.T} H={cfg.H} E={cfg.E} F={cfg.F} k={cfg.k} {cfg.dtype}: "
        "drawing inputs on the device")
    d = W.make_device(cfg, seed=args.seed, device=dev)
    bufs = ops.alloc_layer_bufs(cfg.T, cfg.H, cfg.E, cfg.F, cfg.k, d["x"].dtype, dev)
    bufs_f = ops.alloc_layer_bufs(cfg.T, cfg.H, cfg.E, cfg.F, cfg.k, d["x"].dtype, dev,
                                  fuse_dispatch=True)
    dtc = ops.dtype_code(d["x"].dtype)
    ws = ops.workspace(ops.MOE_WS_LAYER, cfg.T, cfg.H, cfg.E, cfg.F, cfg.k, dtc, dev)
    out = torch.empty_like(d["x"])
    stream = torch.cuda.current_stream()

    if args.up_kernel_only or args.expert_kernels_only:
        step_staged_once = lambda: ops.moe_layer_forward(
            d["x"], d["wg"], d["bias"], d["w1"], d["w3"], d["w2"], cfg.k, out=out, bufs=bufs, ws=ws)
        step_staged_once()
        gws0 = ops.workspace(ops.MOE_WS_GEMM, cfg.N, cfg.H, cfg.E, cfg.F, 1, dtc, dev)
        both = args.expert_kernels_only
        for _ in range(args.steps):     # the products as the layer runs them (dispatch fused)
            ops.moe_grouped_gemm_swiglu(d["x"], bufs["offsets"], d["w1"], d["w3"],
                                        d["w2"] if both else None, h=bufs["h"],
                                        y=bufs["y"] if both else None, ws=gws0,
                                        token_ids=bufs["token_ids"])
        torch.cuda.synchronize()
        print(json.dumps({"expert_kernels_only" if both else "up_kernel_only": args.steps,
                          "workload": cfg.name}), flush=True)
        return 0

    def step():          # the layer with the dispatch fused into the up product
        ops.moe_layer_forward(d["x"], d["wg"], d["bias"], d["w1"], d["w3"], d["w2"], cfg.k,
                              out=out, bufs=bufs_f, ws=ws)

    def step_staged():   # every stage its own kernel, xd written and read back
        ops.moe_layer_forward(d["x"], d["wg"], d["bias"], d["w1"], d["w3"], d["w2"], cfg.k,
                              out=out, bufs=bufs, ws=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    counts = W.to_host(bufs_f["counts"], None)
    log(f"bench: routing {W.routing_summary(counts)}; timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    steps_ms = time_steps(step, args.steps, stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ms_events = steps_ms["median"]
    # what the timed step produced, for the parity record
    out_host = W.to_host(out, cfg.dtype)
    te_host = W.to_host(bufs_f["top_experts"], None)
    tw_host = W.to_host(bufs_f["top_weights"], None)
    refined = int(W.to_host(ws[4:8].view(torch.int32), None)[0])

    step_staged()
    torch.cuda.synchronize()
    staged_ms = time_calls(step_staged, args.steps, stream)

    # The same step captured once into a HIP graph and replayed: no host-side launch work
    # per step (the library enqueues kernels only, no memsets or host reads, so a captured
    # layer replays as is).  Every replay's output is compared with the eager step's.
    graph_ms = None
    graph_ok = True
    try:
        out_ref = out.clone()
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        with torch.cuda.graph(g):
            step()
        reps = max(args.steps, 5)
        for _ in range(3):
            g.replay()
            torch.cuda.synchronize()
            graph_ok = graph_ok and torch.equal(out, out_ref)
        graph_ms = time_steps(g.replay, reps, stream)["median"]
        torch.cuda.synchronize()
        graph_ok = graph_ok and torch.equal(out, out_ref)
        del g
    except RuntimeError as exc:          # capture unsupported: report, do not fail the bench
        log(f"bench: graph capture skipped ({exc})")

    # Per-stage times: each entry point on its own, same buffers, same stream.
    N = cfg.N
    gws = ops.workspace(ops.MOE_WS_GEMM, N, cfg.H, cfg.E, cfg.F, 1, dtc, dev)
    pws = ops.workspace(ops.MOE_WS_PFT, cfg.T, cfg.H, cfg.E, cfg.F, cfg.k, dtc, dev)
    gtw = ops.workspace(ops.MOE_WS_GATE, cfg.T, cfg.H, cfg.E, cfg.F, cfg.k, dtc, dev)
    pft_out = {n: bufs[n] for n in ("counts", "offsets", "token_ids", "expert_ids", "dest_pos")}
    stages = {
        "gate": lambda: ops.moe_gate_topk(d["x"], d["wg"], d["bias"], cfg.k, bufs["top_experts"],
                                          bufs["top_weights"], ws=gtw),
        "buffers": lambda: ops.moe_pft_build(bufs["top_experts"], cfg.E, out=pft_out, ws=pws),
        "dispatch": lambda: ops.moe_dispatch(d["x"], bufs["dest_pos"], xd=bufs["xd"]),
        "grouped_gemm": lambda: ops.moe_grouped_gemm_swiglu(bufs["xd"], bufs["offsets"], d["w1"],
                                                            d["w3"], d["w2"], h=bufs["h"],
                                                            y=bufs["y"], ws=gws),
        "combine": lambda: ops.moe_combine(bufs["y"], bufs["dest_pos"], bufs["top_weights"],
                                           out=out),
    }
    st_ms = {}
    for name, fn in stages.items():
        fn()
        torch.cuda.synchronize()
        st_ms[name] = time_calls(fn, args.steps, stream)
    # The dominant kernel alone, as the timed step runs it: the gate/up product with the
    # dispatch fused (rows gathered from x through token_ids; tile table + one expert launch).
    up_call = lambda: ops.moe_grouped_gemm_swiglu(d["x"], bufs_f["offsets"], d["w1"], d["w3"],
                                                  None, h=bufs_f["h"], ws=gws,
                                                  token_ids=bufs_f["token_ids"])
    up_call()
    torch.cuda.synchronize()
    up_ms = time_calls(up_call, args.steps, stream)
    alg = algorithmic(cfg, counts)
    g_ms = st_ms["grouped_gemm"]
    tflops = alg["gemm_flops"] / (g_ms * 1e-3) / 1e12
    g_attain = min(MFMA_PEAK_TFLOPS[cfg.dtype],
                   alg["gemm_flops"] / alg["gemm_bytes"] * HBM_PEAK_GBS * 1e9 / 1e12)
    up_tflops = alg["up_flops"] / (up_ms * 1e-3) / 1e12
    up_gbs = alg["up_bytes"] / (up_ms * 1e-3) / 1e9
    peak = MFMA_PEAK_TFLOPS[cfg.dtype]
    # roofline bound of the up kernel: its arithmetic intensity against the ridge point
    intensity = alg["up_flops"] / alg["up_bytes"]
    ridge = peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    if intensity >= ridge:
        roof = {"bound": "mfma", "achieved": round(up_tflops, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(up_tflops / peak, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(up_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(up_gbs / HBM_PEAK_GBS, 4)}
    stage_report = {n: round(v * 1e3, 2) for n, v in st_ms.items()}
    # launch floor for the buffer build (three kernels: histogram, scan, scatter): the same
    # number of one-element fill kernels back to back on the same stream, timed the same way
    tiny = torch.zeros(1, dtype=torch.int32, device=dev)

    def chain3():
        tiny.fill_(0)
        tiny.fill_(1)
        tiny.fill_(2)
    chain3()
    torch.cuda.synchronize()
    floor_us = time_calls(chain3, args.steps, stream) * 1e3
    bw = {
        "dispatch_GBs": alg["dispatch_bytes"] / (st_ms["dispatch"] * 1e-3) / 1e9,
        "combine_GBs": alg["combine_bytes"] / (st_ms["combine"] * 1e-3) / 1e9,
        "grouped_gemm_GBs": alg["gemm_bytes"] / (g_ms * 1e-3) / 1e9,
    }
    bwd = None
    if not args.no_backward:
        # The layer backward after the fused forward (bufs_f): gradients of x, Wg, bias, W1,
        # W3 and W2 for a synthetic dout.  Its products: dh, the recomputed a and g, dxd and
        # three weight gradients, 16 N H F flops against the forward's 6 N H F.
        gen = torch.Generator(device=dev)
        gen.manual_seed(args.seed + 1)
        dout = torch.randn((cfg.T, cfg.H), generator=gen, device=dev).to(d["x"].dtype)
        step()
        grads, bws = ops.moe_layer_backward(d["x"], d["wg"], d["bias"], d["w1"], d["w3"],
                                            d["w2"], cfg.k, bufs_f, dout)
        torch.cuda.synchronize()
        bsteps = max(1, min(args.steps, 5))
        bwd_ms = time_calls(lambda: ops.moe_layer_backward(
            d["x"], d["wg"], d["bias"], d["w1"], d["w3"], d["w2"], cfg.k, bufs_f, dout,
            grads=grads, ws=bws), bsteps, stream)
        bflops = 16.0 * cfg.N * cfg.H * cfg.F
        # The same with the forward storing the up product's halves a and g (bufs a, g), so
        # the backward skips their recomputation; the forward that stores them is timed too.
        bufs_t = ops.alloc_layer_bufs(cfg.T, cfg.H, cfg.E, cfg.F, cfg.k, d["x"].dtype, dev,
                                      fuse_dispatch=True, store_ag=True)
        fwd_ag = lambda: ops.moe_layer_forward(d["x"], d["wg"], d["bias"], d["w1"], d["w3"],
                                               d["w2"], cfg.k, out=out, bufs=bufs_t, ws=ws)
        fwd_ag()
        torch.cuda.synchronize()
        fwd_ag_ms = time_calls(fwd_ag, bsteps, stream)
        bwd_ag_ms = time_calls(lambda: ops.moe_layer_backward(
            d["x"], d["wg"], d["bias"], d["w1"], d["w3"], d["w2"], cfg.k, bufs_t, dout,
            grads=grads, ws=bws), bsteps, stream)
        bwd = {"ms_per_step": round(bwd_ms, 3), "tokens_per_s": round(cfg.T / (bwd_ms * 1e-3), 1),
               "steps": bsteps, "tflops": round(bflops / (bwd_ms * 1e-3) / 1e12, 2),
               "workspace_GB": round(bws.numel() / 1e9, 2),
               "note": "moe_layer_backward after the fused forward: dx, dWg, dbias, dW1, dW3, dW2",
               "stored_ag": {"backward_ms": round(bwd_ag_ms, 3),
                             "forward_ms": round(fwd_ag_ms, 4),
                             "note": "forward storing a and g beside h; backward without "
                                     "their recomputation"}}
        del grads, bws, dout, bufs_t
        torch.cuda.empty_cache()
    if args.verbose:
        for n, v in st_ms.items():
            log(f"  {n:13s} {v * 1e3:9.1f} us")
        log(f"  up kernel     {up_ms * 1e3:9.1f} us  {up_tflops:.1f} TFLOP/s")
        log(f"  grouped GEMM {tflops:.1f} TFLOP/s = {100 * tflops / peak:.1f}% of {peak} "
            f"(weights+activations {bw['grouped_gemm_GBs']:.0f} GB/s); dispatch "
            f"{bw['dispatch_GBs']:.0f} GB/s, combine {bw['combine_GBs']:.0f} GB/s")

    rec = {
        "metric": METRIC if cfg.name == "xmoe_large" else METRIC.replace("X-MoE Large", cfg.name),
        "value": cfg.T / (ms_events * 1e-3), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_events,
        "step_ms": {k_: round(steps_ms[k_], 4) for k_ in ("median", "mean", "min", "max")},
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "E": cfg.E, "F": cfg.F,
                   "k": cfg.k, "gate_bias": None if cfg.bias is None else f"{cfg.bias[0]}({cfg.bias[1]})",
                   "seed": args.seed, "active_experts": alg["active_experts"],
                   "dispatch": "fused into the up product (bufs.xd = NULL)",
                   "parallelism": "single GPU"},
        "roofline": roof | {
            "traffic": recorded_traffic(cfg.name),
            "traffic_note": "bytes per launch the L2 exchanged with the memory fabric (FETCH_SIZE "
                            "+ WRITE_SIZE, scaled by a plain copy's reading): Infinity Cache hits "
                            "included, so an upper bound on HBM bytes; null once the kernel "
                            "sources differ from the profiled ones",
            "kernel": "expert_gemm_kernel, gate/up product + SwiGLU, dispatch fused (as in the timed step)",
            "per_launch": {"flop": alg["up_flops"], "bytes": alg["up_bytes"],
                           "us": round(up_ms * 1e3, 1), "flop_per_byte": round(intensity, 1),
                           "ridge_flop_per_byte": round(ridge, 1),
                           "tflops": round(up_tflops, 2), "frac_mfma": round(up_tflops / peak, 4),
                           "gbs": round(up_gbs, 1), "frac_hbm": round(up_gbs / HBM_PEAK_GBS, 4)},
            "source_sha256": kernel_digest()},
        "grouped_gemm": {"tflops": round(tflops, 2), "frac_mfma": round(tflops / peak, 4),
                         "us": round(g_ms * 1e3, 1),
                         # the roofline bound at its arithmetic intensity: min(peak, AI x HBM)
                         "attainable_tflops": round(g_attain, 1),
                         "frac_attainable": round(tflops / g_attain, 4)},
        "stages_us": stage_report | {"up_kernel": round(up_ms * 1e3, 2)},
        "buffers_vs_launch_floor": {"buffers_us": stage_report["buffers"],
                                    "floor_us": round(floor_us, 2), "kernels": 3,
                                    "ratio": round(stage_report["buffers"] / floor_us, 2)},
        "graph_replay": {"ms_per_step": None if graph_ms is None else round(graph_ms, 4),
                         "tokens_per_s": None if graph_ms is None else round(cfg.T / (graph_ms * 1e-3), 1),
                         "outputs_match_eager": graph_ok,
                         "note": "the fused step captured once in a HIP graph and replayed "
                                 "(median per replay): the step without host launch work"},
        "staged_layer": {"ms_per_step": round(staged_ms, 4),
                         "tokens_per_s": round(cfg.T / (staged_ms * 1e-3), 1),
                         "note": "dispatch as its own kernel (xd written and read back)"},
        "bandwidth": {k_: round(v, 1) for k_, v in bw.items()}
        | {"dispatch_frac_hbm": round(bw["dispatch_GBs"] / HBM_PEAK_GBS, 4),
           "combine_frac_hbm": round(bw["combine_GBs"] / HBM_PEAK_GBS, 4),
           "grouped_gemm_frac_hbm": round(bw["grouped_gemm_GBs"] / HBM_PEAK_GBS, 4)},
        "wall_ms_per_step": wall_ms,
    }
    if bwd is not None:
        rec["backward"] = bwd
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle on a bounded sample")
        rec["cpu_baseline"], rec["parity"] = cpu_baseline(cfg, d, args.seed, args.cpu_seconds,
                                                          out_host, te_host, tw_host, refined)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
