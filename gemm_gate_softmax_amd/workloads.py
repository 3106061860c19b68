"""Synthetic workloads: the layer shapes and a seeded input generator.

This module only draws inputs.  It holds none of the layer's arithmetic, and both the HIP
path and the CPU oracle are fed from it.

Shapes.  The three X-MoE rows come from the model-configuration table of the X-MoE review
(section 五, 模型配置: Small H=2048/F=1408/E=64/top-6, Medium H=5120/F=1536/E=128/top-6,
Large H=7168/F=2048/E=256/top-8, with T = 4 x 2048 tokens for Small and 4096 for the others).
The two fp32 rows are a tiny case and one device's share of a top-2 layer in the FlashDMoE
setting (section 6 of that blog: k = 2, synthetic inputs, fp32 evaluation per section 8).

Draws.  Each tensor has its own stream ``numpy.random.default_rng(SeedSequence([seed, id,
chunk]))`` with ids x=0, Wg=1, W1=2, W3=3, W2=4, bias=5 (weights are chunked per expert).
x ~ N(0,1); Wg, W1, W3 ~ N(0, 1/H); W2 ~ N(0, 1/F), drawn in float64, cast to float32 and,
for bf16 layers, rounded to bf16 (nearest, ties to even).  For the large layers the expert
weights can instead be drawn on the device with torch's generator (``make_device``), seeded
from the same (seed, id); the oracle then reads back the bytes it needs.

Gate bias.  ``("zipf", a)``: draw d_e i.i.d. from the finite Zipf law P(r) ~ r^-a on
r in {1..E} and standardise to mean 0, std 1 (population std).  ``None``: no bias.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

X_ID, WG_ID, W1_ID, W3_ID, W2_ID, BIAS_ID = 0, 1, 2, 3, 4, 5


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    H: int
    E: int
    F: int
    k: int
    dtype: str                 # "f32" or "bf16": storage type of x, weights, h, y, out
    bias: tuple | None = None  # None or ("zipf", alpha)

    @property
    def N(self) -> int:
        return self.T * self.k

    def scaled(self, **kw) -> "LayerConfig":
        d = dict(self.__dict__)
        d.update(kw)
        return LayerConfig(**d)


CONFIGS = {
    "tiny_f32": LayerConfig("tiny_f32", T=256, H=256, E=8, F=128, k=2, dtype="f32"),
    "top2_f32": LayerConfig("top2_f32", T=4096, H=2048, E=64, F=2048, k=2, dtype="f32"),
    "xmoe_small": LayerConfig("xmoe_small", T=8192, H=2048, E=64, F=1408, k=6, dtype="bf16",
                              bias=("zipf", 1.0)),
    "xmoe_medium": LayerConfig("xmoe_medium", T=4096, H=5120, E=128, F=1536, k=6,
                               dtype="bf16"),
    "xmoe_large": LayerConfig("xmoe_large", T=4096, H=7168, E=256, F=2048, k=8, dtype="bf16",
                              bias=("zipf", 1.2)),
    # X-MoE review, 模型配置 table, "Super" row (seq 4096, H 7168, FFN 2560, 256 experts,
    # top-8); no routing skew is given for it, so the Large row's Zipf(1.2) gate bias is
    # reused.  Not one of the benchmark configurations: a parity case at a wider F.
    "xmoe_super": LayerConfig("xmoe_super", T=4096, H=7168, E=256, F=2560, k=8, dtype="bf16",
                              bias=("zipf", 1.2)),
}


def _rng(seed: int, tensor_id: int, chunk: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, tensor_id, chunk]))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, nearest with ties to even (torch's CPU conversion)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _store(a64: np.ndarray, dtype: str) -> np.ndarray:
    a32 = a64.astype(np.float32)
    return a32 if dtype == "f32" else f32_to_bf16_bits(a32)


def normal(seed, tensor_id, shape, std, dtype, chunk=0) -> np.ndarray:
    return _store(_rng(seed, tensor_id, chunk).standard_normal(shape) * std, dtype)


def gate_bias(cfg: LayerConfig, seed: int) -> np.ndarray | None:
    if cfg.bias is None:
        return None
    law, alpha = cfg.bias
    if law != "zipf":
        raise ValueError(f"unknown bias law {law!r}")
    r = np.arange(1, cfg.E + 1, dtype=np.float64)
    p = r ** (-float(alpha))
    p /= p.sum()
    d = _rng(seed, BIAS_ID).choice(r, size=cfg.E, p=p)
    sd = d.std()
    b = (d - d.mean()) / (sd if sd > 0 else 1.0)
    return b.astype(np.float32)


def make_gate_inputs(cfg: LayerConfig, seed: int = 0) -> dict:
    """x [T,H], wg [E,H] (storage dtype; bf16 as uint16 bits) and bias [E] f32 or None."""
    return dict(x=normal(seed, X_ID, (cfg.T, cfg.H), 1.0, cfg.dtype),
                wg=normal(seed, WG_ID, (cfg.E, cfg.H), cfg.H ** -0.5, cfg.dtype),
                bias=gate_bias(cfg, seed))


def expert_weights_host(cfg: LayerConfig, seed: int, e: int) -> tuple:
    """Host draw of expert e: (W1[e] [F,H], W3[e] [F,H], W2[e] [H,F])."""
    return (normal(seed, W1_ID, (cfg.F, cfg.H), cfg.H ** -0.5, cfg.dtype, chunk=e),
            normal(seed, W3_ID, (cfg.F, cfg.H), cfg.H ** -0.5, cfg.dtype, chunk=e),
            normal(seed, W2_ID, (cfg.H, cfg.F), cfg.F ** -0.5, cfg.dtype, chunk=e))


def make_host(cfg: LayerConfig, seed: int = 0) -> dict:
    """All inputs on the host (small shapes)."""
    d = make_gate_inputs(cfg, seed)
    ws = [expert_weights_host(cfg, seed, e) for e in range(cfg.E)]
    d["w1"] = np.stack([w[0] for w in ws])
    d["w3"] = np.stack([w[1] for w in ws])
    d["w2"] = np.stack([w[2] for w in ws])
    return d


def torch_dtype(dtype: str):
    import torch
    return torch.float32 if dtype == "f32" else torch.bfloat16


def to_device(a: np.ndarray | None, dtype: str | None, device):
    """Host array (bf16 as uint16 bits when dtype == 'bf16') -> device tensor."""
    import torch
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        t = t.view(torch.bfloat16)
    return t.to(device)


def to_host(t, dtype: str | None) -> np.ndarray:
    """Device tensor -> host array (bf16 -> uint16 bits)."""
    import torch
    t = t.detach().contiguous().cpu()
    if dtype == "bf16" or t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _device_seed(seed: int, tensor_id: int) -> int:
    s = np.random.SeedSequence([seed, tensor_id]).generate_state(1, np.uint64)[0]
    return int(s) & ((1 << 63) - 1)


def make_device(cfg: LayerConfig, seed: int = 0, device="cuda", host_weights=None) -> dict:
    """Inputs resident on the device.

    x, wg and bias are drawn on the host (as in ``make_gate_inputs``) and copied.  Expert
    weights are drawn on the host when ``host_weights`` is True (default for small
    shapes), else on the device with torch's generator seeded from (seed, tensor id).
    """
    import torch
    if host_weights is None:
        host_weights = cfg.E * cfg.F * cfg.H <= (1 << 24)
    g = make_gate_inputs(cfg, seed)
    d = dict(x=to_device(g["x"], cfg.dtype, device), wg=to_device(g["wg"], cfg.dtype, device),
             bias=to_device(g["bias"], None, device))
    if host_weights:
        h = make_host(cfg, seed)
        for n in ("w1", "w3", "w2"):
            d[n] = to_device(h[n], cfg.dtype, device)
        return d
    tdt = torch_dtype(cfg.dtype)
    for n, tid, shape, std in (("w1", W1_ID, (cfg.F, cfg.H), cfg.H ** -0.5),
                               ("w3", W3_ID, (cfg.F, cfg.H), cfg.H ** -0.5),
                               ("w2", W2_ID, (cfg.H, cfg.F), cfg.F ** -0.5)):
        gen = torch.Generator(device=device)
        gen.manual_seed(_device_seed(seed, tid))
        w = torch.empty((cfg.E,) + shape, dtype=tdt, device=device)
        for e in range(cfg.E):
            w[e].copy_(torch.randn(shape, generator=gen, device=device,
                                   dtype=torch.float32).mul_(std))
        d[n] = w
    return d


def routing_summary(counts: np.ndarray) -> dict:
    c = np.asarray(counts)
    return dict(active=int((c > 0).sum()), empty=int((c == 0).sum()), max=int(c.max()),
                mean=float(c.mean()), min=int(c.min()))
