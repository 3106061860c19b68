"""A CPU model of the L2 misses of the grouped expert products (analysis only).

The up product at X-MoE Large runs at the memory fabric's cap, so its time follows the bytes
that miss the L2s.  This model replays a launch's tiles the way ``expert_gemm_kernel`` orders
them (the two tile lists, each XCD's contiguous share of both interleaved evenly, large
experts' token tiles in blocks with the feature tile slowest, the up product's K rotation
keyed on the tile's position) on 8 XCDs of 32 CUs each.  Every CU runs one tile at a time and steps
through its k-slices at a fixed rate (a per-tile factor drawn from [1 - jitter, 1 + jitter]
stands in for the spread of real tile times); each k-slice requests its operand blocks
(one 16-byte-per-lane slice of the activation rows, one of each weight operand) from the
XCD's L2, an LRU of 4 MiB over those blocks.  Small-expert weights carry the non-temporal
hint and do not allocate.  Activation rows shared by two experts' tiles are counted twice.

``python -m gemm_gate_softmax_amd.l2_model`` prints the kept schedule and the alternatives
that were weighed, for the X-MoE Large routing of seed 0.  The routing comes from double
logits on the host (ties resolved to the lower expert id), which matches the layer's
routing up to the few near-tie tokens.
"""
from __future__ import annotations

import argparse
import heapq
from collections import OrderedDict

import numpy as np

L2_BYTES = 4 << 20            # per XCD
XCDS, CUS_PER_XCD = 8, 32
ROW_BYTES = 128               # bytes of K per row and k-slice


def routing_counts(cfg, seed: int = 0) -> np.ndarray:
    """Rows per expert of a workload's routing, from double logits on the host."""
    from gemm_gate_softmax_amd import workloads as W
    g = W.make_gate_inputs(cfg, seed)
    x, wg = g["x"], g["wg"]
    if cfg.dtype == "bf16":
        x, wg = W.bf16_bits_to_f32(x), W.bf16_bits_to_f32(wg)
    logits = x.astype(np.float64) @ wg.astype(np.float64).T
    if g["bias"] is not None:
        logits += g["bias"].astype(np.float64)
    top = np.argsort(-logits, axis=1, kind="stable")[:, :cfg.k]
    return np.bincount(top.ravel(), minlength=cfg.E)


def tile_lists(counts, bt: int, feat_tiles: int, group: int, small: int = 64):
    """(large, small) lists of (expert, token tile, feature tile, rows) in launch order."""
    large, smalls = [], []
    for e, c in enumerate(int(v) for v in counts):
        if c > small:
            n_e = (c + bt - 1) // bt
            for q in range(n_e * feat_tiles):
                blk = min(q // (group * feat_tiles), (n_e - 1) // group)
                width = min(group, n_e - blk * group)
                ql = q - blk * group * feat_tiles
                ftile = ql // width
                ttile = blk * group + (ql - ftile * width)
                large.append((e, ttile, ftile, min(bt, c - ttile * bt)))
        elif c > 0:
            smalls.extend((e, 0, f, c) for f in range(feat_tiles))
    return large, smalls


def xcd_orders(large, smalls):
    """Each XCD's tiles in dispatch order: a contiguous share of each list, interleaved."""
    tot_m, tot_s = len(large), len(smalls)
    chunk_m, chunk_s = (tot_m + XCDS - 1) // XCDS, (tot_s + XCDS - 1) // XCDS
    orders = []
    for x in range(XCDS):
        m_x = max(0, min(chunk_m, tot_m - x * chunk_m))
        s_x = max(0, min(chunk_s, tot_s - x * chunk_s))
        n_x = m_x + s_x
        seq = []
        for j in range(n_x):
            a0, a1 = j * m_x // n_x, (j + 1) * m_x // n_x
            if a1 > a0:
                seq.append((True,) + large[x * chunk_m + a0])
            else:
                seq.append((False,) + smalls[x * chunk_s + (j - a0)])
        orders.append(seq)
    return orders


def simulate(counts, *, n_feat: int, nk: int, nb: int = 2, bt: int = 128, bf: int = 128,
             group: int = 32, rotate: bool = True, rot_period: int = 32, feat_unit: int = 128,
             rot_key: str = "pos",
             t_large: float = 1.0, t_small: float = 1.0, prologue: float = 4.2,
             epilogue: float = 2.3, jitter: float = 0.0, seed: int = 0,
             l2_bytes: int = L2_BYTES) -> tuple[int, int]:
    """(bytes missing the L2s, bytes requested) over one launch.  Times are in k-slices of
    a large tile.  rot_key: the rotation's key, "pos" (rb + w fb, w the expert's 128-row
    blocks capped at 32, as the kernel), "pos7" (rb + 7 fb), "rb" (token block only) or "fb"
    (feature block only)."""
    rng = np.random.default_rng(seed)
    feat_tiles = (n_feat + bf - 1) // bf
    large, smalls = tile_lists(counts, bt, feat_tiles, group)
    rot_on = rotate and len(smalls) > 0
    w_bytes = bf * ROW_BYTES
    miss = req = 0
    for seq in xcd_orders(large, smalls):
        lru: OrderedDict = OrderedDict()
        held = 0
        nxt = 0
        heap = []

        def start(cu, t):
            nonlocal nxt
            if nxt >= len(seq):
                return
            is_large, e, tt, ft, rows = seq[nxt]
            nxt += 1
            rot = 0
            if is_large and rot_on:
                rblk, fblk = tt * bt // 128, ft * bf // feat_unit
                wdt = min((int(counts[e]) + 127) // 128, 32)
                key = {"pos": rblk + wdt * fblk, "pos7": rblk + 7 * fblk, "rb": rblk,
                       "fb": wdt * fblk}[rot_key]
                rot = (key % rot_period) * nk // rot_period
            f = 1.0 + jitter * (2.0 * rng.random() - 1.0)
            heapq.heappush(heap, (t + prologue * f, cu, is_large, e, tt, ft, rows, 0, rot, f))

        for cu in range(CUS_PER_XCD):
            start(cu, 0.0)
        while heap:
            t, cu, is_large, e, tt, ft, rows, step, rot, f = heapq.heappop(heap)
            k = (step + rot) % nk
            blocks = [(("x", e, tt, k), min(rows, bt) * ROW_BYTES, True)]
            blocks += [(("w", b, e, ft, k), w_bytes, is_large) for b in range(nb)]
            for key, nbytes, allocate in blocks:
                req += nbytes
                if key in lru:
                    lru.move_to_end(key)
                    continue
                miss += nbytes
                if allocate:
                    lru[key] = nbytes
                    held += nbytes
                    while held > l2_bytes:
                        held -= lru.popitem(last=False)[1]
            step += 1
            dt = (t_large if is_large else t_small) * f
            if step < nk:
                heapq.heappush(heap, (t + dt, cu, is_large, e, tt, ft, rows, step, rot, f))
            else:
                start(cu, t + dt + epilogue * f)
    return miss, req


def variants(cfg):
    """The kept schedule of each product and the alternatives weighed against it."""
    up = dict(n_feat=cfg.F, nk=cfg.H * 2 // ROW_BYTES)
    down = dict(n_feat=cfg.H, nk=cfg.F * 2 // ROW_BYTES, nb=1, bf=256, feat_unit=256,
                rotate=False)
    return [
        ("up, kept: 128 x (2 x 128), blocks of 32, rotation", up),
        ("up, no K rotation", dict(up, rotate=False)),
        ("up, rotation step 7 in the feature direction", dict(up, rot_key="pos7")),
        ("up, rotation keyed on the token block", dict(up, rot_key="rb")),
        ("up, rotation keyed on the feature block", dict(up, rot_key="fb")),
        ("up, rotation period 16", dict(up, rot_period=16)),
        ("up, rotation period 64", dict(up, rot_period=64)),
        ("up, blocks of 8 token tiles", dict(up, group=8)),
        ("up, blocks of 16 token tiles", dict(up, group=16)),
        ("up, 128 x (2 x 256) tiles", dict(up, bf=256, t_large=2.0, t_small=1.8)),
        ("up, 256 x (2 x 128) tiles", dict(up, bt=256, t_large=2.0)),
        ("down, kept: 128 x 256, blocks of 32, no rotation", down),
        ("down, K rotation", dict(down, rotate=True)),
    ]


def main(argv=None):
    from gemm_gate_softmax_amd import workloads as W
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", default="xmoe_large")
    ap.add_argument("--seed", type=int, default=0)
    args = ap.parse_args(argv)
    cfg = W.CONFIGS[args.config]
    counts = routing_counts(cfg, args.seed)
    print(f"| schedule ({cfg.name}, seed {args.seed}) | requested GB | missed GB, jitter 0 / 0.1 / "
          "0.25 |")
    print("|---|---|---|")
    for label, kw in variants(cfg):
        out = [simulate(counts, jitter=j, **kw) for j in (0.0, 0.1, 0.25)]
        print(f"| {label} | {out[0][1] / 1e9:.2f} | "
              + " / ".join(f"{m / 1e9:.2f}" for m, _ in out) + " |", flush=True)


if __name__ == "__main__":
    main()
