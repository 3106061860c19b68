"""Comparison helpers shared by the parity tests (host side, numpy only)."""
from __future__ import annotations

import numpy as np

from gemm_gate_softmax_amd import workloads as W

# Tolerances on floating-point layer outputs: max |gpu - oracle| / max |oracle| over the
# compared tensor (elementwise relative error is ill-posed at the many near-zero outputs).
TOL = {"f32": 1e-4, "bf16": 2e-2}
# Near-tie windows on the oracle's double logits, for the record only: a token whose
# adjacent gap among its k+1 largest logits is at most TIE_EXACT * max(1, |l|) is a near
# tie; the band up to TIE_ACC is counted separately.  Routing itself must agree with the
# oracle on every token: the gate re-decides near-tie tokens from exactly rounded logits.
TIE_EXACT, TIE_ACC = 1e-6, 1e-5
# Routing weights: w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0) moves by about |dl_j| + |dl_0|
# (relative) for logit errors dl.  fp32-accumulated logits over H <= 7168 terms differ from
# the double sums by a few 1e-6, so weights (all <= 1) are held to 2e-5 absolute.
WEIGHT_ATOL = 2e-5


def as_f64(a: np.ndarray, dt: str) -> np.ndarray:
    a = np.asarray(a)
    return (W.bf16_bits_to_f32(a) if dt == "bf16" else a).astype(np.float64)


def max_abs_rel(got, ref, dt) -> float:
    g, r = as_f64(got, dt), as_f64(ref, dt)
    if r.size == 0:
        return 0.0
    scale = float(np.max(np.abs(r)))
    return float(np.max(np.abs(g - r))) / (scale if scale > 0 else 1.0)


def rms_rel(got, ref, dt) -> float:
    g, r = as_f64(got, dt), as_f64(ref, dt)
    den = float(np.sqrt(np.mean(r * r))) or 1.0
    return float(np.sqrt(np.mean((g - r) ** 2))) / den


def tie_bands(l64: np.ndarray, k: int):
    """Per token: (gap <= TIE_EXACT, TIE_EXACT < gap <= TIE_ACC) over the k+1 largest logits."""
    T, E = l64.shape
    m = min(k + 1, E)
    top = -np.sort(-l64, axis=1)[:, :m]
    gaps = (top[:, :-1] - top[:, 1:]) / np.maximum(1.0, np.abs(top[:, :-1]))
    g = gaps.min(axis=1) if m > 1 else np.full(T, np.inf)
    return g <= TIE_EXACT, (g > TIE_EXACT) & (g <= TIE_ACC)


def compare_routing(te_gpu, te_ref, l64, k):
    """Returns dict(mismatch, near_tie, band): tokens whose picks differ from the oracle's
    (must be none), and the counts of near-tie tokens in the two windows."""
    diff = np.any(np.asarray(te_gpu) != np.asarray(te_ref), axis=1)
    exact, acc = tie_bands(l64, k)
    return dict(mismatch=np.flatnonzero(diff), near_tie=int(exact.sum()), band=int(acc.sum()))


def routing_note(r, refined=None):
    s = (f"routing mismatches {len(r['mismatch'])}; near-tie tokens (gap <= {TIE_EXACT:g}) "
         f"{r['near_tie']}, band ({TIE_EXACT:g}, {TIE_ACC:g}] {r['band']}")
    return s if refined is None else s + f"; tokens re-decided from exact logits {refined}"


def skewed_routing(rng, T, k, E, alpha=1.0, empty_every=0):
    """Distinct top-k expert ids per token drawn without replacement from p_e ~ (e+1)^-alpha
    (Gumbel top-k), optionally never choosing every `empty_every`-th expert."""
    logp = -alpha * np.log(np.arange(1, E + 1, dtype=np.float64))
    if empty_every:
        logp[1::empty_every] = -np.inf
    keys = logp[None, :] + rng.gumbel(size=(T, E))
    return np.argsort(-keys, axis=1)[:, :k].astype(np.int32)
