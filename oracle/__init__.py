"""CPU oracle for the MoE layer forward and backward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import this package.  The product path (``gemm_gate_softmax_amd``) never imports it
and shares no code with it; the C source ``oracle.c`` is compiled on its own with gcc.

Every wrapper takes and returns host numpy arrays.  bf16 tensors travel as ``uint16``
bit patterns.  The arithmetic lives in ``oracle.c`` (double accumulation, rounding only at
storage points); see that file's header for the passages each function follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1
_DT = {"f32": F32, "bf16": BF16}
_ERR = {1: "invalid argument", 2: "index out of range", 3: "out of memory"}


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc (plain C, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
                        "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    """The compiled oracle.  ``ORACLE_LIB`` names a separately compiled copy to load instead
    (the mutation tests point it at deliberately broken builds of this source)."""
    global _lib
    if _lib is None:
        path = os.environ.get("ORACLE_LIB")
        if path is None:
            path = _LIB
            if not os.path.exists(path):
                build()
        L = ctypes.CDLL(path)
        vp, i32, lng = ctypes.c_void_p, ctypes.c_int, ctypes.c_long
        L.oracle_gate_topk.argtypes = [i32] * 6 + [vp] * 7
        L.oracle_pft_build.argtypes = [i32] * 3 + [vp] * 6
        L.oracle_dispatch.argtypes = [i32] * 4 + [vp] * 3
        L.oracle_grouped_gemm_swiglu.argtypes = [i32] * 5 + [vp] * 7
        L.oracle_combine.argtypes = [i32] * 4 + [vp] * 4
        L.oracle_layer_forward.argtypes = [i32] * 7 + [vp] * 8
        L.oracle_combine_backward.argtypes = [i32] * 4 + [vp] * 6
        L.oracle_expert_backward.argtypes = [i32] * 5 + [vp] * 11
        L.oracle_dispatch_backward.argtypes = [i32] * 3 + [vp] * 3
        L.oracle_gate_backward.argtypes = [i32] * 6 + [vp] * 9
        L.oracle_layer_backward.argtypes = [i32] * 7 + [vp] * 14
        L.oracle_round_bf16.argtypes = [vp, vp, lng]
        L.oracle_num_threads.argtypes = []
        for f in ("oracle_gate_topk", "oracle_pft_build", "oracle_dispatch",
                  "oracle_grouped_gemm_swiglu", "oracle_combine", "oracle_layer_forward",
                  "oracle_combine_backward", "oracle_expert_backward",
                  "oracle_dispatch_backward", "oracle_gate_backward", "oracle_layer_backward",
                  "oracle_num_threads"):
            getattr(L, f).restype = ctypes.c_int
        L.oracle_round_bf16.restype = None
        _lib = L
    return _lib


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what}: {_ERR.get(rc, rc)}")


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _storage(dt):
    return np.float32 if dt == "f32" else np.uint16


def num_threads() -> int:
    return lib().oracle_num_threads()


def round_bf16(v: np.ndarray) -> np.ndarray:
    v = _c(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().oracle_round_bf16(_p(v), _p(out), v.size)
    return out


ROUTING = {"softmax": 0, "sigmoid": 1}


def gate_topk(dt, x, wg, bias, k, want_logits=False, routing="softmax"):
    """Returns (top_experts [T,k] i32, top_weights [T,k] f32[, logits f32, logits f64])."""
    st = _storage(dt)
    x, wg = _c(x, st), _c(wg, st)
    T, H = x.shape
    E = wg.shape[0]
    b = None if bias is None else _c(bias, np.float32)
    te = np.empty((T, k), np.int32)
    tw = np.empty((T, k), np.float32)
    l32 = np.empty((T, E), np.float32) if want_logits else None
    l64 = np.empty((T, E), np.float64) if want_logits else None
    _check(lib().oracle_gate_topk(_DT[dt], T, H, E, k, ROUTING[routing], _p(x), _p(wg), _p(b),
                                  _p(te), _p(tw), _p(l32), _p(l64)), "gate_topk")
    return (te, tw, l32, l64) if want_logits else (te, tw)


def pft_build(top_experts, E):
    """Returns dict(counts, offsets, token_ids, expert_ids, dest_pos)."""
    te = _c(top_experts, np.int32)
    T, k = te.shape
    N = T * k
    out = dict(counts=np.empty(E, np.int32), offsets=np.empty(E + 1, np.int32),
               token_ids=np.empty(N, np.int32), expert_ids=np.empty(N, np.int32),
               dest_pos=np.empty((T, k), np.int32))
    _check(lib().oracle_pft_build(T, k, E, _p(te), _p(out["counts"]), _p(out["offsets"]),
                                  _p(out["token_ids"]), _p(out["expert_ids"]),
                                  _p(out["dest_pos"])), "pft_build")
    return out


def dispatch(dt, x, dest_pos):
    st = _storage(dt)
    x = _c(x, st)
    dp = _c(dest_pos, np.int32)
    T, H = x.shape
    k = dp.shape[1]
    xd = np.empty((T * k, H), st)
    _check(lib().oracle_dispatch(_DT[dt], T, k, H, _p(x), _p(dp), _p(xd)), "dispatch")
    return xd


def grouped_gemm_swiglu(dt, xd, offsets, w1, w3, w2, want_h=True):
    """Returns (h [N,F], y [N,H]) in storage type (h is None when want_h is False)."""
    st = _storage(dt)
    xd = _c(xd, st)
    off = _c(offsets, np.int32)
    w1, w3, w2 = _c(w1, st), _c(w3, st), _c(w2, st)
    N, H = xd.shape
    E, F = w1.shape[0], w1.shape[1]
    h = np.empty((N, F), st) if want_h else None
    y = np.empty((N, H), st)
    _check(lib().oracle_grouped_gemm_swiglu(_DT[dt], N, E, H, F, _p(xd), _p(off), _p(w1),
                                            _p(w3), _p(w2), _p(h), _p(y)), "grouped_gemm")
    return h, y


def combine(dt, y, dest_pos, top_weights):
    st = _storage(dt)
    y = _c(y, st)
    dp = _c(dest_pos, np.int32)
    tw = _c(top_weights, np.float32)
    T, k = dp.shape
    H = y.shape[1]
    out = np.empty((T, H), st)
    _check(lib().oracle_combine(_DT[dt], T, k, H, _p(y), _p(dp), _p(tw), _p(out)), "combine")
    return out


def layer_forward(dt, x, wg, bias, w1, w3, w2, k, stage_seconds=False, routing="softmax"):
    st = _storage(dt)
    x, wg = _c(x, st), _c(wg, st)
    w1, w3, w2 = _c(w1, st), _c(w3, st), _c(w2, st)
    b = None if bias is None else _c(bias, np.float32)
    T, H = x.shape
    E, F = w1.shape[0], w1.shape[1]
    out = np.empty((T, H), st)
    secs = np.zeros(5, np.float64)
    _check(lib().oracle_layer_forward(_DT[dt], T, H, E, F, k, ROUTING[routing], _p(x), _p(wg),
                                      _p(b), _p(w1), _p(w3), _p(w2), _p(out), _p(secs)),
           "layer_forward")
    return (out, secs) if stage_seconds else out


# ----------------------------------------------------------------------------- backward
# Gradients (double) of the loss sum(dout * out) with the expert picks held fixed; see the
# backward section of oracle.c for the formulas and the readings behind them.

def combine_backward(dt, dout, y, dest_pos, top_weights):
    """Returns (dy [N,H] f64, dw [T,k] f64)."""
    st = _storage(dt)
    dout, y = _c(dout, st), _c(y, st)
    dp = _c(dest_pos, np.int32)
    tw = _c(top_weights, np.float32)
    T, k = dp.shape
    H = y.shape[1]
    dy = np.empty((T * k, H), np.float64)
    dw = np.empty((T, k), np.float64)
    _check(lib().oracle_combine_backward(_DT[dt], T, k, H, _p(dout), _p(y), _p(dp), _p(tw),
                                         _p(dy), _p(dw)), "combine_backward")
    return dy, dw


def expert_backward(dt, xd, offsets, w1, w3, w2, dy, h=None):
    """Returns dict(dxd [N,H], dw1 [E,F,H], dw3 [E,F,H], dw2 [E,H,F]), all f64."""
    st = _storage(dt)
    xd = _c(xd, st)
    off = _c(offsets, np.int32)
    w1, w3, w2 = _c(w1, st), _c(w3, st), _c(w2, st)
    h = None if h is None else _c(h, st)
    dy = _c(dy, np.float64)
    N, H = xd.shape
    E, F = w1.shape[0], w1.shape[1]
    out = dict(dxd=np.empty((N, H)), dw1=np.empty((E, F, H)), dw3=np.empty((E, F, H)),
               dw2=np.empty((E, H, F)))
    _check(lib().oracle_expert_backward(_DT[dt], N, E, H, F, _p(xd), _p(off), _p(w1), _p(w3),
                                        _p(w2), _p(h), _p(dy), _p(out["dxd"]), _p(out["dw1"]),
                                        _p(out["dw3"]), _p(out["dw2"])), "expert_backward")
    return out


def dispatch_backward(dxd, dest_pos):
    """Returns dx [T,H] f64: the sum of each token's k buffer-row gradients."""
    dxd = _c(dxd, np.float64)
    dp = _c(dest_pos, np.int32)
    T, k = dp.shape
    H = dxd.shape[1]
    dx = np.empty((T, H), np.float64)
    _check(lib().oracle_dispatch_backward(T, k, H, _p(dxd), _p(dp), _p(dx)), "dispatch_backward")
    return dx


def gate_backward(dt, x, wg, bias, top_experts, dw, routing="softmax", dx=None):
    """Returns dict(dx [T,H] (dx + the gate's part when dx is given), dwg [E,H], dbias [E],
    dl [T,k]), all f64."""
    st = _storage(dt)
    x, wg = _c(x, st), _c(wg, st)
    b = None if bias is None else _c(bias, np.float32)
    te = _c(top_experts, np.int32)
    dw = _c(dw, np.float64)
    T, H = x.shape
    E = wg.shape[0]
    k = te.shape[1]
    out = dict(dx=np.zeros((T, H)) if dx is None else np.array(dx, np.float64, copy=True),
               dwg=np.empty((E, H)), dbias=np.empty(E), dl=np.empty((T, k)))
    _check(lib().oracle_gate_backward(_DT[dt], T, H, E, k, ROUTING[routing], _p(x), _p(wg), _p(b),
                                      _p(te), _p(dw), _p(out["dx"]), _p(out["dwg"]),
                                      _p(out["dbias"]), _p(out["dl"])), "gate_backward")
    return out


def layer_backward(dt, x, wg, bias, w1, w3, w2, k, dout, routing="softmax"):
    """Returns dict(dx, dwg, dbias, dw1, dw3, dw2, dtw), all f64."""
    st = _storage(dt)
    x, wg, dout = _c(x, st), _c(wg, st), _c(dout, st)
    w1, w3, w2 = _c(w1, st), _c(w3, st), _c(w2, st)
    b = None if bias is None else _c(bias, np.float32)
    T, H = x.shape
    E, F = w1.shape[0], w1.shape[1]
    out = dict(dx=np.empty((T, H)), dwg=np.empty((E, H)), dbias=np.empty(E),
               dw1=np.empty((E, F, H)), dw3=np.empty((E, F, H)), dw2=np.empty((E, H, F)),
               dtw=np.empty((T, k)))
    _check(lib().oracle_layer_backward(_DT[dt], T, H, E, F, k, ROUTING[routing], _p(x), _p(wg),
                                       _p(b), _p(w1), _p(w3), _p(w2), _p(dout), _p(out["dx"]),
                                       _p(out["dwg"]), _p(out["dbias"]), _p(out["dw1"]),
                                       _p(out["dw3"]), _p(out["dw2"]), _p(out["dtw"])),
           "layer_backward")
    return out
