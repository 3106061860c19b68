"""ctypes binding over libmoe.so: argument marshalling only.

Each function has the name of the C entry point it calls (declared in ``include/moe.h``),
takes torch tensors resident on the GPU, checks their dtype, shape and contiguity, passes
raw device pointers and the current HIP stream, and raises ``MoeError`` on a non-OK status.
Output tensors are allocated with torch when the caller does not pass them.  All compute
happens in the library's HIP kernels; there is no fallback of any kind: if ``libmoe.so``
is missing or cannot be loaded the first call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_F32, MOE_BF16 = 0, 1
MOE_WS_GATE, MOE_WS_PFT, MOE_WS_GEMM, MOE_WS_LAYER, MOE_WS_BACKWARD = 0, 1, 2, 3, 4
STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_VALUE", 2: "MOE_ERR_UNSUPPORTED",
          3: "MOE_ERR_MISALIGNED", 4: "MOE_ERR_WORKSPACE_TOO_SMALL", 5: "MOE_ERR_LAUNCH",
          6: "MOE_ERR_SCRATCH_TOO_SMALL"}
MOE_NOALLOC_SCRATCH_BYTES = 32 << 20

ROUTING = {"softmax": 0, "sigmoid": 1}   # moe_routing_t
EXPORTS = ("moe_workspace_bytes", "moe_status_string", "moe_gate_topk", "moe_pft_build",
           "moe_dispatch", "moe_grouped_gemm_swiglu", "moe_combine", "moe_layer_forward",
           "moe_layer_forward_noalloc", "moe_layer_backward")


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {moe_status_string(status)}")
        self.status = status


class LayerBufs(ctypes.Structure):
    """Mirror of ``moe_layer_bufs``."""
    _fields_ = [(n, ctypes.c_void_p) for n in ("top_experts", "top_weights", "counts", "offsets",
                                               "token_ids", "expert_ids", "dest_pos", "xd", "h",
                                               "y", "a", "g")]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m gemm_gate_softmax_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.moe_workspace_bytes.argtypes = [i32] * 7
        L.moe_workspace_bytes.restype = sz
        L.moe_status_string.argtypes = [i32]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_gate_topk.argtypes = [i32] * 6 + [vp] * 6 + [sz, vp]
        L.moe_pft_build.argtypes = [i32] * 3 + [vp] * 7 + [sz, vp]
        L.moe_dispatch.argtypes = [i32] * 4 + [vp] * 4
        L.moe_grouped_gemm_swiglu.argtypes = [i32] * 5 + [vp] * 2 + [i32] + [vp] * 7 + [sz, vp]
        L.moe_combine.argtypes = [i32] * 4 + [vp] * 5
        L.moe_layer_forward.argtypes = ([i32] * 7 + [vp] * 7 + [ctypes.POINTER(LayerBufs), vp, sz, vp])
        L.moe_layer_forward_noalloc.argtypes = ([i32] * 7 + [vp] * 7 +
                                                [ctypes.POINTER(LayerBufs), vp])
        L.moe_layer_backward.argtypes = ([i32] * 7 + [vp] * 6 + [ctypes.POINTER(LayerBufs)] +
                                         [vp] * 9 + [sz, vp])
        for f in EXPORTS[2:]:
            getattr(L, f).restype = i32
        _lib = L
    return _lib


def moe_status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def moe_workspace_bytes(kind: int, T: int, H: int, E: int, F: int, k: int, dt: int) -> int:
    return int(lib().moe_workspace_bytes(kind, T, H, E, F, k, dt))


# ----------------------------------------------------------------------- marshalling

def dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return MOE_F32
    if t == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"storage dtype must be float32 or bfloat16, got {t}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype=None, shape=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn, status):
    if status != 0:
        raise MoeError(fn, status)


def workspace(kind: int, T, H, E, F, k, dt: int, device) -> torch.Tensor:
    n = moe_workspace_bytes(kind, T, H, E, F, k, dt)
    if n == 0:
        raise MoeError("moe_workspace_bytes", 2)
    return torch.empty(n, dtype=torch.uint8, device=device)


# -------------------------------------------------------------------------- entries

def moe_gate_topk(x, wg, bias, k, top_experts=None, top_weights=None, ws=None, stream=None,
                  routing="softmax"):
    """Top-k gate (routing "softmax" or "sigmoid").  Returns (top_experts [T,k] int32,
    top_weights [T,k] fp32)."""
    dt = dtype_code(x.dtype)
    T, H = x.shape
    E = wg.shape[0]
    _need(x, "x"), _need(wg, "wg", x.dtype, (E, H))
    if bias is not None:
        _need(bias, "bias", torch.float32, (E,))
    dev = x.device
    top_experts = torch.empty((T, k), dtype=torch.int32, device=dev) if top_experts is None else top_experts
    top_weights = torch.empty((T, k), dtype=torch.float32, device=dev) if top_weights is None else top_weights
    _need(top_experts, "top_experts", torch.int32, (T, k))
    _need(top_weights, "top_weights", torch.float32, (T, k))
    ws = workspace(MOE_WS_GATE, T, H, E, 64, k, dt, dev) if ws is None else ws
    _check("moe_gate_topk", lib().moe_gate_topk(dt, T, H, E, k, ROUTING[routing], _ptr(x),
                                                _ptr(wg), _ptr(bias),
                                                _ptr(top_experts), _ptr(top_weights), _ptr(ws),
                                                ws.numel() * ws.element_size(), _stream(stream)))
    return top_experts, top_weights


def moe_pft_build(top_experts, E, out=None, ws=None, stream=None):
    """Padding-free buffers.  Returns dict(counts, offsets, token_ids, expert_ids, dest_pos)
    and, under key "ws", the workspace whose first int32 is the out-of-range-id count."""
    _need(top_experts, "top_experts", torch.int32)
    T, k = top_experts.shape
    N, dev = T * k, top_experts.device
    if out is None:
        out = dict(counts=torch.empty(E, dtype=torch.int32, device=dev),
                   offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
                   token_ids=torch.empty(max(N, 1), dtype=torch.int32, device=dev)[:N],
                   expert_ids=torch.empty(max(N, 1), dtype=torch.int32, device=dev)[:N],
                   dest_pos=torch.empty((T, k), dtype=torch.int32, device=dev))
    for n, shp in (("counts", (E,)), ("offsets", (E + 1,)), ("token_ids", (N,)),
                   ("expert_ids", (N,)), ("dest_pos", (T, k))):
        _need(out[n], n, torch.int32, shp)
    ws = workspace(MOE_WS_PFT, T, 64, E, 64, k, MOE_F32, dev) if ws is None else ws
    _check("moe_pft_build", lib().moe_pft_build(
        T, k, E, _ptr(top_experts), _ptr(out["counts"]), _ptr(out["offsets"]),
        _ptr(out["token_ids"]), _ptr(out["expert_ids"]), _ptr(out["dest_pos"]), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))
    out["ws"] = ws
    return out


def moe_dispatch(x, dest_pos, xd=None, stream=None):
    """xd[dest_pos[t, j]] = x[t].  Returns xd [T*k, H]."""
    dt = dtype_code(x.dtype)
    _need(x, "x"), _need(dest_pos, "dest_pos", torch.int32)
    T, H = x.shape
    k = dest_pos.shape[1]
    _need(dest_pos, "dest_pos", torch.int32, (T, k))
    xd = torch.empty((T * k, H), dtype=x.dtype, device=x.device) if xd is None else xd
    _need(xd, "xd", x.dtype, (T * k, H))
    _check("moe_dispatch", lib().moe_dispatch(dt, T, k, H, _ptr(x), _ptr(dest_pos), _ptr(xd),
                                              _stream(stream)))
    return xd


def moe_grouped_gemm_swiglu(xd, offsets, w1, w3, w2, h=None, y=None, ws=None, stream=None,
                            token_ids=None):
    """SwiGLU experts over the ragged segments.  Returns (h [N,F], y [N,H]).

    w2=None computes only h (the gate/up product and its SwiGLU) and returns (h, None).
    token_ids given: xd holds the token rows x [T,H] and product row p reads
    x[token_ids[p]] (the dispatch fused into the up product); N = token_ids.numel().
    """
    dt = dtype_code(xd.dtype)
    src_rows, H = xd.shape
    N = src_rows if token_ids is None else token_ids.numel()
    if token_ids is not None:
        _need(token_ids, "token_ids", torch.int32, (N,))
    E, F = w1.shape[0], w1.shape[1]
    _need(xd, "xd"), _need(offsets, "offsets", torch.int32, (E + 1,))
    _need(w1, "w1", xd.dtype, (E, F, H)), _need(w3, "w3", xd.dtype, (E, F, H))
    if w2 is not None:
        _need(w2, "w2", xd.dtype, (E, H, F))
    h = torch.empty((N, F), dtype=xd.dtype, device=xd.device) if h is None else h
    _need(h, "h", xd.dtype, (N, F))
    if w2 is None:
        y = None
    else:
        y = torch.empty((N, H), dtype=xd.dtype, device=xd.device) if y is None else y
        _need(y, "y", xd.dtype, (N, H))
    if ws is None:  # sized for N = T*k rows: pass T = N, k = 1
        ws = workspace(MOE_WS_GEMM, N, H, E, F, 1, dt, xd.device)
    _check("moe_grouped_gemm_swiglu", lib().moe_grouped_gemm_swiglu(
        dt, N, E, H, F, _ptr(xd), _ptr(token_ids), src_rows, _ptr(offsets), _ptr(w1), _ptr(w3),
        _ptr(w2), _ptr(h), _ptr(y), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return h, y


def moe_combine(y, dest_pos, top_weights, out=None, stream=None):
    """out[t] = sum_j top_weights[t, j] * y[dest_pos[t, j]].  Returns out [T, H]."""
    dt = dtype_code(y.dtype)
    _need(y, "y"), _need(dest_pos, "dest_pos", torch.int32)
    T, k = dest_pos.shape
    H = y.shape[1]
    _need(top_weights, "top_weights", torch.float32, (T, k))
    out = torch.empty((T, H), dtype=y.dtype, device=y.device) if out is None else out
    _need(out, "out", y.dtype, (T, H))
    _check("moe_combine", lib().moe_combine(dt, T, k, H, _ptr(y), _ptr(dest_pos),
                                            _ptr(top_weights), _ptr(out), _stream(stream)))
    return out


def alloc_layer_bufs(T, H, E, F, k, dtype, device, fuse_dispatch=False, store_ag=False) -> dict:
    """Intermediates of moe_layer_forward.  fuse_dispatch=True leaves xd out (None): the
    layer then gathers the expert rows from x on load and never writes xd.  store_ag=True
    adds a and g [N,F]: the forward then stores the up product's two halves, which
    moe_layer_backward uses instead of recomputing them."""
    N = T * k
    i32 = dict(dtype=torch.int32, device=device)
    ag = (lambda: torch.empty((N, F), dtype=dtype, device=device)) if store_ag else (lambda: None)
    return dict(a=ag(), g=ag(), top_experts=torch.empty((T, k), **i32),
                top_weights=torch.empty((T, k), dtype=torch.float32, device=device),
                counts=torch.empty(E, **i32), offsets=torch.empty(E + 1, **i32),
                token_ids=torch.empty(N, **i32), expert_ids=torch.empty(N, **i32),
                dest_pos=torch.empty((T, k), **i32),
                xd=None if fuse_dispatch else torch.empty((N, H), dtype=dtype, device=device),
                h=torch.empty((N, F), dtype=dtype, device=device),
                y=torch.empty((N, H), dtype=dtype, device=device))


def _need_ag(bufs, N, F, dtype):
    # a and g come together or not at all (the C side rejects one alone as well)
    for n in ("a", "g"):
        if bufs.get(n) is not None:
            _need(bufs[n], n, dtype, (N, F))


def moe_layer_forward(x, wg, bias, w1, w3, w2, k, out=None, bufs=None, ws=None, stream=None,
                      fuse_dispatch=False, routing="softmax"):
    """Whole layer.  Returns (out [T,H], bufs dict of intermediates, ws).  With
    fuse_dispatch (or bufs["xd"] None) the dispatch is fused into the expert product."""
    dt = dtype_code(x.dtype)
    T, H = x.shape
    E, F = w1.shape[0], w1.shape[1]
    _need(x, "x"), _need(wg, "wg", x.dtype, (E, H))
    _need(w1, "w1", x.dtype, (E, F, H)), _need(w3, "w3", x.dtype, (E, F, H))
    _need(w2, "w2", x.dtype, (E, H, F))
    if bias is not None:
        _need(bias, "bias", torch.float32, (E,))
    out = torch.empty((T, H), dtype=x.dtype, device=x.device) if out is None else out
    _need(out, "out", x.dtype, (T, H))
    if bufs is None:
        bufs = alloc_layer_bufs(T, H, E, F, k, x.dtype, x.device, fuse_dispatch)
    ws = workspace(MOE_WS_LAYER, T, H, E, F, k, dt, x.device) if ws is None else ws
    _need_ag(bufs, T * k, F, x.dtype)
    cb = LayerBufs(*[_ptr(bufs.get(n)) for n, _ in LayerBufs._fields_])
    _check("moe_layer_forward", lib().moe_layer_forward(
        dt, T, H, E, F, k, ROUTING[routing], _ptr(x), _ptr(wg), _ptr(bias), _ptr(w1), _ptr(w3),
        _ptr(w2), _ptr(out),
        ctypes.byref(cb), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return out, bufs, ws


def moe_layer_forward_noalloc(x, wg, bias, w1, w3, w2, k, out, bufs, stream=None,
                              routing="softmax"):
    """Whole layer on the library's static scratch (no workspace argument, nothing
    allocated by the call).  out and bufs are required (as from alloc_layer_bufs).
    Returns out."""
    dt = dtype_code(x.dtype)
    T, H = x.shape
    E, F = w1.shape[0], w1.shape[1]
    _need(x, "x"), _need(wg, "wg", x.dtype, (E, H))
    _need(w1, "w1", x.dtype, (E, F, H)), _need(w3, "w3", x.dtype, (E, F, H))
    _need(w2, "w2", x.dtype, (E, H, F))
    if bias is not None:
        _need(bias, "bias", torch.float32, (E,))
    _need(out, "out", x.dtype, (T, H))
    _need_ag(bufs, T * k, F, x.dtype)
    cb = LayerBufs(*[_ptr(bufs.get(n)) for n, _ in LayerBufs._fields_])
    _check("moe_layer_forward_noalloc", lib().moe_layer_forward_noalloc(
        dt, T, H, E, F, k, ROUTING[routing], _ptr(x), _ptr(wg), _ptr(bias), _ptr(w1), _ptr(w3),
        _ptr(w2), _ptr(out), ctypes.byref(cb), _stream(stream)))
    return out


def moe_layer_backward(x, wg, bias, w1, w3, w2, k, bufs, dout, grads=None, ws=None, stream=None,
                       routing="softmax"):
    """Layer backward.  bufs: the intermediates of the forward (as returned by
    moe_layer_forward).  Returns (grads dict: dx, dwg, dbias, dw1, dw3, dw2, dtw; ws)."""
    dt = dtype_code(x.dtype)
    T, H = x.shape
    E, F = w1.shape[0], w1.shape[1]
    _need(x, "x"), _need(wg, "wg", x.dtype, (E, H)), _need(dout, "dout", x.dtype, (T, H))
    _need(w1, "w1", x.dtype, (E, F, H)), _need(w3, "w3", x.dtype, (E, F, H))
    _need(w2, "w2", x.dtype, (E, H, F))
    if bias is not None:
        _need(bias, "bias", torch.float32, (E,))
    if grads is None:
        dev = x.device
        grads = dict(dx=torch.empty((T, H), dtype=x.dtype, device=dev),
                     dwg=torch.empty((E, H), dtype=x.dtype, device=dev),
                     dbias=torch.empty((E,), dtype=torch.float32, device=dev),
                     dw1=torch.empty((E, F, H), dtype=x.dtype, device=dev),
                     dw3=torch.empty((E, F, H), dtype=x.dtype, device=dev),
                     dw2=torch.empty((E, H, F), dtype=x.dtype, device=dev),
                     dtw=torch.empty((T, k), dtype=torch.float32, device=dev))
    ws = workspace(MOE_WS_BACKWARD, T, H, E, F, k, dt, x.device) if ws is None else ws
    _need_ag(bufs, T * k, F, x.dtype)
    cb = LayerBufs(*[_ptr(bufs.get(n)) for n, _ in LayerBufs._fields_])
    _check("moe_layer_backward", lib().moe_layer_backward(
        dt, T, H, E, F, k, ROUTING[routing], _ptr(x), _ptr(wg), _ptr(bias), _ptr(w1), _ptr(w3),
        _ptr(w2), ctypes.byref(cb), _ptr(dout), _ptr(grads["dx"]), _ptr(grads["dwg"]),
        _ptr(grads["dbias"]), _ptr(grads["dw1"]), _ptr(grads["dw3"]), _ptr(grads["dw2"]),
        _ptr(grads.get("dtw")), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return grads, ws
