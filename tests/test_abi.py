"""The C ABI on a machine without a GPU: the library loads, exports every entry point the
header declares, sizes workspaces, names statuses, and rejects invalid arguments on the
host before anything is enqueued (no compute call is made here)."""
import ctypes
import os
import re

import pytest

from gemm_gate_softmax_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

OK, INVALID, UNSUPPORTED, MISALIGNED, WS_SMALL = 0, 1, 2, 3, 4


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ops.LIB_PATH):
        from gemm_gate_softmax_amd import build
        build.build()
    return ops.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_header_declares_the_six_stages():
    names = declared_functions()
    for n in ("moe_gate_topk", "moe_pft_build", "moe_dispatch", "moe_grouped_gemm_swiglu",
              "moe_combine", "moe_layer_forward"):
        assert n in names


def test_every_declared_function_is_exported(L):
    for n in declared_functions():
        assert hasattr(L, n), n
    assert set(declared_functions()) == set(ops.EXPORTS)


def test_status_strings(L):
    for code, name in ops.STATUS.items():
        assert ops.moe_status_string(code).startswith(name)
    assert "unknown" in ops.moe_status_string(99)


def test_workspace_bytes(L):
    T, H, E, F, k = 4096, 7168, 256, 2048, 8
    for kind in range(4):
        n = ops.moe_workspace_bytes(kind, T, H, E, F, k, ops.MOE_BF16)
        assert n > 0 and n % 256 == 0
    layer = ops.moe_workspace_bytes(ops.MOE_WS_LAYER, T, H, E, F, k, ops.MOE_BF16)
    parts = sum(ops.moe_workspace_bytes(w, T, H, E, F, k, ops.MOE_BF16) for w in range(3))
    assert layer == parts
    assert ops.moe_workspace_bytes(ops.MOE_WS_GATE, T, H, E, F, k, 0) >= T * E * 4
    # unsupported arguments size to 0
    assert ops.moe_workspace_bytes(0, T, H, E, F, E + 1, 1) == 0
    assert ops.moe_workspace_bytes(0, T, H, 2000, F, k, 1) == 0
    assert ops.moe_workspace_bytes(9, T, H, E, F, k, 1) == 0
    assert ops.moe_workspace_bytes(0, T, H, E, F, k, 7) == 0


P = ctypes.c_void_p
A = P(0x10000)      # aligned, never dereferenced: validation fails before any use
MIS = P(0x10004)


def test_gate_rejects(L):
    g = L.moe_gate_topk
    assert g(1, 8, 64, 4, 5, 0, A, A, None, A, A, A, 1 << 20, None) == UNSUPPORTED      # k > E
    assert g(1, 8, 64, 4, 0, 0, A, A, None, A, A, A, 1 << 20, None) == INVALID          # k < 1
    assert g(1, 8, 96, 4, 2, 0, A, A, None, A, A, A, 1 << 20, None) == UNSUPPORTED      # H % 64
    assert g(1, 8, 64, 2048, 2, 0, A, A, None, A, A, A, 1 << 30, None) == UNSUPPORTED   # E > max
    assert g(3, 8, 64, 4, 2, 0, A, A, None, A, A, A, 1 << 20, None) == INVALID          # dtype
    assert g(1, 8, 64, 4, 2, 0, None, A, None, A, A, A, 1 << 20, None) == INVALID       # NULL x
    assert g(1, 8, 64, 4, 2, 0, MIS, A, None, A, A, A, 1 << 20, None) == MISALIGNED
    assert g(1, 8, 64, 4, 2, 0, A, A, MIS, A, A, A, 1 << 20, None) == MISALIGNED        # bias
    assert g(1, 8, 64, 4, 2, 0, A, A, None, A, A, A, 16, None) == WS_SMALL
    assert g(1, 0, 64, 4, 2, 0, None, None, None, None, None, None, 0, None) == OK      # T == 0
    assert g(1, -1, 64, 4, 2, 0, A, A, None, A, A, A, 1 << 20, None) == INVALID
    assert g(1, 8, 64, 4, 2, 2, A, A, None, A, A, A, 1 << 20, None) == INVALID       # routing


def test_pft_rejects(L):
    f = L.moe_pft_build
    assert f(8, 9, 4, A, A, A, A, A, A, A, 1 << 20, None) == UNSUPPORTED  # k > E
    assert f(8, 65, 100, A, A, A, A, A, A, A, 1 << 20, None) == UNSUPPORTED  # k > K_MAX
    assert f(1 << 28, 16, 64, A, A, A, A, A, A, A, 1 << 40, None) == UNSUPPORTED  # N >= 2^31
    assert f(8, 2, 4, None, A, A, A, A, A, A, 1 << 20, None) == INVALID
    assert f(8, 2, 4, A, A, A, MIS, A, A, A, 1 << 20, None) == MISALIGNED
    assert f(8, 2, 4, A, A, A, A, A, A, A, 8, None) == WS_SMALL


def test_move_rejects(L):
    d, c = L.moe_dispatch, L.moe_combine
    assert d(1, 8, 2, 100, A, A, A, None) == UNSUPPORTED
    assert d(1, 8, 0, 64, A, A, A, None) == INVALID
    assert d(1, 8, 2, 64, A, None, A, None) == INVALID
    assert d(1, 8, 2, 64, A, A, MIS, None) == MISALIGNED
    assert d(1, 0, 2, 64, None, None, None, None) == OK
    assert c(0, 8, 2, 64, A, A, None, A, None) == INVALID
    assert c(0, 8, 2, 64, A, A, A, MIS, None) == MISALIGNED
    assert c(0, 8, 70, 64, A, A, A, A, None) == UNSUPPORTED
    assert c(0, 0, 2, 64, None, None, None, None, None) == OK


def test_gemm_and_layer_reject(L):
    L_g = L.moe_grouped_gemm_swiglu
    # (dt, N, E, H, F, xd, offsets, w1, w3, w2, h, y, ws, ws_bytes, stream), token_ids NULL
    g = lambda dt, N, E, H, F, xd, *rest: L_g(dt, N, E, H, F, xd, None, 0, *rest)
    assert g(1, 100, 8, 64, 100, A, A, A, A, A, A, A, A, 1 << 20, None) == UNSUPPORTED  # F % 64
    assert g(1, 100, 0, 64, 64, A, A, A, A, A, A, A, A, 1 << 20, None) == INVALID      # E < 1
    assert g(1, 100, 8, 64, 64, A, A, A, A, A, A, A, A, 0, None) == WS_SMALL
    assert g(1, 100, 8, 64, 64, A, A, A, MIS, A, A, A, A, 1 << 20, None) == MISALIGNED
    assert g(1, 0, 8, 64, 64, None, None, None, None, None, None, None, None, 0, None) == OK
    # up product only needs w2 and y both NULL; one of them alone is an error
    assert g(1, 100, 8, 64, 64, A, A, A, A, None, A, A, A, 1 << 20, None) == INVALID
    assert g(1, 100, 8, 64, 64, A, A, A, A, A, A, None, A, 1 << 20, None) == INVALID
    assert g(1, 100, 8, 64, 64, A, A, A, A, None, None, None, A, 1 << 20, None) == INVALID  # h
    # fused dispatch: token_ids needs src_rows >= 1 and an aligned pointer
    assert L_g(1, 100, 8, 64, 64, A, A, 0, A, A, A, A, A, A, A, 1 << 20, None) == INVALID
    assert L_g(1, 100, 8, 64, 64, A, MIS, 10, A, A, A, A, A, A, A, 1 << 20, None) == MISALIGNED
    lf = L.moe_layer_forward
    bufs = ops.LayerBufs(*([A] * 10))
    args = lambda **kw: [kw.get("dt", 1), kw.get("T", 8), kw.get("H", 64), kw.get("E", 4),
                         kw.get("F", 64), kw.get("k", 2), kw.get("routing", 0), A, A, None, A,
                         A, A, A,
                         ctypes.byref(kw.get("bufs", bufs)), A, kw.get("ws", 1 << 30), None]
    assert lf(*args(k=5)) == UNSUPPORTED
    assert lf(*args(routing=7)) == INVALID
    assert lf(*args(F=32)) == UNSUPPORTED
    assert lf(*args(ws=100)) == WS_SMALL
    nb = ops.LayerBufs(*([A] * 9 + [None]))
    assert lf(*args(bufs=nb)) == INVALID
    mb = ops.LayerBufs(*([A] * 8 + [MIS, A]))
    assert lf(*args(bufs=mb)) == MISALIGNED
    xb = ops.LayerBufs(*([A] * 7 + [MIS, A, A]))        # xd may be NULL, never misaligned
    assert lf(*args(bufs=xb)) == MISALIGNED
    nb7 = ops.LayerBufs(*([A] * 6 + [None, None, A, A]))  # dest_pos stays required
    assert lf(*args(bufs=nb7)) == INVALID
    # the up product's halves a and g: both or neither, aligned
    assert lf(*args(bufs=ops.LayerBufs(*([A] * 10 + [A, None])))) == INVALID
    assert lf(*args(bufs=ops.LayerBufs(*([A] * 10 + [None, A])))) == INVALID
    assert lf(*args(bufs=ops.LayerBufs(*([A] * 10 + [MIS, A])))) == MISALIGNED
    assert lf(*args(T=0)) == OK


def test_layer_forward_noalloc_rejects(L):
    """The no-workspace layer forward validates like moe_layer_forward and refuses, before
    touching any device, a call whose layer workspace exceeds its static scratch."""
    lf = L.moe_layer_forward_noalloc
    bufs = ops.LayerBufs(*([A] * 10))
    args = lambda **kw: [kw.get("dt", 1), kw.get("T", 8), kw.get("H", 64), kw.get("E", 4),
                         kw.get("F", 64), kw.get("k", 2), kw.get("routing", 0), A, A, None, A,
                         A, A, A, ctypes.byref(kw.get("bufs", bufs)), None]
    assert lf(*args(k=5)) == UNSUPPORTED
    assert lf(*args(routing=7)) == INVALID
    assert lf(*args(F=32)) == UNSUPPORTED
    assert lf(*args(bufs=ops.LayerBufs(*([A] * 9 + [None])))) == INVALID
    assert lf(*args(T=0)) == OK
    # 65536 tokens x 256 experts: 64 MiB of partial logits alone
    T, H, E, F, k = 65536, 7168, 256, 2048, 8
    need = ops.moe_workspace_bytes(ops.MOE_WS_LAYER, T, H, E, F, k, ops.MOE_BF16)
    assert need > ops.MOE_NOALLOC_SCRATCH_BYTES
    assert lf(*args(T=T, H=H, E=E, F=F, k=k)) == 6
    assert "MOE_ERR_SCRATCH_TOO_SMALL" in ops.moe_status_string(6)
    # the X-MoE Large layer fits
    assert ops.moe_workspace_bytes(ops.MOE_WS_LAYER, 4096, H, E, F, k, ops.MOE_BF16) <= \
        ops.MOE_NOALLOC_SCRATCH_BYTES


def test_layer_backward_rejects(L):
    lb = L.moe_layer_backward
    bufs = ops.LayerBufs(*([A] * 10))
    args = lambda **kw: [kw.get("dt", 1), kw.get("T", 8), kw.get("H", 64), kw.get("E", 4),
                         kw.get("F", 64), kw.get("k", 2), kw.get("routing", 0), A, A, None, A,
                         A, A, ctypes.byref(kw.get("bufs", bufs)), kw.get("dout", A),
                         A, A, kw.get("dbias", A), A, A, A, kw.get("dtw", None), A,
                         kw.get("ws", 1 << 40), None]
    assert lb(*args(k=5)) == UNSUPPORTED
    assert lb(*args(routing=3)) == INVALID
    assert lb(*args(F=96 + 1)) == UNSUPPORTED
    assert lb(*args(ws=100)) == WS_SMALL
    assert lb(*args(dout=None)) == INVALID
    assert lb(*args(dbias=MIS)) == MISALIGNED
    assert lb(*args(dtw=MIS)) == MISALIGNED
    nh = ops.LayerBufs(*([A] * 8 + [None, A]))          # h is required by the backward
    assert lb(*args(bufs=nh)) == INVALID
    xb = ops.LayerBufs(*([A] * 7 + [MIS, A, A]))        # xd may be NULL, never misaligned
    assert lb(*args(bufs=xb)) == MISALIGNED
    assert lb(*args(bufs=ops.LayerBufs(*([A] * 10 + [A, None])))) == INVALID   # a without g
    assert lb(*args(bufs=ops.LayerBufs(*([A] * 10 + [A, MIS])))) == MISALIGNED
    assert lb(*args(T=0)) == OK


def test_backward_workspace_size(L):
    ws = L.moe_workspace_bytes
    small = ws(4, 8, 64, 4, 64, 2, 1)
    assert small > 0 and small % 256 == 0
    # row-sized intermediates only (no weight copies): within the documented bound, and
    # under 4 GB at T=4096, H=7168, E=256, F=2048, top-8, bf16
    T, H, E, F, k = 4096, 7168, 256, 2048, 8
    big = ws(4, T, H, E, F, k, 1)
    assert (3 * H + 5 * F) * T * k * 2 < big <= ((3 * H + 5 * F) * T * k + (H + E) * (T + 63)) * 2 + (4 << 20)
    assert big < 2.5e9
    assert ws(4, 8, 64, 4, 100, 2, 1) == 0              # F not a multiple of 64
