"""The L2 model's bookkeeping (CPU only): tile lists, request totals and its two limits."""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

from gemm_gate_softmax_amd import l2_model as M  # noqa: E402

COUNTS = np.array([0, 3, 700, 64, 65, 1, 300, 0, 129, 2000], dtype=np.int64)
KW = dict(n_feat=384, nk=12)


def test_tile_lists_cover_every_row_once():
    large, small = M.tile_lists(COUNTS, 128, 3, 4)
    big = [e for e, c in enumerate(COUNTS) if c > 64]
    keys = [(e, tt, ft) for e, tt, ft, _ in large]
    assert len(keys) == len(set(keys))
    for e in big:
        rows = sum(r for e2, _, ft, r in large if e2 == e and ft == 0)
        assert rows == COUNTS[e]
    assert sorted({e for e, *_ in small}) == [e for e, c in enumerate(COUNTS) if 0 < c <= 64]
    orders = M.xcd_orders(large, small)
    assert sum(len(o) for o in orders) == len(large) + len(small)


def _requested(counts, n_feat, nk, bf=128, nb=2, bt=128):
    ft = (n_feat + bf - 1) // bf
    large, small = M.tile_lists(counts, bt, ft, 32)
    per = lambda rows: nk * (min(rows, bt) * M.ROW_BYTES + nb * bf * M.ROW_BYTES)
    return sum(per(r) for *_, r in large) + sum(per(r) for *_, r in small)


def test_requests_and_the_two_limits():
    miss, req = M.simulate(COUNTS, **KW)
    assert req == _requested(COUNTS, **KW)
    # no L2: every request misses
    assert M.simulate(COUNTS, l2_bytes=0, **KW) == (req, req)
    # an L2 that holds everything: each distinct block misses once on every XCD whose tiles
    # read it (each XCD has its own L2); small-tile weights do not allocate but are read once
    nk = KW["nk"]
    large, small = M.tile_lists(COUNTS, 128, 3, 32)
    compulsory = 0
    for seq in M.xcd_orders(large, small):
        seen = {}
        for is_large, e, tt, ft, r in seq:
            seen[("x", e, tt)] = min(r, 128) * M.ROW_BYTES * nk
            if is_large:
                seen[("w", e, ft)] = 2 * 128 * M.ROW_BYTES * nk
            else:
                compulsory += 2 * 128 * M.ROW_BYTES * nk
        compulsory += sum(seen.values())
    assert M.simulate(COUNTS, l2_bytes=1 << 50, **KW)[0] == compulsory
    assert compulsory <= miss <= req
