"""Host-side model of the expert products' persistent tile loop (CPU only).

bf16 expert products launch one workgroup per CU; workgroup i of an XCD (W per XCD) starts
with the XCD's tile i, and near the end of every tile one loader lane claims the next,
W + (the XCD's counter, incremented), until the claim passes the XCD's tile count.  The
loader waves of tile i + 1 fill the ring slots below the staging region before that tile's
barrier 0, while the compute waves still stage tile i's outputs in the last STG bytes of
the LDS array (``expert_gemm_kernel`` and ``compute_tile`` with LDS_BYTES > 0 in
csrc/gemm.hip).  This model restates the kernel's tile geometry and checks:

* every tile of an XCD runs exactly once and every workgroup's loop ends, whatever order
  tiles finish in and however many tiles and workgroups there are;
* for every pair of tile kinds that can follow each other in one launch, the slots the
  second fills before its barrier 0 lie clear of the region where the first stages its
  outputs, and every ring and staging region fits the LDS array and the CU's 160 KiB.
"""
import heapq
import random

import pytest

RB, S, SMALL_BT, SMALL_S, LDS_MAX = 128, 3, 64, 3, 160 * 1024
BF16 = 2


def stage_bytes(bt, bf, nb):
    return (bt + nb * bf) * RB


def staging_bytes(bt, bf):
    # 4 compute waves x bt/2 token rows of bf/2 outputs, rows padded by 16 bytes
    return 4 * (bt // 2) * ((bf // 2) * BF16 + 16)


# (product, large tile height, feature tile width, weight operands) of every bf16 expert
# launch: the forward's up and down products on 128-token tiles, the same on the 64-token
# tiles of small problems, and the backward's products (the recompute of a and g has the up
# product's geometry, dh and dxd the down product's)
LAUNCHES = [("up", 128, 128, 2), ("down", 128, 256, 1), ("up small problem", 64, 64, 2),
            ("down small problem", 64, 128, 1)]


@pytest.mark.parametrize("launch", LAUNCHES, ids=lambda l: l[0])
def test_next_tile_fills_no_slot_under_the_staging(launch):
    _, bt, bf, nb = launch
    kinds = {"large": (bt, S), "small": (SMALL_BT, SMALL_S)}   # tile height, ring slots
    lds = max(s * stage_bytes(h, bf, nb) for h, s in kinds.values())
    stg = staging_bytes(bt, bf)                                # sized for the large tile
    assert lds <= LDS_MAX and stg <= lds
    region = {k: (lds - stg, lds - stg + staging_bytes(h, bf)) for k, (h, _) in kinds.items()}
    for k, (h, s) in kinds.items():
        assert s * stage_bytes(h, bf, nb) <= lds
        assert region[k][1] <= lds                             # staging inside the array
        pre = min(s - 1, (lds - stg) // stage_bytes(h, bf, nb))
        assert pre >= 1, (launch, k)
        filled = (0, pre * stage_bytes(h, bf, nb))             # slots filled before barrier 0
        for prev in kinds:
            lo, hi = region[prev]
            assert filled[1] <= lo or filled[0] >= hi, (launch, prev, k, filled, region[prev])


def run_xcd(n_tiles, w, rng):
    """Replays one XCD's workgroups over its tile sequence with random tile lengths; returns
    the tiles each workgroup ran, in order, and the counter's final value."""
    counter = 0
    ran = [[] for _ in range(w)]
    events = []                                     # (finish time, workgroup, tile)
    for g in range(w):
        if g < n_tiles:                             # first tile: the XCD's tile g
            heapq.heappush(events, (rng.uniform(0.5, 2.0), g, g))
    while events:
        t, g, j = heapq.heappop(events)
        ran[g].append(j)
        nxt = w + counter                           # claimed near the end of tile j
        counter += 1
        if nxt < n_tiles:
            heapq.heappush(events, (t + rng.uniform(0.5, 2.0), g, nxt))
    return ran, counter


def test_claims_run_every_tile_once():
    rng = random.Random(7)
    for _ in range(3000):
        n_tiles = rng.choice([0, 1, 5, 31, 32, 33, 64, 100, rng.randrange(0, 3000)])
        w = rng.choice([1, 2, 8, 31, 32])
        ran, counter = run_xcd(n_tiles, w, rng)
        tiles = sorted(j for r in ran for j in r)
        assert tiles == list(range(n_tiles)), (n_tiles, w)
        # one claim per tile run; the ones past the end stop their workgroups
        assert counter == n_tiles
        started = min(w, n_tiles)
        assert sum(1 for r in ran if r) == started
        for g, r in enumerate(ran):
            if r:
                assert r[0] == g and all(a < b for a, b in zip(r, r[1:]))
