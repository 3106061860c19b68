"""Host-side model of the tile GEMM's loader ring (CPU only).

The loader waves of ``compute_tile`` (csrc/gemm.hip) fill an S-slot LDS ring with k-slices
and hand each slice to the compute waves at one workgroup barrier; their only
synchronisation is ``s_waitcnt vmcnt(n)`` (at most n of the wave's transfers still in
flight; a wave's loads retire in issue order) before each barrier.  This model replays a
loader wave's issue sequence and its wait counts exactly as the kernel states them, for
every ring depth the kernels use, every K range and every per-slice transfer count, and
checks the three properties the kernel relies on:

* at barrier b every transfer of slice b has landed;
* a slot is refilled only after the barrier that ends the compute waves' reads of it;
* nothing is in flight when the loaders meet the compute waves for the epilogue.
"""
import pytest


def loader_schedule(S, nk, c, pre=None):
    """Events of one loader wave: ("issue", stage, slot) per transfer, ("wait", n), ("barrier", b).
    pre: stages issued before barrier 0 (S - 1, or fewer in a persistent run of tiles, where
    the rest follow barrier 0)."""
    pre = S - 1 if pre is None else pre
    ev = []

    def issue(stage, slot):
        ev.extend(("issue", stage, slot) for _ in range(c))

    if nk == 1:
        issue(0, 0)
        ev += [("wait", 0), ("barrier", 0)]
    else:
        for s in range(pre):
            issue(min(s, nk - 1), s)
        ev += [("wait", (pre - 1) * c), ("barrier", 0)]
        for s in range(pre, S - 1):
            issue(min(s, nk - 1), s)
    refill = S - 1
    for kt in range(nk - 1):
        if kt + S - 1 < nk:
            issue(kt + S - 1, refill)
            ev.append(("wait", (S - 2) * c))
        elif S == 3:
            ev.append(("wait", 0))
        else:
            ev.append(("wait", (nk - 2 - kt) * c))
        ev.append(("barrier", kt + 1))
        refill = 0 if refill == S - 1 else refill + 1
    ev += [("wait", 0), ("barrier", "epilogue")]
    return ev


def check(S, nk, c, pre=None):
    issued = []          # (stage, slot) per transfer, in issue order
    landed = 0           # transfers retired (in order)
    last_barrier = -1    # compute waves read slice b between barriers b and b + 1
    for e in loader_schedule(S, nk, c, pre):
        if e[0] == "issue":
            _, stage, slot = e
            # the slot must not hold a slice the compute waves may still read: the slice in
            # it was read between barriers (its stage) and (its stage + 1)
            holders = {st for st, sl in issued if sl == slot}
            for st in holders:
                if st != stage:
                    assert last_barrier >= st + 1, (S, nk, c, "slot reused early", stage, st)
            # a slot holds the slice of its index mod S (clamped copies excepted: they
            # land in a slot no slice reads)
            if stage % S != slot:
                assert stage == nk - 1 and slot >= nk, (S, nk, c, stage, slot)
            issued.append((stage, slot))
        elif e[0] == "wait":
            landed = max(landed, len(issued) - e[1])
            assert e[1] >= 0
        else:
            b = e[1]
            if b == "epilogue":
                assert landed == len(issued), (S, nk, c, "transfers in flight at the epilogue")
                continue
            mine = [i for i, (st, _) in enumerate(issued) if st == b]
            assert mine, (S, nk, c, "slice never issued", b)
            assert max(mine) < landed, (S, nk, c, "slice not landed at its barrier", b)
            last_barrier = b
    # every slice was issued exactly once, apart from clamped copies of the last one
    stages = [st for st, _ in issued]
    for s in range(nk):
        assert stages.count(s) == c or (s == nk - 1 and stages.count(s) % c == 0)


@pytest.mark.parametrize("S", [2, 3, 4])
def test_loader_ring_counts(S):
    for nk in range(1, 61):
        for c in range(1, 13):
            check(S, nk, c)


@pytest.mark.parametrize("S", [3, 4])
def test_loader_ring_counts_persistent_prologue(S):
    # a tile of a persistent run issues only its first `pre` stages before barrier 0 (the
    # previous tile's outputs may still be staged in the others' slots) and the rest after it
    for pre in range(1, S - 1):
        for nk in range(1, 61):
            for c in range(1, 13):
                check(S, nk, c, pre)


def test_no_redundant_transfers_once_k_covers_the_ring():
    # with at least S - 1 slices every transfer is of a slice the compute waves read
    for S in (2, 3, 4):
        for nk in range(S - 1, 40):
            stages = [e[1] for e in loader_schedule(S, nk, 1) if e[0] == "issue"]
            assert stages == list(range(nk)), (S, nk, stages)
