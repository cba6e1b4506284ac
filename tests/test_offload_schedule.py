"""The copy / compute schedule of attention over host-resident K/V (runs without a GPU).

[ETE]'s KV-offload passage copies one tile of positions at a time into a device buffer; its
next-steps list asks for several buffers with the two event edges of its layer streaming: a tile's
compute waits for that tile's copy (data ready), and a copy into a buffer waits for the compute
that last read it (buffer free).  qdec_offload_schedule returns the enqueue order the library
issues.  These tests run that order through a model of two in-order streams with per-tile events
and random durations, and check: every compute reads the tile it names, no copy overwrites a
buffer a compute is still reading, one buffer serialises copy and compute, and two or more
overlap them.  Removing the buffer-free waits (planted here, on the CPU) is caught.
"""
import random

import pytest

from decode_step_04_amd import qdec as Q

WAIT_FREE, COPY, WAIT_READY, COMPUTE, MERGE = range(5)


def simulate(records, n_slots, copy_t, comp_t):
    """Runs the records on a copy stream and a compute stream.  Returns (end time, hazards)."""
    cs = ks = 0.0                      # time each stream is free
    copied, computed = {}, {}          # tile -> end time of its copy / compute
    slot_tile, writes, reads = {}, {}, {}
    hazards = []
    for kind, tile, slot, other in records:
        if kind == WAIT_FREE:
            cs = max(cs, computed[other])
        elif kind == COPY:
            start, end = cs, cs + copy_t[tile]
            writes.setdefault(slot, []).append((start, end, tile))
            cs = end
            copied[tile] = end
        elif kind == WAIT_READY:
            ks = max(ks, copied[other])
        elif kind == COMPUTE:
            start, end = ks, ks + comp_t[tile]
            reads.setdefault(slot, []).append((start, end, tile))
            ks = end
            computed[tile] = end
        elif kind == MERGE:
            ks += 1.0
    for slot, rs in reads.items():
        ws = sorted(writes.get(slot, []))
        for (r0, r1, t) in rs:
            own = [w for w in ws if w[2] == t]
            if not own or own[0][1] > r0:
                hazards.append(("read before its copy", t))
            for (w0, w1, wt) in ws:
                if wt != t and w0 < r1 and w1 > r0:
                    hazards.append(("overwritten while read", t, wt))
    return max(cs, ks), hazards


@pytest.mark.parametrize("n_tiles,n_slots", [(1, 1), (1, 3), (5, 1), (7, 2), (13, 3), (40, 8)])
def test_schedule_shape(n_tiles, n_slots):
    recs = Q.qdec_offload_schedule(n_tiles, n_slots)
    kinds = [r[0] for r in recs]
    assert kinds.count(COPY) == n_tiles and kinds.count(COMPUTE) == n_tiles
    assert kinds.count(WAIT_READY) == n_tiles
    assert kinds.count(WAIT_FREE) == max(0, n_tiles - n_slots)
    assert recs[-1][0] == MERGE and kinds.count(MERGE) == 1
    for kind, tile, slot, other in recs:
        if kind in (COPY, COMPUTE, WAIT_READY):
            assert slot == tile % n_slots
        if kind == WAIT_READY:
            assert other == tile
        if kind == WAIT_FREE:
            assert other == tile - n_slots and other % n_slots == slot


@pytest.mark.parametrize("n_slots", [1, 2, 3, 5])
def test_no_hazard_under_random_durations(n_slots):
    rng = random.Random(n_slots)
    for trial in range(200):
        n = rng.randint(1, 30)
        recs = Q.qdec_offload_schedule(n, n_slots)
        copy_t = [rng.uniform(0.1, 10.0) for _ in range(n)]
        comp_t = [rng.uniform(0.1, 10.0) for _ in range(n)]
        _, hazards = simulate(recs, n_slots, copy_t, comp_t)
        assert not hazards, (trial, hazards[:3])


def test_one_buffer_serialises_and_two_overlap():
    n, c, k = 20, 4.0, 1.0
    t1, _ = simulate(Q.qdec_offload_schedule(n, 1), 1, [c] * n, [k] * n)
    t2, _ = simulate(Q.qdec_offload_schedule(n, 2), 2, [c] * n, [k] * n)
    assert t1 == pytest.approx(n * (c + k) + 1.0)       # copy, compute, copy, ...
    assert t2 == pytest.approx(n * c + k + 1.0)         # copies back to back, compute hidden
    # compute-bound tiles: the copies hide instead
    t2b, _ = simulate(Q.qdec_offload_schedule(n, 2), 2, [k] * n, [c] * n)
    assert t2b == pytest.approx(k + n * c + 1.0)


def test_missing_buffer_free_edge_is_caught():
    recs = [r for r in Q.qdec_offload_schedule(12, 2) if r[0] != WAIT_FREE]
    # fast copies race ahead of slow computes and overwrite buffers still being read
    _, hazards = simulate(recs, 2, [0.1] * 12, [5.0] * 12)
    assert any(h[0] == "overwritten while read" for h in hazards)


def test_schedule_rejects_bad_counts():
    for nt, ns in ((0, 1), (3, 0), (3, 9)):
        with pytest.raises(Q.QdecError):
            Q.qdec_offload_schedule(nt, ns)
