"""Schedule model of the decode attention kernel's loader waves (CPU).

The loader waves of ``attend_mfma_kernel`` (long_context_sparse_10_amd/csrc/
attend.hip) gather each 32-row tile into one of R register sets (R = 2, or 3
for splits of 8 tiles or more), commit tile u to the LDS buffer u & 1, and
meet the math waves at one barrier per tile after a first one.  The phases run
in unrolled groups of R while every stage is a real tile, then up to 2R last
phases with their conditions.  This model replays that schedule and checks
what the kernel relies on: the barrier count equals the math waves' (tiles +
1), every tile is committed once, from the set that staged it, between the
barrier after which its LDS buffer is free and the barrier after which the
math waves read it.
"""
import pytest


def schedule(ntiles, R):
    ev = []

    def stage(st, t):
        ev.append(("stage", st, t))

    def commit(st, u):
        ev.append(("commit", st, u))

    def bar():
        ev.append(("bar",))

    if ntiles > 0:
        for i in range(R):
            stage(i, i)
        commit(0, 0)
        stage(0, R)
    bar()
    u = 1
    while u + 2 * R - 1 < ntiles:        # every stage of the group is a real tile
        for j in range(R):
            commit((u + j) % R, u + j)
            stage((u + j) % R, u + j + R)
            bar()
        u += R
    for j in range(2 * R):               # the last phases, with their conditions
        v = u + j
        if v <= ntiles:
            if v < ntiles:
                commit(v % R, v)
            if v + R < ntiles:
                stage(v % R, v + R)
            bar()
    return ev


@pytest.mark.parametrize("R", [2, 3])
def test_loader_ring_schedule(R):
    for ntiles in range(0, 80):
        ev = schedule(ntiles, R)
        assert sum(1 for e in ev if e[0] == "bar") == ntiles + 1
        held, committed, barriers = {}, [], 0
        for e in ev:
            if e[0] == "stage":
                held[e[1]] = e[2]        # a tile index >= ntiles re-reads the last tile
            elif e[0] == "commit":
                st, u = e[1], e[2]
                assert held.get(st) == u, (ntiles, st, held.get(st), u)
                assert barriers == u     # LDS buffer u & 1 is free, not yet read
                committed.append(u)
                held[st] = None
            else:
                barriers += 1
        assert committed == list(range(ntiles))
