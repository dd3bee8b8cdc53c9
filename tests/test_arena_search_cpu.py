"""The region search's policy (arena.search_regions) on the CPU, with a fake
set of region operations: every backing handle it creates must end up either
mapped or released exactly once (never released while mapped, never leaked),
each region must keep the fastest backing it saw, a region within the
tolerance of the best rate so far is not searched, and running out of memory
for candidates ends that array's tries."""
import random

import pytest

from sharded_mixed_precision_amd.arena import search_regions


class FakeOps:
    """Region j's pass-2 time is its length times 1 + the penalties of the
    handles mapped there (one per array); every handle gets a random
    penalty when created."""

    def __init__(self, nreg, keys, seed, region_len=100, memory=10 ** 9):
        self.rng = random.Random(seed)
        self.keys = keys
        self.pen = {}
        self.next = 0
        self.mapped = {}
        self.released = []
        self.live = set()
        self.memory = memory
        self.region_len = region_len
        for key in keys:
            for j in range(nreg):
                self.mapped[(key, j)] = self._new()
        self.timed = []

    def _new(self):
        self.next += 1
        self.pen[self.next] = self.rng.choice([0.0, 0.0, 0.13, 0.15, 0.2]) + self.rng.random() * 0.004
        self.live.add(self.next)
        return self.next

    def region_ms(self, j):
        m = self.region_len if j < 5 else self.region_len // 3  # a shorter last region
        t = m * (1.0 + sum(self.pen[self.mapped[(k, j)]] for k in self.keys)) * 1e-3
        self.timed.append((j, t))
        return t, m

    def create(self, key, j):
        if self.memory <= 0:
            return None
        self.memory -= 1
        return self._new()

    def current(self, key, j):
        return self.mapped[(key, j)]

    def use(self, key, j, h):
        assert h in self.live, "mapping a released handle"
        self.mapped[(key, j)] = h

    def release(self, h):
        assert h in self.live, "released twice"
        assert h not in self.mapped.values(), "released while mapped"
        self.live.remove(h)
        self.released.append(h)


@pytest.mark.parametrize("seed", range(12))
def test_every_handle_mapped_or_released_once_and_regions_keep_their_best(seed):
    keys = ["grad", "param", "master", "exp_avg", "exp_avg_sq"]
    ops = FakeOps(6, keys, seed)
    before = {j: ops.region_ms(j)[0] for j in range(6)}
    rep = search_regions(ops, 6, keys, tries=4, sweeps=2, tol=0.01)
    assert [r[0] for r in rep] == list(range(6))
    mapped = set(ops.mapped.values())
    assert ops.live == mapped  # nothing leaked: every live handle is mapped
    assert len(ops.released) == len(set(ops.released))
    assert ops.next == len(mapped) + len(ops.released)
    for j, first, best, tried in rep:
        now = ops.region_ms(j)[0]
        assert best == round(now, 4)  # the kept backings give the recorded time
        assert best <= first + 1e-12 and now <= before[j] + 1e-12  # never worse
        assert 0 <= tried <= 4 * len(keys)


def test_tolerance_stops_regions_near_the_best_rate():
    keys = ["a", "b"]
    ops = FakeOps(6, keys, 3)
    for k in ops.pen:
        ops.pen[k] = 0.0  # every region already at the best rate
    rep = search_regions(ops, 6, keys, tries=5, sweeps=1, tol=0.01)
    assert rep[0][3] == 10  # the first region has no rate to compare with
    assert all(r[3] == 0 for r in rep[1:])
    assert ops.live == set(ops.mapped.values())


def test_out_of_memory_for_candidates_ends_the_tries():
    keys = ["a", "b", "c"]
    ops = FakeOps(6, keys, 5, memory=3)
    rep = search_regions(ops, 6, keys, tries=4, sweeps=2, tol=0.0)
    assert sum(r[3] for r in rep) <= 3
    assert ops.live == set(ops.mapped.values())
