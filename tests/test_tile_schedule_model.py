"""A model of how the GEMM kernels hand out their tiles, on the CPU.

The forward runs one persistent worker per compute unit; the backward GEMM kernels run 1.25
workgroups per tile. Either way the tiles of a launch are split into 8 contiguous per-XCD
queues. A queue's first three quarters go out by position with no synchronisation; its last
quarter goes out one tile at a time through a counter, own XCD first and then the others',
with a flag once every queue is empty. A tile's arithmetic does not depend on who runs it, so
the results are right if every tile runs exactly once, whatever order the claims race in.

This file models those rules in plain Python. The split into queues and the vocabulary-major
tile order within a group follow the kernels' definitions. Workers make their claims in a
random interleaving. The tests check on many grids and schedules that:
- every tile runs exactly once;
- every worker ends;
- a planted mistake (a dynamic part that overlaps the static part) is caught.
The model is test infrastructure and shares no code with the kernels.
"""
import numpy as np
import pytest

NUM_XCD = 8


def queue_first(n, x):
    full, rem = divmod(n, NUM_XCD)
    return x * full + min(x, rem)


def queue_size(n, x):
    return n // NUM_XCD + (1 if x < n % NUM_XCD else 0)


def queue_static(size, quarter=4):
    return size - (size + quarter - 1) // quarter


class Counters:
    """The launch's counters: one per XCD queue, then the all-empty flag."""

    def __init__(self, n, static_of=queue_static):
        self.n = n
        self.ctr = [0] * (NUM_XCD + 1)
        self.static_of = static_of

    def claim(self, x):
        """One dynamic tile for a worker of XCD x, or -1 (the kernels' claim, atomics as +=)."""
        n = self.n
        k = self.ctr[x]
        self.ctr[x] += 1
        if k < queue_size(n, x) - self.static_of(queue_size(n, x)):
            return queue_first(n, x) + self.static_of(queue_size(n, x)) + k
        if self.ctr[NUM_XCD] == 0:
            for d in range(1, NUM_XCD):
                y = (x + d) % NUM_XCD
                sy = self.static_of(queue_size(n, y))
                k = self.ctr[y]
                self.ctr[y] += 1
                if k < queue_size(n, y) - sy:
                    return queue_first(n, y) + sy + k
            self.ctr[NUM_XCD] = 1
        return -1


def persistent_workers(n, workers, rng, static_of=queue_static):
    """The forward: worker w of XCD w % 8 walks positions w / 8, + nwx, ... of its queue's
    static part, then claims. Returns the tiles in the order each worker ran them."""
    grid = -(-min(workers, n) // NUM_XCD) * NUM_XCD
    nwx = grid // NUM_XCD
    cn = Counters(n, static_of)
    state = []
    for b in range(grid):
        x = b % NUM_XCD
        state.append(dict(x=x, pos=b // NUM_XCD, s0=static_of(queue_size(n, x)),
                          qf=queue_first(n, x), done=False, ran=[]))
    live = list(range(grid))
    while live:
        b = live[rng.integers(len(live))]        # any worker may be next to need a tile
        st = state[b]
        if st["pos"] < st["s0"]:
            st["ran"].append(st["qf"] + st["pos"])
            st["pos"] += nwx
            continue
        t = cn.claim(st["x"])
        if t < 0:
            live.remove(b)
        else:
            st["ran"].append(t)
    return [s["ran"] for s in state]


def workgroup_per_tile(n, rng, oversubscribe=(5, 4)):
    """The backward kernels: workgroup b of XCD b % 8 takes position b / 8 of its queue's
    static part, else claims one tile (or none). Workgroups start in any order."""
    grid = -(-n * oversubscribe[0] // oversubscribe[1])
    cn = Counters(n)
    ran = []
    for b in rng.permutation(grid):
        x, i = b % NUM_XCD, b // NUM_XCD
        s0 = queue_static(queue_size(n, x))
        t = queue_first(n, x) + i if i < s0 else cn.claim(x)
        if t >= 0:
            ran.append(t)
    return ran


def vocab_token_tile(tile, nvt, ntb, vg):
    grp, gi = divmod(tile, vg * ntb)
    gsz = min(vg, nvt - grp * vg)
    return grp * vg + gi % gsz, gi // gsz


GRIDS = [1, 7, 8, 9, 63, 255, 256, 257, 1000, 9488, 9504]


@pytest.mark.parametrize("n", GRIDS)
def test_queues_partition_the_tiles(n):
    starts = [queue_first(n, x) for x in range(NUM_XCD)]
    sizes = [queue_size(n, x) for x in range(NUM_XCD)]
    assert sum(sizes) == n
    assert all(starts[x] + sizes[x] == (starts[x + 1] if x + 1 < NUM_XCD else n)
               for x in range(NUM_XCD))


@pytest.mark.parametrize("n", GRIDS)
@pytest.mark.parametrize("workers", [8, 256, 304])
def test_persistent_workers_run_every_tile_once(n, workers):
    rng = np.random.default_rng(n * 1000 + workers)
    for _ in range(5):
        ran = persistent_workers(n, workers, rng)
        flat = sorted(t for r in ran for t in r)
        assert flat == list(range(n))


@pytest.mark.parametrize("n", GRIDS)
def test_workgroup_per_tile_runs_every_tile_once(n):
    rng = np.random.default_rng(n)
    for _ in range(5):
        assert sorted(workgroup_per_tile(n, rng)) == list(range(n))


def test_static_part_keeps_the_round_order():
    # With no claims interleaved, worker w's static tiles are positions w/8, w/8 + nwx, ...: the
    # order in which one workgroup per tile would have started them, 32 per XCD round.
    n, workers = 9488, 256
    ran = persistent_workers(n, workers, np.random.default_rng(0))
    for b in (0, 9, 255):
        x, w = b % NUM_XCD, b // NUM_XCD
        s0 = queue_static(queue_size(n, x))
        static = [t for t in ran[b] if t < queue_first(n, x) + s0]
        assert static == [queue_first(n, x) + p for p in range(w, s0, workers // NUM_XCD)]


def test_round_of_32_tiles_shares_8_weight_and_4_hidden_slices():
    # Vocabulary-major groups of 8: each XCD round of 32 consecutive positions covers 8
    # vocabulary tiles x 4 token blocks.
    nvt, ntb = 593, 16
    for r in range(8):
        tiles = [vocab_token_tile(t, nvt, ntb, 8) for t in range(32 * r, 32 * r + 32)]
        assert len({v for v, _ in tiles}) == 8 and len({b for _, b in tiles}) == 4
    # and the order is a bijection onto the grid
    seen = {vocab_token_tile(t, nvt, ntb, 8) for t in range(nvt * ntb)}
    assert seen == {(v, b) for v in range(nvt) for b in range(ntb)}


def test_overlapping_dynamic_part_is_caught():
    # Planted mistake: the dynamic part starts one tile early, inside the static part.
    def bad_static(size, quarter=4):
        return max(0, queue_static(size, quarter) - 1)
    n, workers = 1000, 256
    rng = np.random.default_rng(5)
    grid = -(-min(workers, n) // NUM_XCD) * NUM_XCD
    nwx = grid // NUM_XCD
    cn = Counters(n, bad_static)
    ran = []
    for b in range(grid):      # the static walk as the kernels have it, then the bad claims
        x = b % NUM_XCD
        s0 = queue_static(queue_size(n, x))
        ran += [queue_first(n, x) + p for p in range(b // NUM_XCD, s0, nwx)]
    while True:
        t = cn.claim(int(rng.integers(NUM_XCD)))
        if t < 0:
            break
        ran.append(t)
    assert sorted(ran) != list(range(n))
