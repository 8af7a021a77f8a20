"""A lane-level model of the compact top-p scorer's wave algorithm, on the CPU.

[top-p replay], "Changes" table: the replay kernel validates the replay ids, sorts and
deduplicates up to 64 of them per row and sums over the distinct ones. The GPU scorer does this
with wave primitives: in-shard keys packed into low lanes, a bitonic network over the next
power of two above their count, dedup by comparing with the previous lane, compaction, then a
max and a sum by xor butterflies. It scores 4 rows per wave in 16-lane groups and claims that
each row gets exactly the bits of scoring it with the whole wave. This file models both forms
lane by lane (numpy arrays of 64 lanes, `shfl_xor` / `shfl_up` as permutations) and pins that
claim on random rows, so the grouping's design is checked independently of the GPU. The model
is test infrastructure: it shares no code with the oracle or the HIP library. Both forms use
the same float32 exp, so bitwise equality here tests the order of the operations, which is
what the grouping must preserve.
"""
import numpy as np
import pytest

SENT = 0x7FFFFFFF          # sorts after every local key
LANES = np.arange(64)


def pow2(n):
    p = 1
    while p < n:
        p <<= 1
    return p


def shfl_xor(v, m):
    return v[LANES ^ m]


def shfl_up(v, d):
    idx = LANES - d
    idx[idx < 0] = LANES[idx < 0]          # lanes below d keep their own value
    return v[idx]


def set_sum(z, live, span):
    """Max, then the sum of exp(z - max) over lanes, by xor butterflies of width `span`."""
    M = z.copy()
    off = span >> 1
    while off > 0:
        M = np.maximum(M, shfl_xor(M, off))
        off >>= 1
    with np.errstate(invalid="ignore"):             # dead lanes: -inf - -inf, masked below
        d = (z - M).astype(np.float32)
    e = np.where(live, np.exp(np.where(live, d, 0)).astype(np.float32), np.float32(0))
    off = span >> 1
    while off > 0:
        e = (e + shfl_xor(e, off)).astype(np.float32)
        off >>= 1
    return e, M


def bitonic(key, P, direction_index):
    """Ascending bitonic network over blocks of P lanes; a lane's direction at stage k comes
    from bit k of `direction_index` (its index within the block being sorted)."""
    k = 2
    while k <= P:
        j = k >> 1
        while j > 0:
            other = shfl_xor(key, j)
            up = (direction_index & k) == 0
            lower = (LANES & j) == 0
            key = np.where(lower == up, np.minimum(key, other), np.maximum(key, other))
            j >>= 1
        k <<= 1
    return key


def whole_wave(ids, x, n_real):
    """One row by the whole wave: lane k holds slot k."""
    ins = (ids >= 0) & (ids < n_real)
    c = int(ins.sum())
    key = np.full(64, SENT, np.int64)
    key[:c] = ids[ins]                      # packed in slot order (ballot + mbcnt)
    key = bitonic(key, pow2(c), LANES)
    keep = (key != SENT) & ((LANES == 0) | (key != shfl_up(key, 1)))
    n = int(keep.sum())
    z = np.full(64, -np.inf, np.float32)
    z[:n] = x[key[keep]]
    e, M = set_sum(z, LANES < n, pow2(n))
    return e[0], M[0], n, z[:n].copy()


def grouped(rows_ids, xrows, n_real, direction="group"):
    """Four rows by one wave, 16 lanes each: lane l of group g holds slots l, l+16, l+32, l+48
    of row g. Rows with more than 16 in-shard ids are left to the whole-wave form (wide)."""
    g, gl = LANES >> 4, LANES & 15
    key = np.full(64, SENT, np.int64)
    cnt, wide = [], []
    for r in range(4):
        ids = rows_ids[r]
        order = [l + 16 * s for s in range(4) for l in range(16)]   # the group's slot order
        vals = [ids[s] for s in order if 0 <= ids[s] < n_real]
        cnt.append(len(vals))
        wide.append(len(vals) > 16)
        if len(vals) <= 16:
            key[(g == r) & (gl < len(vals))] = vals
    P = max(pow2(1 if wide[r] else cnt[r]) for r in range(4))
    key = bitonic(key, P, gl if direction == "group" else LANES)
    keep = (key != SENT) & ((gl == 0) | (key != shfl_up(key, 1)))
    z = np.full(64, -np.inf, np.float32)
    n = np.zeros(4, int)
    for r in range(4):
        m = keep & (g == r)
        n[r] = int(m.sum())
        z[16 * r:16 * r + n[r]] = xrows[r][key[m]]
    e, M = set_sum(z, gl < np.repeat(n, 16), max(pow2(v) for v in n))
    return [(e[16 * r], M[16 * r], int(n[r]), wide[r], z[16 * r:16 * r + n[r]].copy())
            for r in range(4)]


def random_batch(rng, n_real, max_in_shard=16):
    rows_ids, xrows = [], []
    for _ in range(4):
        ids = np.full(64, -1, np.int64)
        k = int(rng.integers(0, max_in_shard + 1))
        lst = rng.integers(-3, n_real + 8, k)              # out-of-shard ids and -1 mixed in
        if rng.random() < 0.5:
            lst = np.concatenate([lst, lst[:k // 2]])      # duplicates
        rng.shuffle(lst)
        slots = rng.choice(64, lst.size, replace=False)    # anywhere among the 64 slots
        ids[slots] = lst
        rows_ids.append(ids)
        xrows.append((rng.standard_normal(n_real) * 3).astype(np.float32))
    return rows_ids, xrows


def mismatches(rng, batches, n_real, direction):
    bad = total = 0
    for _ in range(batches):
        rows_ids, xrows = random_batch(rng, n_real)
        for r, (e, M, n, wide, z) in enumerate(grouped(rows_ids, xrows, n_real, direction)):
            if wide:
                continue
            e1, M1, n1, z1 = whole_wave(rows_ids[r], xrows[r], n_real)
            total += 1
            same = n == n1 and z.tobytes() == z1.tobytes() and (
                n == 0 or (np.float32(e).tobytes() == np.float32(e1).tobytes()
                           and np.float32(M).tobytes() == np.float32(M1).tobytes()))
            bad += not same
    return bad, total


def test_grouped_rows_get_the_whole_wave_bits():
    bad, total = mismatches(np.random.default_rng(11), 600, n_real=120, direction="group")
    assert total > 2000
    assert bad == 0


def test_sort_direction_from_the_wave_lane_is_caught():
    # Planted mistake: at the 16-lane stage the direction taken from the lane's index in the
    # wave sorts groups 1 and 3 descending; their compacted logits come out reversed.
    bad, total = mismatches(np.random.default_rng(11), 600, n_real=120, direction="wave")
    assert bad > 0


def test_more_than_16_in_shard_ids_go_to_the_whole_wave():
    rng = np.random.default_rng(3)
    n_real = 500
    rows_ids, xrows = random_batch(rng, n_real, max_in_shard=4)
    rows_ids[2] = np.full(64, -1, np.int64)
    rows_ids[2][:17] = rng.choice(n_real, 17, replace=False)
    res = grouped(rows_ids, xrows, n_real)
    assert [w for (_, _, _, w, _) in res] == [False, False, True, False]
    e, M, n, z = whole_wave(rows_ids[2], xrows[2], n_real)
    assert n == 17
    ref = np.log(np.sum(np.exp(xrows[2][np.sort(rows_ids[2][:17])].astype(np.float64))))
    assert abs(float(M + np.log(e)) - ref) < 1e-5


@pytest.mark.parametrize("n", [0, 1, 2, 5, 16])
def test_whole_wave_sum_is_the_log_sum_exp_of_the_distinct_ids(n):
    rng = np.random.default_rng(n)
    x = (rng.standard_normal(300) * 3).astype(np.float32)
    ids = np.full(64, -1, np.int64)
    distinct = rng.choice(300, n, replace=False)
    lst = np.concatenate([distinct, distinct[:n // 2], [310, -1]])
    ids[rng.choice(64, lst.size, replace=False)] = lst
    e, M, m, z = whole_wave(ids, x, 300)
    assert m == n
    assert np.array_equal(z, x[np.sort(distinct)])
    if n:
        ref = np.log(np.sum(np.exp(x[distinct].astype(np.float64))))
        assert abs(float(M + np.log(e)) - ref) < 1e-5
