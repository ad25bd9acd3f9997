"""CPU model of the packed-sequence planner (k_varlen_plan in generic.hip):
the same block-serial walk -- 256-thread blocks, block-wide exclusive scans,
per-bucket counters taken with atomics (their order is drawn at random here,
since the hardware fixes none) -- with every index the kernel writes
recorded and checked against its array, on well-formed and on malformed
cu_seqlens (decreasing, negative, past the total, a first entry not 0).

What must hold for any input: every write stays inside tab [2 cap],
first [num_seqs + 1], order [cap / sub] and the bucket arrays; every range
of the table lies in [0, total]; first is nondecreasing and ends at the
parts used (<= cap); every dispatched segment index is -1 or < cap / sub.
For well-formed input the parts of each sequence tile it exactly.
"""
import numpy as np
import pytest

NT = 256
NB = 128


class Bounded:
    """An array that records and checks every index written."""

    def __init__(self, n, fill, name):
        self.a = np.full(max(n, 0), fill, dtype=np.int64)
        self.name = name

    def __setitem__(self, i, x):
        assert 0 <= i < len(self.a), f"{self.name}[{i}] written, size {len(self.a)}"
        self.a[i] = x

    def __getitem__(self, i):
        assert 0 <= i < len(self.a), f"{self.name}[{i}] read, size {len(self.a)}"
        return self.a[i]


def seq_bounds(cu, i, total):
    s0 = min(max(int(cu[i]), 0), total)
    s1 = min(max(int(cu[i + 1]), s0), total)
    return s0, s1


def block_exclusive_scan(xs):
    inc = np.cumsum(np.asarray(xs, dtype=np.int64))
    return [int(v) for v in inc - np.asarray(xs, dtype=np.int64)], int(inc[-1])


def plan(cu, num_seqs, total, seg_len, sub, cap, rng):
    """The planner's walk; returns tab, first, order (Bounded)."""
    part_len = seg_len // sub
    seg_cap = cap // sub
    nb = min(NB, (seg_len + 63) // 64)
    tab = Bounded(2 * cap, -7, "tab")
    first = Bounded(num_seqs + 1, -7, "first")
    order = Bounded(seg_cap, -7, "order")
    bucket_n = Bounded(NB, 0, "bucket_n")
    bucket_at = Bounded(NB, 0, "bucket_at")
    for e in range(seg_cap):
        order[e] = -1
    base = full_base = 0
    pending = []  # bucket increments of one block, applied in a random order
    for i0 in range(0, num_seqs, NT):
        ids = range(i0, i0 + NT)
        bounds = [seq_bounds(cu, i, total) if i < num_seqs else (0, 0) for i in ids]
        n = [(s1 - s0 + seg_len - 1) // seg_len * sub if i < num_seqs else 0
             for i, (s0, s1) in zip(ids, bounds)]
        nf = [(s1 - s0) // seg_len if i < num_seqs else 0 for i, (s0, s1) in zip(ids, bounds)]
        off, tot = block_exclusive_scan(n)
        _, ftot = block_exclusive_scan(nf)
        for t, i in enumerate(ids):
            if i >= num_seqs:
                continue
            s0, s1 = bounds[t]
            e0 = base + off[t]
            first[i] = min(e0, cap)
            j = 0
            while j < n[t] and e0 + j < cap:
                x = s0 + j * part_len
                tab[2 * (e0 + j)] = min(x, s1)
                tab[2 * (e0 + j) + 1] = min(x + part_len, s1)
                j += 1
            rem = (s1 - s0) % seg_len
            if rem > 0:
                pending.append(min(nb - 1, (rem - 1) // 64))
        rng.shuffle(pending)
        for b in pending:
            bucket_n[b] = bucket_n[b] + 1
        pending.clear()
        base += tot
        full_base += ftot
    used = min(base, cap)
    first[num_seqs] = used
    for e in range(used, cap):
        tab[2 * e] = 0
        tab[2 * e + 1] = 0
    # bucket offsets, longest partials first
    counts = [bucket_n[nb - 1 - t] if t < nb else 0 for t in range(NT)]
    off, _ = block_exclusive_scan(counts)
    for t in range(nb):
        bucket_at[nb - 1 - t] = min(full_base + off[t], seg_cap)
    fbase = pbase = 0
    for i0 in range(0, num_seqs, NT):
        ids = range(i0, i0 + NT)
        bounds = [seq_bounds(cu, i, total) if i < num_seqs else (0, 0) for i in ids]
        n = [(s1 - s0 + seg_len - 1) // seg_len * sub if i < num_seqs else 0
             for i, (s0, s1) in zip(ids, bounds)]
        nf = [(s1 - s0) // seg_len if i < num_seqs else 0 for i, (s0, s1) in zip(ids, bounds)]
        e0s, tot = block_exclusive_scan(n)
        f0s, ftot = block_exclusive_scan(nf)
        claims = []
        for t, i in enumerate(ids):
            if i >= num_seqs:
                continue
            s0, s1 = bounds[t]
            g0 = min(pbase + e0s[t], cap) // sub  # the parts' offsets scanned again
            f0 = fbase + f0s[t]
            j = 0
            while j < nf[t] and f0 + j < seg_cap and g0 + j < seg_cap:
                order[f0 + j] = g0 + j
                j += 1
            rem = (s1 - s0) % seg_len
            if rem > 0:
                claims.append((min(nb - 1, (rem - 1) // 64), g0, nf[t]))
        rng.shuffle(claims)  # atomicAdd order
        for b, g0, nft in claims:
            pos = bucket_at[b]
            bucket_at[b] = pos + 1
            if pos < seg_cap:
                order[pos] = g0 + nft if g0 + nft < seg_cap else -1
        fbase += ftot
        pbase += tot
    return tab, first, order


def check_invariants(tab, first, order, num_seqs, total, cap, sub):
    t = tab.a.reshape(-1, 2)
    assert np.all(t >= 0) and np.all(t <= total) and np.all(t[:, 0] <= t[:, 1])
    f = first.a
    assert np.all(np.diff(f) >= 0) and 0 <= f[0] and f[-1] <= cap
    o = order.a
    assert np.all((o == -1) | ((o >= 0) & (o < cap // sub)))


def cap_of(total, num_seqs, seg_len, sub):
    # segments of the uniform plan over all tokens, plus one partial per sequence
    return ((total + seg_len - 1) // seg_len + num_seqs) * sub


@pytest.mark.parametrize("seed", range(12))
def test_wellformed_batches_are_tiled_exactly(seed):
    rng = np.random.default_rng(seed)
    num_seqs = int(rng.integers(1, 700))
    lens = rng.integers(0, 3000, num_seqs)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total = int(cu[-1])
    seg_len = 64 * int(rng.integers(1, 40))
    sub = int(rng.integers(1, 3))
    cap = cap_of(total, num_seqs, seg_len, sub)
    tab, first, order = plan(cu, num_seqs, total, seg_len, sub, cap, rng)
    check_invariants(tab, first, order, num_seqs, total, cap, sub)
    t = tab.a.reshape(-1, 2)
    for i in range(num_seqs):
        parts = t[first.a[i]:first.a[i + 1]]
        covered = [p for p in parts if p[1] > p[0]]
        # contiguous, in order, from cu[i] to cu[i + 1]
        pos = cu[i]
        for a, b in covered:
            assert a == pos and b > a
            pos = b
        assert pos == cu[i + 1]
    # every segment with tokens is dispatched exactly once
    segs = {e // sub for e in range(first.a[-1]) if t[e][1] > t[e][0]}
    dispatched = [g for g in order.a if g >= 0]
    assert len(dispatched) == len(set(dispatched)) and segs <= set(dispatched)


@pytest.mark.parametrize("seed", range(40))
def test_malformed_boundaries_stay_in_bounds(seed):
    rng = np.random.default_rng(1000 + seed)
    num_seqs = int(rng.integers(1, 600))
    total = int(rng.integers(0, 200000))
    kind = seed % 4
    if kind == 0:    # arbitrary values, any sign or order
        cu = rng.integers(-5000, total + 5000, num_seqs + 1)
    elif kind == 1:  # decreasing
        cu = np.sort(rng.integers(0, total + 1, num_seqs + 1))[::-1]
    elif kind == 2:  # increasing past the total, first entry not 0
        cu = np.sort(rng.integers(100, 3 * total + 200, num_seqs + 1))
    else:            # extreme int32 values mixed in
        cu = rng.integers(0, total + 1, num_seqs + 1)
        cu[rng.integers(0, num_seqs + 1, 5)] = np.iinfo(np.int32).max
        cu[rng.integers(0, num_seqs + 1, 5)] = np.iinfo(np.int32).min
    cu = cu.astype(np.int32)
    seg_len = 64 * int(rng.integers(1, 130))
    sub = int(rng.integers(1, 3))
    cap = cap_of(total, num_seqs, seg_len, sub)
    tab, first, order = plan(cu, num_seqs, total, seg_len, sub, cap, rng)
    check_invariants(tab, first, order, num_seqs, total, cap, sub)
