"""CPU model of the per-head scan over packed sequences
(k_segment_scan_varlen_heads in generic.hip), one state element: the head's
parts split into P consecutive ranges, each range's last sequence summed
within the range (from its starting state when it starts there), the
carries formed in range order (a range whose last sequence starts inside it
restarts the carry), then each range's prefixes written from its carry.
Every read and write is bounds-checked.  The starting and final states
share one array (the library updates the caller's state in place), and the
ranges' second passes run first to last and last to first: a range must not
read a starting state that another range has already replaced by a final
one.

Checked against the plain definition -- each sequence walks its own parts
from its starting state, writing the exclusive prefix at every
prefix_stride-th part and ending with its total -- on integer-valued data
(so the sums are exact whatever their order), for every range count the
launcher uses, with empty sequences, sequences cut at the part capacity
(first[i] clamped to it) and prefix strides 0, 1, 2 and 4.
"""
import numpy as np
import pytest


class Bounded:
    def __init__(self, a, name):
        self.a = np.array(a, dtype=np.float64)
        self.name = name

    def __setitem__(self, i, x):
        assert 0 <= i < len(self.a), f"{self.name}[{i}] written, size {len(self.a)}"
        self.a[i] = x

    def __getitem__(self, i):
        assert 0 <= i < len(self.a), f"{self.name}[{i}] read, size {len(self.a)}"
        return self.a[i]


def seq_of(first, ns, g):
    lo, hi = 0, ns - 1
    while lo < hi:
        mid = (lo + hi + 1) >> 1
        if first[mid] <= g:
            lo = mid
        else:
            hi = mid - 1
    return lo


def model(first, inc, start0, P, stride, batch=16, order=1):
    """order: 1 runs the ranges' second passes first to last, -1 last to
    first (the hardware fixes no order between them)."""
    ns = len(first) - 1
    parts = len(inc)
    ws = Bounded(inc, "ws")
    # the starting states and the final states share one array, as when the
    # library updates the caller's state in place
    state = Bounded(start0, "state")
    done = [False] * ns

    def start(i):
        return state[i]

    def finish(i, v):
        assert 0 <= i < ns and not done[i], f"sequence {i} finished twice"
        done[i] = True
        state[i] = v

    Pn = min(first[ns], parts)
    per = (Pn + P - 1) // P
    rng = [(min(Pn, k * per), min(Pn, min(Pn, k * per) + per)) for k in range(P)]
    tails, restarts, lasts = [], [], []
    for g0, g1 in rng:
        n0 = min(batch, g1 - g0)
        gl = g0 if g1 > g0 else 0
        a = [ws[gl + (j if j < n0 else 0)] for j in range(batch)]
        tail, restart, il, start_last = 0.0, False, -1, 0.0
        if g1 > g0:
            il = seq_of(first, ns, g1 - 1)
            fl = first[il]
            restart = fl >= g0
            start_last = start(il) if restart else 0.0
            tail = start_last
            for j in range(batch):
                if j < n0 and g0 + j >= fl:
                    tail += a[j]
            for g in range(max(g0 + batch, fl), g1):
                tail += ws[g]
        tails.append(tail)
        restarts.append(restart)
        lasts.append((il, start_last))
    # (the barrier)
    for part in range(P)[::order]:
        g0, g1 = rng[part]
        carry = 0.0
        for u in range(part):
            carry = tails[u] if restarts[u] else carry + tails[u]
        for i in range(part, ns, P):
            if first[i + 1] <= first[i]:
                finish(i, start(i))
        if g1 <= g0:
            continue
        il, start_last = lasts[part]

        def start_of(i):
            return start_last if i == il else start(i)

        i = seq_of(first, ns, g0)
        sf, se = first[i], first[i + 1]
        run = start_of(i) if sf == g0 else carry
        for g in range(g0, g1):
            x = inc[g]
            if stride > 0 and ((g - sf) & (stride - 1)) == 0:
                ws[g] = run
            run += x
            if g + 1 >= se:
                finish(i, run)
                if g + 1 < g1:
                    i = seq_of(first, ns, g + 1)
                    sf, se = first[i], first[i + 1]
                    run = start_of(i)
    assert all(done)
    return ws.a, list(state.a)


def plain(first, inc, start, stride):
    ws = np.array(inc, dtype=np.float64)
    fin = []
    for i in range(len(first) - 1):
        run = start[i]
        for g in range(first[i], first[i + 1]):
            if stride > 0 and ((g - first[i]) & (stride - 1)) == 0:
                ws[g] = run
            run += inc[g]
        fin.append(run)
    return ws, fin


@pytest.mark.parametrize("seed", range(6))
def test_range_split_scan_equals_per_sequence_walk(seed):
    g = np.random.default_rng(400 + seed)
    for _ in range(150):
        ns = int(g.integers(1, 40))
        cnt = g.integers(0, 12, size=ns)
        cnt[g.random(ns) < 0.3] = 0
        total = int(cnt.sum())
        cap = int(g.integers(1, total + 3))  # below the total: sequences cut at the capacity
        first = [int(min(x, cap)) for x in np.concatenate([[0], np.cumsum(cnt)])]
        inc = g.integers(-5, 6, size=cap).astype(np.float64)
        start = g.integers(-100, 100, size=ns).astype(np.float64)
        stride = int(g.choice([0, 1, 2, 4]))
        want_ws, want_fin = plain(first, inc, start, stride)
        for P in (1, 2, 4, 8, 16):
            for order in (1, -1):
                ws, fin = model(first, inc, start, P, stride, order=order)
                assert np.array_equal(ws, want_ws), (P, order, first, stride)
                assert fin == want_fin, (P, order, first, stride)
