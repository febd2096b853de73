"""The stream-K schedule's arithmetic (CPU model of the kernel's integer steps).

W workers share I = tiles x nk iterations: worker w owns [start(w), start(w+1)) with
start(w) = w q + min(w, r), I = q W + r, and walks its tiles in decreasing order.
The model checks what the kernel relies on: every iteration is owned exactly once,
no range is empty, a worker leaves at most one partial tile (the first one it
processes), a finisher's contributors are exactly the other owners of its tile and
all of them have lower numbers (so waits never go upward), and the owner formula
inverts the ranges.
"""
import pytest


def start(w, q, r):
    return w * q + min(w, r)


def owner(i, q, r):
    big = r * (q + 1)
    return i // (q + 1) if i < big else r + (i - big) // q


def schedule(tiles, nk, W):
    I = tiles * nk
    W = min(W, I)  # the host never launches more workers than iterations
    q, r = divmod(I, W)
    items = {}
    for w in range(W):
        s0, e0 = start(w, q, r), start(w + 1, q, r)
        assert s0 < e0
        order = []
        for t in range((e0 - 1) // nk, s0 // nk - 1, -1):  # decreasing tiles
            ts = t * nk
            kb, ke = max(s0, ts) - ts, min(e0, ts + nk) - ts
            order.append((t, kb, ke))
        items[w] = order
    return I, W, q, r, items


@pytest.mark.parametrize("tiles,nk,W", [(240, 33, 256), (480, 33, 256), (1, 4, 256), (4, 128, 256),
                                        (7, 3, 5), (1000, 64, 256), (3, 1, 256), (256, 16, 256),
                                        (17, 19, 8), (2048, 64, 256)])
def test_schedule_invariants(tiles, nk, W):
    I, W, q, r, items = schedule(tiles, nk, W)
    seen = [0] * I
    partials = {}
    for w, order in items.items():
        for n, (t, kb, ke) in enumerate(order):
            assert 0 <= kb < ke <= nk
            for k in range(kb, ke):
                seen[t * nk + k] += 1
            if ke < nk:  # not the finisher: only the first tile it processes
                assert n == 0, (w, order)
                assert w not in partials
                partials[w] = t
    assert seen == [1] * I
    for i in range(I):
        o = owner(i, q, r)
        assert start(o, q, r) <= i < start(o + 1, q, r)
    for w, order in items.items():
        for t, kb, ke in order:
            if ke == nk and kb > 0:  # finisher with contributors
                contributors = list(range(owner(t * nk, q, r), w))
                assert contributors and all(v < w for v in contributors)
                assert all(partials.get(v) == t for v in contributors)
    # every partial is consumed by exactly one finisher
    finishers = {}
    for w, order in items.items():
        for t, kb, ke in order:
            if ke == nk:
                finishers[t] = w
    for v, t in partials.items():
        assert finishers[t] > v
