"""A host model of the pipelined kernel's work queues (next_item in
bsfa_fwd_kernels.h), run under random interleavings of its atomic adds.

A launch over n work items keeps eight counters, one per XCD queue; queue x
holds the items L < n with L % 8 == x in increasing order (heaviest first).
Each counter packs the items taken from its queue's front (high 32 bits) and
back (low 32 bits).  Each persistent workgroup repeatedly asks for an item: it
claims the front of its own XCD's queue, then the back of the next ones in
turn, with one atomic add per try, and leaves once a full pass finds every
queue empty.  The model runs each request as a generator that yields after
every atomic add, and a scheduler that picks which workgroup's next add
happens, so that adds from different workgroups interleave in any order.
Checked: every item is taken exactly once, every workgroup leaves, a queue's
front hands out its items in increasing order and its back in decreasing
order, and a workgroup takes from other queues only once its own is empty.
"""

import random

import pytest


def next_item(counters, n, xcd, log):
    """One request: yields after each atomic add, returns the item or -1.
    log records (xcd, queue, position handed out or None) in the order of
    the adds."""
    for t in range(8):
        x = (xcd + t) & 7
        nq = (n - x + 7) >> 3
        if nq <= 0:
            continue
        old = counters[x]
        counters[x] += (1 << 32) if t == 0 else 1  # the 64-bit atomic add
        front, back = old >> 32, old & 0xFFFFFFFF
        pos = (front if t == 0 else nq - 1 - back) if front + back < nq else None
        log.append((xcd, x, pos))
        yield
        if pos is not None:
            return pos * 8 + x
    return -1


def simulate(n, n_wg, seed, next_fn=next_item, xcd_of=lambda g: g % 8, weights=None):
    """Run n_wg persistent workgroups to the end; returns (items taken, the
    adds in order, counters)."""
    rng = random.Random(seed)
    counters = [0] * 8
    taken = []
    log = []

    def wg(xcd):
        while True:
            item = yield from next_fn(counters, n, xcd, log)
            if item < 0:
                return
            taken.append((xcd, item))
            yield  # the item's work, during which other workgroups go on

    live = {g: wg(xcd_of(g)) for g in range(n_wg)}
    steps = 0
    while live:
        g = rng.choices(list(live), weights=[(weights or {}).get(k, 1.0) for k in live])[0]
        try:
            next(live[g])
        except StopIteration:
            del live[g]
        steps += 1
        assert steps < 100 * (n + 8) * max(n_wg, 1), "a workgroup does not leave"
    return taken, log, counters


@pytest.mark.parametrize("n", [1, 5, 8, 13, 64, 255, 1000])
@pytest.mark.parametrize("n_wg", [1, 7, 32, 256])
def test_every_item_taken_once(n, n_wg):
    for seed in range(3):
        taken, log, counters = simulate(n, min(n_wg, n), seed)
        items = sorted(item for _, item in taken)
        assert items == list(range(n))
        for x in range(8):
            nq = (n - x + 7) // 8
            # the front handed out 0, 1, 2, ... and the back nq-1, nq-2, ...
            front = [pos for xcd, q, pos in log if q == x and pos is not None and xcd == x]
            back = [pos for xcd, q, pos in log if q == x and pos is not None and xcd != x]
            assert front == list(range(len(front)))
            assert back == list(range(nq - 1, nq - 1 - len(back), -1))
            # every counter ran past its queue (the last pass found it empty)
            assert (counters[x] >> 32) + (counters[x] & 0xFFFFFFFF) >= nq


def test_own_queue_first():
    # a workgroup takes an item from another XCD's queue only after its own
    # queue has run out (the share the static grid would give its XCD)
    _, log, _ = simulate(400, 64, seed=1, weights={g: (3.0 if g % 8 == 2 else 1.0) for g in range(64)})
    stole = 0
    for at, (xcd, q, pos) in enumerate(log):
        if q != xcd and pos is not None:
            stole += 1
            own_later = [p for x, qq, p in log[at:] if qq == xcd and p is not None]
            assert not own_later, f"XCD {xcd} took from queue {q} before its own queue ran out"
    assert stole > 0


def test_stolen_items_are_the_lightest_left():
    # XCD 0 runs three times as fast: what it takes from the other queues at
    # the end comes from their backs, the highest positions (lightest items)
    taken, log, _ = simulate(4096, 64, seed=3, weights={g: (3.0 if g % 8 == 0 else 1.0) for g in range(64)})
    nq = 512
    stolen = [pos for xcd, q, pos in log if xcd != q and pos is not None]
    assert stolen and min(stolen) > nq // 2


def test_fast_xcd_takes_more():
    # workgroups of XCD 0 run three times as often as the others: they end up
    # with more than their eighth of the items (what the queues are for)
    taken, _, _ = simulate(2048, 64, seed=2, weights={g: (3.0 if g % 8 == 0 else 1.0) for g in range(64)})
    share = sum(1 for xcd, _ in taken if xcd == 0) / len(taken)
    assert share > 0.2


def _variant(nq_of, valid, pos_of):
    def f(counters, n, xcd, log):
        for t in range(8):
            x = (xcd + t) & 7
            nq = nq_of(n, x)
            if nq <= 0:
                continue
            old = counters[x]
            counters[x] += (1 << 32) if t == 0 else 1
            front, back = old >> 32, old & 0xFFFFFFFF
            pos = pos_of(t, front, back, nq) if valid(front, back, nq) else None
            log.append((xcd, x, pos))
            yield
            if pos is not None:
                return pos * 8 + x
        return -1
    return f


def test_model_detects_a_wrong_queue_length():
    # a queue length computed as n // 8 drops the tail items of the first queues
    bad = _variant(lambda n, x: n >> 3, lambda f, b, nq: f + b < nq, lambda t, f, b, nq: f if t == 0 else nq - 1 - b)
    taken, _, _ = simulate(13, 4, seed=0, next_fn=bad)
    assert sorted(item for _, item in taken) != list(range(13))


def test_model_detects_an_off_by_one_bound():
    # front + back <= nq hands out one item twice or past the end
    bad = _variant(lambda n, x: (n - x + 7) >> 3, lambda f, b, nq: f + b <= nq,
                   lambda t, f, b, nq: f if t == 0 else nq - 1 - b)
    taken, _, _ = simulate(13, 4, seed=0, next_fn=bad)
    assert sorted(item for _, item in taken) != list(range(13))


def test_model_detects_a_bound_that_ignores_the_other_end():
    # a front claim checked against the front count alone meets the back claims
    bad = _variant(lambda n, x: (n - x + 7) >> 3, lambda f, b, nq: (f < nq) and (b < nq),
                   lambda t, f, b, nq: f if t == 0 else nq - 1 - b)
    taken, _, _ = simulate(200, 32, seed=4, next_fn=bad, weights={g: (4.0 if g % 8 == 1 else 1.0) for g in range(32)})
    assert sorted(item for _, item in taken) != list(range(200))
