"""A host model of the pipelined forward kernel's schedule (bsfa_fwd_pipe.h),
checked for races on its LDS tiles and vote slots.

The kernel keeps two K tiles, two V tiles and two vote slots in LDS, chosen
by step parity, and has one workgroup barrier per step.  The model lists, for
one workgroup, every request (direct-to-LDS load) and every read of those
buffers with the barrier epoch it happens in (epoch e = after the e-th
barrier); each wave waits for its own loads before every barrier, so a load
issued in epoch e has landed by epoch e + 1.  Inside an epoch the waves run in
any order, so the checks are:

* a read in epoch e finds the expected tile, written by a load issued in an
  earlier epoch, and no load into that buffer is issued in epoch e;
* a load into a buffer in epoch e meets no read of that buffer in epoch e;
* a vote slot read in epoch e was written in epoch e - 1 and is not written
  again in epoch e.

Step j of the kernel: phase A (epoch j + 1) reads K_j and writes the votes of
tile j; phase B (epoch j + 2) requests K_{j+2} into K_j's tile, reads the votes,
requests V_j when some unit keeps tile j, and reads V_{j-1} in each unit that
kept tile j - 1.  Tile t lives in buffer (t + p) mod 2, p the parity of the last
step.  After the last step, one more barrier if it requested V, then the last
P~V.  Causal attention: the last step is the diagonal, kept by both units, and
requests no K.  Every (last step, keep pattern) combination up to 9 steps is
checked, for head pairs (one diagonal) and block pairs (the second unit's
diagonal one step later, bidirectional and causal).

The kernel is persistent: in phase B of an item's last step it requests the
next item's K_0 and K_1 into the two K buffers (by that item's own parity),
and one more barrier starts the next item, whose step 0 reads K_0 and step 1
K_1.  With ``next_send`` the model appends those loads and reads.
"""

import itertools

import pytest


def schedule(send, keep, causal, next_send=None):
    """Events (epoch, kind, buffer, tile) of one workgroup.

    keep[u][j]: unit u keeps tile j (diagonal tiles included); next_send: the
    last step of the next item, whose first two K tiles are prefetched."""
    par = send & 1
    kbuf = lambda t: ("K", (t + par) & 1)
    vbuf = lambda t: ("V", (t + par) & 1)
    slot = lambda t: ("vote", (t + par) & 1)
    ev = [(0, "load", kbuf(0), 0)]                  # prologue, then the first barrier
    if send >= 1:
        ev.append((1, "load", kbuf(1), 1))
    kept_prev = [False, False]
    vmask = False
    for j in range(send + 1):
        a, b = j + 1, j + 2                         # epochs of phases A and B
        ev.append((a, "read", kbuf(j), j))
        ev.append((a, "write", slot(j), j))
        if not (causal and j == send) and j + 2 <= send:
            ev.append((b, "load", kbuf(j + 2), j + 2))
        ev.append((b, "readvote", slot(j), j))
        vmask = keep[0][j] or keep[1][j]
        if vmask:
            ev.append((b, "load", vbuf(j), j))
        for u in (0, 1):
            if kept_prev[u]:
                ev.append((b, "read", vbuf(j - 1), j - 1))
        kept_prev = [keep[0][j], keep[1][j]]
    end = send + 2                                   # epoch of the last step's phase B
    if vmask:                                        # drain
        end += 1
        for u in (0, 1):
            if kept_prev[u]:
                ev.append((send + 3, "read", vbuf(send), send))
    if next_send is not None:
        npar = next_send & 1
        nk = lambda t: ("K", (t + npar) & 1)
        ev.append((send + 2, "load", nk(0), ("next", 0)))
        if next_send >= 1:
            ev.append((send + 2, "load", nk(1), ("next", 1)))
        start = end + 1                              # after the item barrier
        ev.append((start, "read", nk(0), ("next", 0)))   # next item's step 0, phase A
        if next_send >= 1:
            ev.append((start + 1, "read", nk(1), ("next", 1)))  # its step 1 (after step 0's barrier)
            if next_send >= 2:
                ev.append((start + 1, "load", nk(2), ("next", 2)))  # K_2 requested in step 0's phase B
    return ev


def check(ev):
    loads = [e for e in ev if e[1] == "load"]
    for epoch, kind, buf, tile in ev:
        if kind == "read":
            before = [l for l in loads if l[2] == buf and l[0] < epoch]
            assert before, f"read of {buf} in epoch {epoch} before any load"
            last = max(before, key=lambda l: l[0])
            assert last[3] == tile, f"epoch {epoch}: {buf} holds tile {last[3]}, tile {tile} expected"
            assert not [l for l in loads if l[2] == buf and l[0] == epoch], \
                f"epoch {epoch}: {buf} loaded while it is read"
        elif kind == "load":
            reads = [r for r in ev if r[1] == "read" and r[2] == buf and r[0] == epoch]
            assert not reads, f"epoch {epoch}: load into {buf} races with a read"
        elif kind == "readvote":
            writes = [w for w in ev if w[1] == "write" and w[2] == buf]
            assert [w for w in writes if w[0] == epoch - 1 and w[3] == tile], f"epoch {epoch}: votes of {tile} missing"
            assert not [w for w in writes if w[0] == epoch], f"epoch {epoch}: vote slot {buf} rewritten while read"


def _patterns(n):
    return itertools.product((False, True), repeat=n)


@pytest.mark.parametrize("send", range(0, 9))
def test_head_pair_schedule_has_no_race(send):
    # both units share the query block: off-diagonal tiles 0..send-1 free, the
    # last tile kept (causal diagonal); bidirectional layers take the diagonal
    # anywhere, so every step is free there
    n = send + 1
    for causal in (True, False):
        for k0 in _patterns(n):
            for k1 in ([k0] if n > 6 else _patterns(n)):
                keep = [list(k0), list(k1)]
                if causal:
                    keep[0][send] = keep[1][send] = True
                check(schedule(send, keep, causal))


@pytest.mark.parametrize("send", range(1, 9))
def test_block_pair_schedule_has_no_race(send):
    # bidirectional block pairs: query blocks 2i and 2i + 1 keep their own
    # diagonal tiles, one step apart
    n = send + 1
    for d0 in range(0, send):
        for k in _patterns(n):
            keep = [list(k), list(reversed(k))]
            keep[0][d0] = True
            keep[1][d0 + 1] = True
            check(schedule(send, keep, False))


@pytest.mark.parametrize("send", range(1, 9))
def test_causal_block_pair_schedule_has_no_race(send):
    # causal block pairs: the first unit's diagonal is the step before the
    # last (kept), the second unit's the last step (kept); the first unit has
    # no tile in the last step
    n = send + 1
    for k in _patterns(n):
        keep = [list(k), list(reversed(k))]
        keep[0][send - 1] = True
        keep[0][send] = False
        keep[1][send] = True
        check(schedule(send, keep, True))


def test_model_detects_a_shifted_buffer_choice():
    # a schedule whose V_j load goes into V_{j-1}'s tile races with the P~V of
    # tile j - 1 in the same epoch: the checker must say so
    def bad(send, keep):
        ev = schedule(send, keep, False)
        par = send & 1
        out = []
        for e in ev:
            if e[1] == "load" and e[2][0] == "V":
                e = (e[0], e[1], ("V", (e[3] - 1 + par) & 1), e[3])
            out.append(e)
        return out
    with pytest.raises(AssertionError):
        check(bad(4, [[True] * 5, [True] * 5]))


def test_model_detects_a_missing_barrier_between_k_load_and_use():
    # requesting K_{j+1} (instead of K_{j+2}) in phase B of step j would need it
    # in the very next phase, before any barrier: the checker must say so
    def bad(send, keep):
        ev = [e for e in schedule(send, keep, False) if not (e[1] == "load" and e[2][0] == "K" and e[3] >= 2)]
        par = send & 1
        for j in range(send):
            ev.append((j + 2, "load", ("K", (j + 1 + par) & 1), j + 1))
        return ev
    with pytest.raises(AssertionError):
        check(bad(4, [[True] * 5, [True] * 5]))


@pytest.mark.parametrize("send", range(0, 7))
@pytest.mark.parametrize("next_send", range(0, 4))
def test_next_item_prefetch_has_no_race(send, next_send):
    # the next item's K_0 and K_1, requested in the last step's phase B, meet
    # no read of their buffers and are what the next item's first steps read
    n = send + 1
    for causal in (True, False):
        for k in _patterns(n):
            keep = [list(k), list(k)]
            if causal:
                keep[0][send] = keep[1][send] = True
            check(schedule(send, keep, causal, next_send))


def test_model_detects_a_prefetch_before_the_last_read():
    # requesting the next item's K tiles in phase A of the last step would
    # overwrite the tile that step is reading
    ev = schedule(3, [[True] * 4, [True] * 4], True, next_send=2)
    ev = [(e[0] - 1, e[1], e[2], e[3]) if e[1] == "load" and isinstance(e[3], tuple) and e[3][1] < 2 else e
          for e in ev]
    with pytest.raises(AssertionError):
        check(ev)
