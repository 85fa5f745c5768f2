"""CPU model of the main launch's role assignment (static_role and
take_role in the kernels).

Static roles (default): workgroup index -> role.  The model checks that each
consumer's producers have lower indices, on the same XCD (index mod 8) when
8 divides BH, or that every producer-class index precedes every
consumer-class index when heads spread over XCDs; so with each XCD
dispatching in index order, producers are dispatched before anyone waits on
them.

Tickets (LAPATTN_FLAG_TICKETS): roles are handed out per queue in ticket
order: a queue's solvers, then per head its key units, then its query units.
The model walks many plan shapes and checks that
  * every role of the launch is handed out exactly once, and each queue has
    exactly as many workgroups as tickets;
  * every wait inside the launch is on a producer with an earlier ticket of
    the same queue (so the producer has started before anyone waits on it):
    query units wait for the head's key units, for the W^T slices of the
    head's first `nslice` query units and for the head's solver;
  * the one exception, the slice exchange among the first `nslice` query
    units of a head, spans consecutive tickets, at most 32 of them.
"""
import itertools

import pytest

MP = 64


def n_queues(BH):
    return 8 if BH % 8 == 0 else min(BH, 8)


def queue_sizes(BH, per, grid):
    nq = n_queues(BH)
    sizes = [((BH - x + nq - 1) // nq) * per for x in range(nq)]
    assert sum(sizes) == grid
    return sizes


def block_queue(b, BH, per):
    """Queue of workgroup index b (the kernel's mapping)."""
    nq = n_queues(BH)
    if nq == 8 and BH % 8 == 0:
        return b & 7
    start = 0
    for x in range(nq - 1):
        size = ((BH - x + nq - 1) // nq) * per
        if b < start + size:
            return x
        start += size
    return nq - 1


def role(BH, nP, nQ, with_solver, x, t):
    """Role of ticket t of queue x (the kernel's mapping)."""
    nq = n_queues(BH)
    nh = (BH - x + nq - 1) // nq
    ns = nh if with_solver else 0
    if t < ns:
        return ("solver", x + nq * t, 0)
    i = t - ns
    head, u = x + nq * (i // (nP + nQ)), i % (nP + nQ)
    return ("key", head, u) if u < nP else ("query", head, u - nP)


def nslice(D, nQ):
    lines = D * MP // 32
    R = min(nQ, 32)
    lps = -(-lines // R)
    return -(-lines // lps)


SHAPES = list(itertools.product((1, 3, 8, 9, 16, 150),
                                (1, 17, 25, 86, 128),
                                (0, 1, 25, 128),
                                (16, 64),
                                (True, False)))


@pytest.mark.parametrize("BH,nP,nQ,D,with_solver", SHAPES)
def test_every_wait_is_on_an_earlier_ticket(BH, nP, nQ, D, with_solver):
    per = (1 if with_solver else 0) + nP + nQ
    grid = BH * per
    sizes = queue_sizes(BH, per, grid)
    # workgroup count per queue equals its ticket count
    counts = [0] * len(sizes)
    for b in range(grid):
        counts[block_queue(b, BH, per)] += 1
    assert counts == sizes
    ticket = {}
    for x, size in enumerate(sizes):
        for t in range(size):
            r = role(BH, nP, nQ, with_solver, x, t)
            assert r not in ticket, f"role {r} handed out twice"
            ticket[r] = (x, t)
    expect = {("key", h, u) for h in range(BH) for u in range(nP)}
    expect |= {("query", h, u) for h in range(BH) for u in range(nQ)}
    if with_solver:
        expect |= {("solver", h, 0) for h in range(BH)}
    assert set(ticket) == expect
    ns = nslice(D, nQ) if nQ else 0
    for h in range(BH):
        for u in range(nQ):
            xq, tq = ticket[("query", h, u)]
            producers = [("key", h, k) for k in range(nP)]
            if with_solver:
                producers.append(("solver", h, 0))
            producers += [("query", h, s) for s in range(min(ns, u))]
            for p in producers:
                xp, tp = ticket[p]
                assert xp == xq and tp < tq, f"{('query', h, u)} waits on later {p}"
        if ns:
            ts = sorted(ticket[("query", h, s)][1] for s in range(ns))
            assert ts == list(range(ts[0], ts[0] + ns)) and ns <= 32


def static_role(BH, nP, nQ, with_solver, b):
    """Role of workgroup index b without tickets (the kernel's mapping)."""
    ns = BH if with_solver else 0
    if b < ns:
        return ("solver", b, 0)
    b -= ns
    if BH % 8 == 0:
        per = nP + nQ
        x, i = b % 8, b // 8
        head, u = 8 * (i // per) + x, i % per
        return ("key", head, u) if u < nP else ("query", head, u - nP)
    if b < BH * nP:
        return ("key", b // nP, b % nP)
    bq = b - BH * nP
    return ("query", bq // nQ, bq % nQ)


@pytest.mark.parametrize("BH,nP,nQ,D,with_solver", SHAPES)
def test_static_roles_put_producers_first(BH, nP, nQ, D, with_solver):
    ns_blocks = BH if with_solver else 0
    grid = ns_blocks + BH * (nP + nQ)
    index = {}
    for b in range(grid):
        r = static_role(BH, nP, nQ, with_solver, b)
        assert r not in index, f"role {r} given twice"
        index[r] = b
    expect = {("key", h, u) for h in range(BH) for u in range(nP)}
    expect |= {("query", h, u) for h in range(BH) for u in range(nQ)}
    if with_solver:
        expect |= {("solver", h, 0) for h in range(BH)}
    assert set(index) == expect
    ns = nslice(D, nQ) if nQ else 0
    producers_max = max((b for r, b in index.items() if r[0] != "query"), default=-1)
    consumers_min = min((b for r, b in index.items() if r[0] == "query"), default=grid)
    for h in range(BH):
        for u in range(nQ):
            bq = index[("query", h, u)]
            producers = [("key", h, k) for k in range(nP)]
            if with_solver:
                producers.append(("solver", h, 0))
            producers += [("query", h, s) for s in range(min(ns, u))]
            for p in producers:
                bp = index[p]
                assert bp < bq, f"{('query', h, u)} waits on later {p}"
                if BH % 8 == 0:
                    assert bp % 8 == bq % 8, "producer on another XCD"
        if ns and BH % 8 == 0:
            xs = {index[("query", h, s)] % 8 for s in range(ns)}
            assert len(xs) == 1 and ns <= 32
    if BH % 8 != 0:
        assert producers_max < consumers_min
