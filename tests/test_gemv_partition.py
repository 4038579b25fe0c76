"""Work split of the streaming GEMV over the 8 waves of a workgroup.

While 8 whole units remain, wave w owns unit w of each round.  The R last
units (R = nunits % 8) are cut into p = min(8 // R, J) slab ranges of
ceil(J / p) slabs each, and wave w < R*p takes piece w % p of tail unit
w // p.  Each wave writes one partial per segment (a round unit or its tail
piece), and the finalize pass adds, per unit, the partials of the waves that
covered it.  This re-derives the kernel's issue and consume state machines in
Python from that description and checks, for many shapes, that every
(unit, slab) step is loaded and accumulated exactly once and that the
finalize pass reads exactly the partials that were written (host-side check
of the rule the kernel implements)."""
import itertools

W = 8


def split(nunits, J):
    nr = nunits // W
    R = nunits - nr * W
    p = 0 if R == 0 else min(W // R, J)
    pl = 0 if p == 0 else -(-J // p)
    return nr, R, p, pl


def tail(w, nunits, J):
    nr, R, p, pl = split(nunits, J)
    if w < R * p:
        q, k = divmod(w, p)
        j0 = k * pl
        return nr * W + q, j0, max(0, min(J, j0 + pl) - j0)
    return 0, 0, 0


def wave_steps(w, nunits, J):
    """(unit, j) in the order wave w issues them, following the kernel."""
    nr = split(nunits, J)[0]
    tu, tj, tl = tail(w, nunits, J)
    nA = nr * J
    n = nA + tl
    iu, ij = (w, 0) if nA else (tu, tj)
    out = []
    for ik in range(1, n + 1):
        out.append((iu, ij))
        ij += 1
        if ij == J:
            ij, iu = 0, iu + W
        if ik == nA:
            iu, ij = tu, tj
    return out


def flushes(w, nunits, J, DS):
    """Units wave w writes a partial for, each with the steps it summed."""
    nr = split(nunits, J)[0]
    tu, tj, tl = tail(w, nunits, J)
    nA = nr * J
    n = nA + tl
    steps = wave_steps(w, nunits, J)
    out = {}
    if n == 0:
        return out
    ck, cu, cj = 0, *((w, 0) if nA else (tu, tj))
    acc = []
    for _ in range(-(-n // DS) * DS):
        if ck < n:
            assert steps[ck] == (cu, cj)
            acc.append((cu, cj))
        ck += 1
        cj += 1
        unit_end = cj == J
        if ck <= n and (unit_end or ck == n):
            assert cu not in out
            out[cu] = acc
            acc = []
        if unit_end:
            cj, cu = 0, cu + W
        if ck == nA:
            cu, cj = tu, tj
    return out


def row_waves(u, nunits, J):
    nr, R, p, pl = split(nunits, J)
    if u < nr * W:
        return {u % W}
    q = u - nr * W
    return {q * p + k for k in range(p) if k * pl < J}


def test_every_step_once():
    for nunits, J, DS in itertools.product([1, 2, 3, 5, 7, 8, 9, 12, 16, 17, 56, 501], [1, 2, 3, 7, 8, 28],
                                           [2, 4, 8, 16]):
        seen = {}
        written = {}
        for w in range(W):
            for st in wave_steps(w, nunits, J):
                assert 0 <= st[0] < nunits and 0 <= st[1] < J
                assert st not in seen, (nunits, J, w, st)
                seen[st] = w
            for u, acc in flushes(w, nunits, J, DS).items():
                written[(u, w)] = acc
        assert len(seen) == nunits * J
        for u in range(nunits):
            got = []
            for w in sorted(row_waves(u, nunits, J)):
                assert (u, w) in written, (nunits, J, DS, u, w)
                got += written[(u, w)]
            assert sorted(got) == [(u, j) for j in range(J)], (nunits, J, DS, u)
        # nothing written that the finalize pass ignores
        for (u, w) in written:
            assert w in row_waves(u, nunits, J)


def test_rounds_are_adjacent_rows():
    # with whole rounds every wave streams one unit of 8 adjacent ones
    for nunits in (8, 16, 56):
        for w in range(W):
            units = sorted({u for u, _ in wave_steps(w, nunits, 4)})
            assert units == list(range(w, nunits, W))


def test_tail_balance():
    # 12 units of 8 slabs (a QKV task of the 8B shape): 4 tail units in halves
    lens = [tail(w, 12, 8)[2] for w in range(W)]
    assert lens == [4] * 8
