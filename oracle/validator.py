"""Brute-force reference of the schedule safety gate: TEST INFRASTRUCTURE ONLY.

AutoMegaKernel summary, section "Methodology", the safety gate: before a
launch, static checks on the schedule graph certify deadlock freedom
(acyclic producer/consumer graph, wait thresholds between 1 and the number
of producers, valid per-multiprocessor queue orders), race freedom
(multi-producer counters fully joined before a consumer reads what they
guard, ordered memory accesses) and correctness (every output reachable,
every reference valid).  The pages name the checks but do not define them;
this module writes out the reading used here as plainly as possible, with
no graph algorithms beyond depth-first reachability:

  V1 REF          every queue entry names a task; each task sits in exactly
                  one queue, the queue of its cu; counters, buffers, access
                  modes and byte ranges are in range; a typed task declares
                  exactly (as a multiset) the accesses its type and params
                  imply (the table in include/amk.h, restated in `derive`).
  V2 THRESHOLD    each wait (C, t) has 1 <= t <= P(C), P(C) = number of
                  signal entries naming C.
  V3 CYCLE        no task reaches itself through producer -> waiter edges.
  V4 QUEUE_ORDER  no task reaches itself through producer -> waiter edges
                  plus queue-order edges.
  V5 UNDER_JOINED a wait (C, t < P(C)) by a task that reads bytes some
                  producer of C writes.
  V6 RACE         two distinct tasks with overlapping accesses, one of them
                  a write, neither reaching the other through queue edges
                  and full-join edges (producer -> waiter of (C, P(C))).
  V7 OUTPUT       each OUTPUT buffer is fully written (else the buffer is
                  named), there is at least one OUTPUT buffer, and every task
                  is live: it writes an OUTPUT or STATE buffer, or writes
                  bytes that a live task reads after it in happens-before.

The first failing rule is reported as (code, task, counter, aux):
  V1: (1, -1, -1, cu) for a bad queue entry (first cu, in order), else
      (1, smallest bad task, -1, -1);
  V2: (2, task, counter, index of the wait) for the first task, first wait;
  V3 / V4: (code, smallest task on a cycle, -1, -1);
  V5: (5, smallest waiting task, counter of its first under-joined wait in
      declared order, smallest conflicting producer);
  V6: (6, a, -1, b) for the lexicographically smallest racing pair a < b;
  V7: (7, -1, -1, buffer) for an output buffer not fully written,
      (7, -1, -1, -1) when there is none, (7, smallest dead task, -1, -1).

Schedules are plain dicts: {"model": {...}, "n_counters": int,
"buffers": [(size, kind)], "tasks": [{"type", "cu", "p", "waits": [(c, t)],
"sigs": [c], "acc": [(buf, mode, begin, end)]}], "queues": [[task ids]]}.
"""

OK, REF, THRESHOLD, CYCLE, QUEUE_ORDER, UNDER_JOINED, RACE, OUTPUT = range(8)
NOP, QKV, ATTN, MERGE, OPROJ, GATEUP, DOWN, LMHEAD = range(8)
N_TYPES = 8
READ, WRITE = 1, 2
BUF_WEIGHT, BUF_SCRATCH, BUF_OUTPUT, BUF_STATE, BUF_HISTORY = range(5)

# buffer ids of a lowered schedule (include/amk.h)
EMBED, FINAL_NORM, LM, KV_HIST, KV_CUR, LOGITS, X, Q, PART, O, A = range(11)
LAYER0 = 11
ATTN_NORM, W_QKV, W_O, MLP_NORM, W_GATEUP, W_DOWN = range(6)
WFMT_BF16, WFMT_INT8, WFMT_INT4 = 0, 1, 2


def layer_buffer(l, k):
    return LAYER0 + 6 * l + k


def row_bytes(fmt, cols):
    """(data bytes, meta bytes) per row of a packed tensor."""
    if fmt == WFMT_BF16:
        return 2 * cols, 0
    if fmt == WFMT_INT8:
        return cols, 4                    # one fp32 scale per row
    return cols // 2, (cols // 128) * 4   # two nibbles per byte; fp16 scale + zero per 128


def packed_shape(m, k):
    """(format, rows, cols) of packed tensor k."""
    H, F, hd = m["hidden"], m["ffn"], m["head_dim"]
    qd, kvd = m["n_heads"] * hd, m["n_kv_heads"] * hd
    if k == 0:
        return WFMT_BF16, m["vocab"], H
    if k == 1:
        return WFMT_BF16, 1, H
    if k == 2:
        return m["wfmt"], m["vocab"], H
    sub = (k - 3) % 6
    return {ATTN_NORM: (WFMT_BF16, 1, H), MLP_NORM: (WFMT_BF16, 1, H),
            W_QKV: (m["wfmt"], qd + 2 * kvd, H), W_O: (m["wfmt"], H, qd),
            W_GATEUP: (m["wfmt"], 2 * F, H), W_DOWN: (m["wfmt"], H, F)}[sub]


def derive(m, t):
    """Accesses a typed task performs, or None when its params are invalid."""
    L, H, F, hd = m["n_layers"], m["hidden"], m["ffn"], m["head_dim"]
    nq, nkv, mc, V = m["n_heads"], m["n_kv_heads"], m["max_ctx"], m["vocab"]
    half, grp = hd // 2, nq // nkv
    p = list(t["p"]) + [0] * 8
    out = []

    def rows(buf, k, a, b):
        fmt, nrows, cols = packed_shape(m, k)
        rb, mb = row_bytes(fmt, cols)
        out.append((buf, READ, a * rb, b * rb))
        if mb:
            out.append((buf, READ, nrows * rb + a * mb, nrows * rb + b * mb))

    def x_in(l, r0, r1):
        if l == 0:
            out.append((EMBED, READ, 0, V * H * 2))
        else:
            base = ((l - 1) * 2 + 1) * H
            out.append((X, READ, (base + r0) * 4, (base + r1) * 4))

    ty = t["type"]
    if ty == QKV:
        l, u0, u1 = p[0], p[1], p[2]
        if not (0 <= l < L and 0 <= u0 < u1 <= (nq + 2 * nkv) * half):
            return None
        x_in(l, 0, H)
        out.append((layer_buffer(l, ATTN_NORM), READ, 0, H * 2))
        rows(layer_buffer(l, W_QKV), 3 + 6 * l + W_QKV, 2 * u0, 2 * u1)
        for hs in range(u0 // half, (u1 - 1) // half + 1):
            i0, i1 = max(u0, hs * half) - hs * half, min(u1, (hs + 1) * half) - hs * half
            if hs < nq:
                base, buf, el = (l * nq + hs) * hd, Q, 4
            else:
                kv = 0 if hs < nq + nkv else 1
                g = hs - nq - kv * nkv
                base, buf, el = ((l * 2 + kv) * nkv + g) * hd, KV_CUR, 2
            out.append((buf, WRITE, (base + i0) * el, (base + i1) * el))
            out.append((buf, WRITE, (base + half + i0) * el, (base + half + i1) * el))
    elif ty == ATTN:
        l, g, s, S = p[0], p[1], p[2], p[3]
        if not (0 <= l < L and 0 <= g < nkv and S >= 1 and 0 <= s < S):
            return None
        out.append((Q, READ, (l * nq + g * grp) * hd * 4, (l * nq + (g + 1) * grp) * hd * 4))
        for kv in (0, 1):
            slot = (l * 2 + kv) * nkv + g
            out.append((KV_HIST, READ, slot * mc * hd * 2, (slot + 1) * mc * hd * 2))
            out.append((KV_CUR, READ, slot * hd * 2, (slot + 1) * hd * 2))
        for h in range(g * grp, (g + 1) * grp):
            b = ((l * nq + h) * S + s) * (hd + 2) * 4
            out.append((PART, WRITE, b, b + (hd + 2) * 4))
    elif ty == MERGE:
        l, h, S = p[0], p[1], p[2]
        if not (0 <= l < L and 0 <= h < nq and S >= 1):
            return None
        out.append((PART, READ, (l * nq + h) * S * (hd + 2) * 4, (l * nq + h + 1) * S * (hd + 2) * 4))
        out.append((O, WRITE, (l * nq + h) * hd * 4, (l * nq + h + 1) * hd * 4))
    elif ty == OPROJ:
        l, r0, r1 = p[0], p[1], p[2]
        if not (0 <= l < L and 0 <= r0 < r1 <= H):
            return None
        out.append((O, READ, l * nq * hd * 4, (l + 1) * nq * hd * 4))
        x_in(l, r0, r1)
        rows(layer_buffer(l, W_O), 3 + 6 * l + W_O, r0, r1)
        out.append((X, WRITE, (l * 2 * H + r0) * 4, (l * 2 * H + r1) * 4))
    elif ty == GATEUP:
        l, j0, j1 = p[0], p[1], p[2]
        if not (0 <= l < L and 0 <= j0 < j1 <= F):
            return None
        out.append((X, READ, l * 2 * H * 4, (l * 2 + 1) * H * 4))
        out.append((layer_buffer(l, MLP_NORM), READ, 0, H * 2))
        rows(layer_buffer(l, W_GATEUP), 3 + 6 * l + W_GATEUP, 2 * j0, 2 * j1)
        out.append((A, WRITE, (l * F + j0) * 4, (l * F + j1) * 4))
    elif ty == DOWN:
        l, r0, r1 = p[0], p[1], p[2]
        if not (0 <= l < L and 0 <= r0 < r1 <= H):
            return None
        out.append((A, READ, l * F * 4, (l + 1) * F * 4))
        out.append((X, READ, (l * 2 * H + r0) * 4, (l * 2 * H + r1) * 4))
        rows(layer_buffer(l, W_DOWN), 3 + 6 * l + W_DOWN, r0, r1)
        out.append((X, WRITE, ((l * 2 + 1) * H + r0) * 4, ((l * 2 + 1) * H + r1) * 4))
    elif ty == LMHEAD:
        r0, r1 = p[0], p[1]
        if not (0 <= r0 < r1 <= V):
            return None
        out.append((X, READ, ((L - 1) * 2 + 1) * H * 4, ((L - 1) * 2 + 2) * H * 4))
        out.append((FINAL_NORM, READ, 0, H * 2))
        rows(LM, 2, r0, r1)
        out.append((LOGITS, WRITE, r0 * 4, r1 * 4))
    else:
        return None
    return out


def overlap(x, y):
    return x[0] == y[0] and x[2] < y[3] and y[2] < x[3]


def reaches(succ, a, b):
    """Is there a non-empty path a -> ... -> b?"""
    seen, stack = set(), list(succ[a])
    while stack:
        v = stack.pop()
        if v == b:
            return True
        if v not in seen:
            seen.add(v)
            stack.extend(succ[v])
    return False


def reach_sets(succ, n):
    """All nodes reachable from each node (non-empty paths), as Python sets."""
    out = []
    for a in range(n):
        seen, stack = set(), list(succ[a])
        while stack:
            v = stack.pop()
            if v not in seen:
                seen.add(v)
                stack.extend(succ[v])
        out.append(seen)
    return out


def validate(s):
    tasks, queues, nc, bufs = s["tasks"], s["queues"], s["n_counters"], s["buffers"]
    nt, ncu, nb = len(tasks), len(queues), len(bufs)

    # V1 REF
    places = [[] for _ in range(nt)]
    for c, q in enumerate(queues):
        for pos, t in enumerate(q):
            if not 0 <= t < nt:
                return (REF, -1, -1, c)
            places[t].append(c)
    for i, t in enumerate(tasks):
        ok = 0 <= t["cu"] < ncu and 0 <= t["type"] < N_TYPES and places[i] == [t["cu"]]
        ok = ok and all(0 <= c < nc for c, _ in t["waits"]) and all(0 <= c < nc for c in t["sigs"])
        for (b, mode, lo, hi) in t["acc"]:
            ok = ok and 0 <= b < nb and mode in (READ, WRITE) and 0 <= lo < hi and hi <= bufs[b][0]
        if ok and t["type"] != NOP:
            d = derive(s["model"], t)
            ok = d is not None and sorted(d) == sorted(tuple(a) for a in t["acc"])
        if not ok:
            return (REF, i, -1, -1)

    # V2 THRESHOLD
    P = [0] * nc
    producers = [[] for _ in range(nc)]
    for i, t in enumerate(tasks):
        for c in t["sigs"]:
            P[c] += 1
            producers[c].append(i)
    for i, t in enumerate(tasks):
        for k, (c, thr) in enumerate(t["waits"]):
            if not 1 <= thr <= P[c]:
                return (THRESHOLD, i, c, k)

    # V3 CYCLE / V4 QUEUE_ORDER
    wait_succ = [set() for _ in range(nt)]
    for w, t in enumerate(tasks):
        for c, _ in t["waits"]:
            for p in producers[c]:
                wait_succ[p].add(w)
    for i in range(nt):
        if reaches(wait_succ, i, i):
            return (CYCLE, i, -1, -1)
    qsucc = [set(x) for x in wait_succ]
    for q in queues:
        for a, b in zip(q, q[1:]):
            qsucc[a].add(b)
    for i in range(nt):
        if reaches(qsucc, i, i):
            return (QUEUE_ORDER, i, -1, -1)

    # V5 UNDER_JOINED
    for w, t in enumerate(tasks):
        reads = [a for a in t["acc"] if a[1] == READ]
        for c, thr in t["waits"]:
            if thr >= P[c]:
                continue
            for p in sorted(set(producers[c])):
                writes = [a for a in tasks[p]["acc"] if a[1] == WRITE]
                if any(overlap(r, x) for r in reads for x in writes):
                    return (UNDER_JOINED, w, c, p)

    # happens-before: queue edges and full-join edges
    hb_succ = [set() for _ in range(nt)]
    for q in queues:
        for a, b in zip(q, q[1:]):
            hb_succ[a].add(b)
    for w, t in enumerate(tasks):
        for c, thr in t["waits"]:
            if thr == P[c]:
                for p in producers[c]:
                    hb_succ[p].add(w)
    hb = reach_sets(hb_succ, nt)

    # V6 RACE: conflicting task pairs, found per buffer
    per_buf = [[] for _ in range(nb)]
    for i, t in enumerate(tasks):
        for a in t["acc"]:
            per_buf[a[0]].append((i, tuple(a)))
    conflicts = set()
    flow = set()  # (writer, reader) with writer before reader
    for lst in per_buf:
        for x in range(len(lst)):
            for y in range(x + 1, len(lst)):
                (i, a), (j, b) = lst[x], lst[y]
                if i == j or not overlap(a, b) or (a[1] != WRITE and b[1] != WRITE):
                    continue
                if j not in hb[i] and i not in hb[j]:
                    conflicts.add((min(i, j), max(i, j)))
                if a[1] == WRITE and b[1] == READ and j in hb[i]:
                    flow.add((i, j))
                if b[1] == WRITE and a[1] == READ and i in hb[j]:
                    flow.add((j, i))
    if conflicts:
        a, b = min(conflicts)
        return (RACE, a, -1, b)

    # V7 OUTPUT
    outputs = [b for b in range(nb) if bufs[b][1] == BUF_OUTPUT]
    for b in outputs:
        covered = 0
        for lo, hi in sorted((a[2], a[3]) for _, a in per_buf[b] if a[1] == WRITE):
            if lo > covered:
                break
            covered = max(covered, hi)
        if covered < bufs[b][0]:
            return (OUTPUT, -1, -1, b)
    if not outputs:
        return (OUTPUT, -1, -1, -1)
    live = set(i for i, t in enumerate(tasks)
               if any(a[1] == WRITE and bufs[a[0]][1] in (BUF_OUTPUT, BUF_STATE) for a in t["acc"]))
    changed = True
    while changed:
        changed = False
        for (w, r) in flow:
            if r in live and w not in live:
                live.add(w)
                changed = True
    for i in range(nt):
        if i not in live:
            return (OUTPUT, i, -1, -1)
    return (OK, -1, -1, -1)
