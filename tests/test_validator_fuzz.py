"""Seeded mutation fuzz of the safety gate: the library's amk_validate and the
brute-force oracle (oracle/validator.py) must return bit-identical
(code, task, counter, aux) on thousands of mutated schedules.

Bases: the library's own lowerings of small decoders (several CU counts,
split counts, CU policies, all three weight formats) and random schedules of
untyped tasks.  Mutation classes, with the rule each is built to trip:
cycle injected (V3), queue order reversed against a wait (V4), threshold set
to 0 or P+1 (V2), full join lowered on a counter whose writes are read (V5),
wait removed (V6 unless another path orders the pair), queue entry / counter
/ byte range out of bounds, task listed twice, bad type (V1), output writer
emptied (V7), and safe edits (threshold raised to full, duplicated wait).
Every schedule the gate accepts must also run to completion in the abstract
machine (oracle/sim.py), for one launch and for three launches on
monotonic counters."""
import random

import pytest

import persistent_megakernel_wg_amd as amk
import synth
from oracle import sim, validator
from tests.validator_common import clone, lib_verdict, lowered

N_LOWERED = 3700   # mutated lowerings
N_RANDOM = 3700    # random untyped schedules (base and mutated)


def small_models():
    tiny = amk.ModelConfig.from_workload(synth.get("tiny"))
    out = [tiny]
    for wfmt in (1, 2):  # int8, int4: meta byte ranges in the accesses
        m = amk.ModelConfig.from_workload(synth.get("tiny"))
        m.ffn, m.vocab, m.wfmt = 512, 512, wfmt
        out.append(m)
    return out


def bases():
    out = []
    for m in small_models():
        for ncu in (1, 2, 3, 5, 8):
            for splits in (1, 2, 3):
                for pol in (0, 1):
                    if m.wfmt != 0 and (splits == 3 or pol == 1):
                        continue
                    out.append(lowered(m, num_cus=ncu, attn_splits=splits, cu_policy=pol))
    return out


def producers(s):
    P = {}
    for i, t in enumerate(s["tasks"]):
        for c in t["sigs"]:
            P.setdefault(c, []).append(i)
    return P


def mutate(s, rng):
    """One mutation; returns (schedule, class name, expected code or None)."""
    s = clone(s)
    tasks, nt = s["tasks"], len(s["tasks"])
    P = producers(s)
    waiting = [(i, k) for i, t in enumerate(tasks) for k in range(len(t["waits"]))]
    kind = rng.choice(["cycle", "queue_swap", "thr_zero", "thr_over", "thr_lower", "drop_wait",
                       "queue_oob", "ctr_oob", "range_oob", "dup_task", "bad_type", "drop_output",
                       "raise_thr", "dup_wait", "double"])
    if kind == "double":
        s, _, _ = mutate(s, rng)
        s, k2, _ = mutate(s, rng)
        return s, "double+" + k2, None
    if kind in ("cycle", "thr_zero", "thr_over", "thr_lower", "drop_wait", "dup_wait", "raise_thr") and not waiting:
        kind = "queue_oob"
    if kind == "cycle":
        w, k = rng.choice(waiting)
        c = tasks[w]["waits"][k][0]
        p = rng.choice(P[c])
        nc = s["n_counters"]
        s["n_counters"] = nc + 1
        tasks[w]["sigs"].append(nc)
        tasks[p]["waits"].append((nc, 1))
        return s, kind, validator.CYCLE
    if kind == "thr_zero":
        w, k = rng.choice(waiting)
        tasks[w]["waits"][k] = (tasks[w]["waits"][k][0], 0)
        return s, kind, validator.THRESHOLD
    if kind == "thr_over":
        w, k = rng.choice(waiting)
        c = tasks[w]["waits"][k][0]
        tasks[w]["waits"][k] = (c, len(P[c]) + 1)
        return s, kind, validator.THRESHOLD
    if kind == "thr_lower":
        cand = [(i, k) for i, k in waiting if tasks[i]["waits"][k][1] >= 2]
        if cand:
            w, k = rng.choice(cand)
            c, t = tasks[w]["waits"][k]
            tasks[w]["waits"][k] = (c, rng.randint(1, t - 1))
        return s, kind, None
    if kind == "drop_wait":
        w, k = rng.choice(waiting)
        del tasks[w]["waits"][k]
        return s, kind, None
    if kind == "dup_wait":
        w, k = rng.choice(waiting)
        tasks[w]["waits"].append(tasks[w]["waits"][k])
        return s, kind, None
    if kind == "raise_thr":
        w, k = rng.choice(waiting)
        c = tasks[w]["waits"][k][0]
        tasks[w]["waits"][k] = (c, len(P[c]))
        return s, kind, None
    if kind == "queue_swap":
        qs = [q for q in s["queues"] if len(q) >= 2]
        if qs:
            q = rng.choice(qs)
            i = rng.randrange(len(q) - 1)
            q[i], q[i + 1] = q[i + 1], q[i]
        return s, kind, None
    if kind == "queue_oob":
        c = rng.randrange(len(s["queues"]))
        s["queues"][c].insert(rng.randint(0, len(s["queues"][c])), nt + rng.randint(0, 3))
        return s, kind, None
    if kind == "ctr_oob":
        i = rng.randrange(nt)
        if rng.random() < 0.5:
            tasks[i]["sigs"].append(s["n_counters"] + rng.randint(0, 2))
        else:
            tasks[i]["waits"].append((s["n_counters"] + rng.randint(0, 2), 1))
        return s, kind, validator.REF
    if kind == "range_oob":
        i = rng.randrange(nt)
        if tasks[i]["acc"]:
            k = rng.randrange(len(tasks[i]["acc"]))
            b, m, lo, hi = tasks[i]["acc"][k]
            size = s["buffers"][b][0]
            tasks[i]["acc"][k] = rng.choice([(b, m, lo, size + 4), (b, m, hi, hi), (b, m, -4, hi),
                                             (len(s["buffers"]), m, lo, hi), (b, 3, lo, hi)])
            return s, kind, validator.REF
        return s, kind, None
    if kind == "dup_task":
        i = rng.randrange(nt)
        c = rng.randrange(len(s["queues"]))
        s["queues"][c].append(i)
        return s, kind, validator.REF
    if kind == "bad_type":
        i = rng.randrange(nt)
        tasks[i]["type"] = rng.choice([8, 11, -1])
        return s, kind, validator.REF
    if kind == "drop_output":
        writers = [i for i, t in enumerate(tasks)
                   if any(a[1] == validator.WRITE and s["buffers"][a[0]][1] == validator.BUF_OUTPUT for a in t["acc"])]
        if writers:
            i = rng.choice(writers)
            tasks[i]["type"] = validator.NOP
            tasks[i]["acc"] = [a for a in tasks[i]["acc"] if a[1] == validator.READ]
        return s, kind, None
    raise AssertionError(kind)


def random_schedule(rng):
    """Random untyped schedule: tasks in index order form a DAG of full or
    partial joins, queues keep index order, accesses are random 8-byte-aligned
    ranges of five buffers (output, two scratch, state, history)."""
    nt = rng.randint(2, 18)
    ncu = rng.randint(1, 4)
    bufs = [(64, validator.BUF_OUTPUT), (64, validator.BUF_SCRATCH), (48, validator.BUF_SCRATCH),
            (32, validator.BUF_STATE), (32, validator.BUF_HISTORY)]
    tasks = []
    nc = 0
    sig_of = {}
    for i in range(nt):
        t = {"type": 0, "cu": rng.randrange(ncu), "p": [], "waits": [], "sigs": [], "acc": []}
        if i and rng.random() < 0.7:
            for j in rng.sample(range(i), min(i, rng.randint(1, 2))):
                if j not in sig_of:
                    sig_of[j] = nc
                    nc += 1
                    tasks[j]["sigs"].append(sig_of[j])
        for _ in range(rng.randint(0, 3)):
            b = rng.randrange(len(bufs))
            lo = 8 * rng.randrange(bufs[b][0] // 8)
            hi = lo + 8 * rng.randint(1, (bufs[b][0] - lo) // 8)
            t["acc"].append((b, rng.choice([1, 2]) if bufs[b][1] != validator.BUF_HISTORY else 1, lo, hi))
        tasks.append(t)
    # counters shared by several producers sometimes
    for i, t in enumerate(tasks):
        if t["sigs"] and rng.random() < 0.2 and i + 1 < nt:
            tasks[rng.randrange(i + 1, nt)]["sigs"].append(t["sigs"][0])
    Pn = [0] * nc
    for t in tasks:
        for c in t["sigs"]:
            Pn[c] += 1
    for i, t in enumerate(tasks):
        for j in range(i):
            if j in sig_of and rng.random() < 0.3:
                c = sig_of[j]
                t["waits"].append((c, Pn[c] if rng.random() < 0.85 else rng.randint(1, Pn[c])))
    queues = [[i for i in range(nt) if tasks[i]["cu"] == c] for c in range(ncu)]
    # usually make the output whole
    if rng.random() < 0.7:
        tasks[-1]["acc"].append((0, 2, 0, 64))
    return {"model": {"n_layers": 1, "hidden": 8, "n_heads": 2, "n_kv_heads": 1, "head_dim": 4,
                      "ffn": 16, "vocab": 4, "max_ctx": 4, "wfmt": 0},
            "n_counters": nc, "buffers": bufs, "tasks": tasks, "queues": queues}


def check_pair(s, expect=None, label=""):
    ov = validator.validate(s)
    lv = lib_verdict(s)
    assert lv == ov, (label, lv, ov)
    if expect is not None:
        assert ov[0] == expect, (label, ov)
    if ov[0] == validator.OK:
        ok, order = sim.run(s)
        assert ok and sorted(order) == list(range(len(s["tasks"]))), label
        assert sim.run_epochs(s, 3), label
    return ov[0]


@pytest.fixture(scope="module")
def base_schedules():
    return bases()


def test_lowerings_are_accepted(base_schedules):
    assert len(base_schedules) >= 40
    for s in base_schedules:
        assert check_pair(s, validator.OK) == validator.OK


def test_mutated_lowerings_agree(base_schedules):
    rng = random.Random(20261202)
    codes = {}
    for n in range(N_LOWERED):
        s, kind, expect = mutate(base_schedules[n % len(base_schedules)], rng)
        c = check_pair(s, expect, f"{n}:{kind}")
        codes[c] = codes.get(c, 0) + 1
    # every rule fires on mutated real schedules
    for code in range(8):
        assert codes.get(code, 0) > 0, codes


def test_random_schedules_agree():
    rng = random.Random(7160)
    codes = {}
    for n in range(N_RANDOM):
        s = random_schedule(rng)
        if n % 2:
            s, _, _ = mutate(s, rng)
        c = check_pair(s, None, f"random {n}")
        codes[c] = codes.get(c, 0) + 1
    for code in range(8):
        assert codes.get(code, 0) > 0, codes


def test_fuzz_volume():
    assert N_LOWERED + N_RANDOM >= 7160
