"""Abstract machine of the per-CU queue walk: TEST INFRASTRUCTURE ONLY.

AutoMegaKernel summary, section "Methodology", layer 0: one persistent
block per multiprocessor walks its own queue in order; each task waits until
its counters reach their thresholds, runs, and adds one to each counter it
signals.  This module runs that rule on a schedule dict (the form documented
in validator.py) with no timing: in each round every queue whose head task
has all waits satisfied runs that task.  It stops when every queue is empty
(the schedule completed) or when no head can run (deadlock).

"""


def run(s, max_rounds=1_000_000):
    """Returns (completed, order): order lists task ids in execution order."""
    tasks, queues = s["tasks"], s["queues"]
    ctr = [0] * s["n_counters"]
    head = [0] * len(queues)
    order = []
    for _ in range(max_rounds):
        progressed = False
        for c, q in enumerate(queues):
            while head[c] < len(q):
                t = tasks[q[head[c]]]
                if not all(ctr[k] >= thr for k, thr in t["waits"]):
                    break
                for k in t["sigs"]:
                    ctr[k] += 1
                order.append(q[head[c]])
                head[c] += 1
                progressed = True
        if all(head[c] == len(q) for c, q in enumerate(queues)):
            return True, order
        if not progressed:
            return False, order
    return False, order


def run_epochs(s, epochs):
    """Runs the schedule `epochs` times back to back without resetting the
    counters, with thresholds epoch * P(C) + t (the monotonic-counter form
    the kernel uses across launches).  Returns True when every epoch
    completes."""
    nc = s["n_counters"]
    P = [0] * nc
    for t in s["tasks"]:
        for c in t["sigs"]:
            P[c] += 1
    ctr = [0] * nc
    for e in range(epochs):
        head = [0] * len(s["queues"])
        while True:
            progressed = False
            for c, q in enumerate(s["queues"]):
                while head[c] < len(q):
                    t = s["tasks"][q[head[c]]]
                    if not all(ctr[k] >= e * P[k] + thr for k, thr in t["waits"]):
                        break
                    for k in t["sigs"]:
                        ctr[k] += 1
                    head[c] += 1
                    progressed = True
            if all(head[c] == len(q) for c, q in enumerate(s["queues"])):
                break
            if not progressed:
                return False
    return True
