"""The multi-step safety rule (amk_multistep_check), host only.

A greedy multi-step launch starts step s + 1 on a queue once that queue
finished step s and every LM-head task of step s stored its argmax partial.
So every task must happen-before some LM-head task; a task that does not
could still run while another queue's step s + 1 overwrites what it reads.
"""
import pytest

import synth
from tests.validator_common import clone, lib_model, lib_verdict, lowered

import persistent_megakernel_wg_amd as amk


def _tiny():
    return amk.ModelConfig.from_workload(synth.get("tiny"))


def _check(s):
    d = dict(s)
    d["model"] = lib_model(d["model"])
    sch = amk.Schedule.from_dict(d)
    try:
        return sch.multistep_check()
    finally:
        sch.close()


def _append(s, task, q):
    """s with `task` appended at the end of queue q (its cu set to q)."""
    s = clone(s)
    t = dict(task, cu=q)
    s["tasks"].append(t)
    s["queues"][q].append(len(s["tasks"]) - 1)
    return s


def test_lowerings_are_multistep_safe():
    for cfg in ({}, {"sync_mode": 0}, {"attn_splits": 3}, {"merge_place": 1}, {"cu_policy": 1}):
        s = lowered(_tiny(), num_cus=8, **cfg)
        assert lib_verdict(s)[0] == 0
        assert _check(s) == (amk.OK, -1), cfg
    s = lowered(amk.ModelConfig.from_workload(synth.get("1b")), num_cus=64)
    assert _check(s) == (amk.OK, -1)


def test_late_duplicate_kv_writer_passes_the_gate_but_not_multistep():
    """A copy of a last-layer QKV task at the end of a queue, after that
    queue's LM-head task: every access is ordered (the gate accepts it: it
    writes the KV row, which is state), but it happens-before no LM-head
    task, so a next step could start while it still writes q and the KV row."""
    s = lowered(_tiny(), num_cus=8)
    L = s["model"]["n_layers"]
    src = max(i for i, t in enumerate(s["tasks"]) if t["type"] == amk.TASK_QKV and t["p"][0] == L - 1)
    q = 3
    assert s["tasks"][s["queues"][q][-1]]["type"] == amk.TASK_LMHEAD
    bad = _append(s, {k: (list(v) if isinstance(v, list) else v) for k, v in s["tasks"][src].items()}, q)
    bad["tasks"][-1]["waits"] = []
    bad["tasks"][-1]["sigs"] = []
    assert lib_verdict(bad)[0] == 0
    st, task = _check(bad)
    assert st == amk.ERR_UNSUPPORTED and task == len(bad["tasks"]) - 1


def test_late_nop_output_writer_is_not_multistep_safe():
    """A NOP after an LM-head task declaring a write of that task's logits
    rows: ordered after it on the same queue, so the gate accepts it, but it
    precedes no LM-head task (and the engine refuses NOPs that declare
    accesses at all)."""
    s = lowered(_tiny(), num_cus=8)
    q = 0
    lm = s["queues"][q][-1]
    assert s["tasks"][lm]["type"] == amk.TASK_LMHEAD
    w = [a for a in s["tasks"][lm]["acc"] if a[1] == amk.ACCESS_WRITE][0]
    bad = _append(s, {"type": amk.TASK_NOP, "p": [0] * 8, "waits": [], "sigs": [], "acc": [w]}, q)
    assert lib_verdict(bad)[0] == 0
    assert _check(bad) == (amk.ERR_UNSUPPORTED, len(bad["tasks"]) - 1)


def test_schedule_without_lm_head_has_no_multistep():
    """Only LM-head tasks feed the next token; without them the check reports -2
    (here the gate already refuses: nothing writes the logits)."""
    s = lowered(_tiny(), num_cus=8)
    keep = [i for i, t in enumerate(s["tasks"]) if t["type"] != amk.TASK_LMHEAD]
    remap = {old: new for new, old in enumerate(keep)}
    t2 = clone(s)
    t2["tasks"] = [clone(s["tasks"][i]) for i in keep]
    t2["queues"] = [[remap[i] for i in q if i in remap] for q in s["queues"]]
    assert lib_verdict(t2)[0] != 0
    with pytest.raises(amk.AmkError) as e:
        _check(t2)
    assert e.value.status == amk.ERR_UNSAFE_SCHEDULE
