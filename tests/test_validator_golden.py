"""The safety gate on hand-enumerated schedules whose verdicts were worked
out by hand (tests/golden/validator_cases.json): both the brute-force
oracle (oracle/validator.py) and the library (amk_validate) must return the
recorded (code, task, counter, aux)."""
import json
import os

import pytest

from oracle import sim, validator
from tests.validator_common import lib_verdict

CASES = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "validator_cases.json")))["cases"]
DUMMY_MODEL = {"n_layers": 1, "hidden": 8, "n_heads": 2, "n_kv_heads": 1, "head_dim": 4, "ffn": 16,
               "vocab": 4, "max_ctx": 4, "wfmt": 0}


def as_schedule(c):
    return {"model": c.get("model", DUMMY_MODEL), "n_counters": c["n_counters"],
            "buffers": [tuple(b) for b in c["buffers"]],
            "tasks": [{"type": t["type"], "cu": t["cu"], "p": t["p"], "waits": [tuple(w) for w in t["waits"]],
                       "sigs": t["sigs"], "acc": [tuple(a) for a in t["acc"]]} for t in c["tasks"]],
            "queues": c["queues"]}


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_oracle_verdict(case):
    assert validator.validate(as_schedule(case)) == tuple(case["expect"]), case["why"]


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_library_verdict(case):
    assert lib_verdict(as_schedule(case)) == tuple(case["expect"]), case["why"]


def test_every_rule_is_exercised():
    codes = {c["expect"][0] for c in CASES}
    assert codes == set(range(8))


def test_safe_golden_schedules_complete_in_the_abstract_machine():
    for c in CASES:
        if c["expect"][0] == 0:
            ok, order = sim.run(as_schedule(c))
            assert ok and sorted(order) == list(range(len(c["tasks"]))), c["name"]


def test_deadlocking_golden_schedules_stall():
    # the two cycle cases really deadlock when run
    for name in ("wait_cycle", "queue_order_deadlock"):
        c = next(x for x in CASES if x["name"] == name)
        assert not sim.run(as_schedule(c))[0]
