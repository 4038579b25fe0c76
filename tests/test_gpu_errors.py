"""Error paths and edge positions of the engine (runs on MI355X).

Argument errors are refused on the host before any launch.  The time-out
path is forced from the host with a tiny spin budget on the kernel's own
bounded waits, so every workgroup still exits normally; the engine must then
report AMK_ERR_TIMEOUT, reset its counters and decode correctly again.
"""
import numpy as np
import pytest

import oracle
import persistent_megakernel_wg_amd as amk
import synth
from tests.gpu_common import MAX_ABS, REL_L2, compare, gpu_step, log, make_engine
from tests.validator_common import lowered

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tiny():
    wl = synth.get("tiny")
    return wl, synth.model_weights(wl, seed=1)


def expect_status(code, fn, *args):
    with pytest.raises(amk.AmkError) as e:
        fn(*args)
    assert e.value.status == code, str(e.value)


def test_decode_step_argument_errors(tiny):
    wl, w = tiny
    eng = make_engine(wl, w)
    expect_status(amk.ERR_OUT_OF_RANGE, eng.decode_step, wl.vocab, 0)
    expect_status(amk.ERR_OUT_OF_RANGE, eng.decode_step, -1, 0)
    expect_status(amk.ERR_OUT_OF_RANGE, eng.decode_step, 0, wl.max_ctx)
    expect_status(amk.ERR_INVALID_ARG, eng.decode_step, 0, 1)      # gap: nothing written yet
    gpu_step(eng, 3, 0)
    expect_status(amk.ERR_INVALID_ARG, eng.decode_step, 0, 2)      # gap after one position
    expect_status(amk.ERR_OUT_OF_RANGE, eng.set_kv_length, wl.max_ctx + 1)
    eng.close()


def test_engine_refuses_unsafe_and_foreign_schedules(tiny):
    import torch
    wl, w = tiny
    m = amk.ModelConfig.from_workload(wl)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    s = lowered(m, num_cus=cus)
    dev_w = amk.upload_model(m, w)
    kv, logits = amk.alloc_state(m)
    # a wait removed from a consumer: the gate refuses the schedule (race)
    bad = {**s, "tasks": [dict(t) for t in s["tasks"]]}
    i = next(k for k, t in enumerate(bad["tasks"]) if t["type"] == 4 and t["waits"])
    bad["tasks"][i] = {**bad["tasks"][i], "waits": []}
    bad["model"] = m
    sch = amk.Schedule.from_dict(bad)
    assert sch.validate()[0] != 0
    expect_status(amk.ERR_UNSAFE_SCHEDULE, amk.Engine, sch, dev_w, kv, logits)
    # a safe schedule whose config is not the resolved one the lowering used
    good = {**s, "model": m}
    cfg = amk.default_schedule_config(m, cus)
    cfg.pipeline_depth = 0
    good["config"] = cfg
    sch = amk.Schedule.from_dict(good)
    assert sch.validate()[0] == 0
    expect_status(amk.ERR_UNSUPPORTED, amk.Engine, sch, dev_w, kv, logits)


@pytest.mark.parametrize("sync_mode", [0, 1])
def test_timeout_is_reported_and_the_engine_recovers(tiny, sync_mode):
    """Both wait protocols (counters, tagged words) give up at the spin
    budget, report it, and decode correctly afterwards."""
    wl, w = tiny
    toks = synth.tokens(2, 12, wl.vocab)
    eng = make_engine(wl, w, {"sync_mode": sync_mode})
    orc = oracle.Model(wl, w)
    kv_o = orc.new_kv()
    for p in range(8):
        gpu_step(eng, int(toks[p]), p)
        orc.step(kv_o, int(toks[p]), p)
    log("forcing a time-out with a 1 us spin budget")
    eng.set_spin_budget(1)
    eng.decode_step(int(toks[8]), 8)
    import torch
    torch.cuda.synchronize()
    expect_status(amk.ERR_TIMEOUT, eng.check)
    eng.check()  # the error was consumed and the counters restarted
    eng.set_spin_budget(2_000_000)
    for p in range(8, 12):  # position 8 again (rewind onto the aborted row), then onwards
        g = gpu_step(eng, int(toks[p]), p)
        o = orc.step(kv_o, int(toks[p]), p)
        rel, mab, same = compare(g, o)
        assert rel <= 1e-2 and mab <= 2e-2 and same, (p, rel, mab)
    eng.close()


def test_last_position_and_rewind(tiny):
    """Decode up to the last cache position, then rewind to an earlier one and
    decode a different continuation: both match the oracle."""
    wl, w = tiny
    n = wl.max_ctx
    toks = synth.tokens(4, n, wl.vocab)
    alt = synth.tokens(5, 6, wl.vocab)
    eng = make_engine(wl, w)
    orc = oracle.Model(wl, w)
    kv_o = orc.new_kv()
    worst = 0.0
    for p in range(n):
        g = gpu_step(eng, int(toks[p]), p)
        o = orc.step(kv_o, int(toks[p]), p)
        rel, mab, same = compare(g, o)
        worst = max(worst, rel)
        assert rel <= 1e-2 and mab <= 2e-2 and same, (p, rel)
    log(f"tiny to pos {n - 1}: worst relL2 {worst:.2e}")
    r = 20
    kv_o[:, :, :, r:, :] = 0
    for i, tok in enumerate(alt):
        g = gpu_step(eng, int(tok), r + i)
        o = orc.step(kv_o, int(tok), r + i)
        rel, mab, same = compare(g, o)
        assert rel <= 1e-2 and mab <= 2e-2 and same, (r + i, rel)
    eng.close()


def test_engine_refuses_unexecutable_nops_and_unsafe_multistep(tiny):
    """A schedule that passes the gate but fails amk_multistep_check (a late
    copy of a last-layer QKV task after an LM-head task) decodes single steps
    correctly and refuses amk_decode_steps before launching; a NOP task that
    declares an access (which the kernel would never make) is refused at
    engine creation."""
    import torch

    from tests.test_multistep_check import _append
    wl, w = tiny
    m = amk.ModelConfig.from_workload(wl)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    s = lowered(m, num_cus=cus)
    L = wl.n_layers
    src = max(i for i, t in enumerate(s["tasks"]) if t["type"] == amk.TASK_QKV and t["p"][0] == L - 1)
    q = next(c for c, qq in enumerate(s["queues"]) if qq and s["tasks"][qq[-1]]["type"] == amk.TASK_LMHEAD)
    late = _append(s, {k: (list(v) if isinstance(v, list) else v) for k, v in s["tasks"][src].items()}, q)
    late["tasks"][-1]["waits"], late["tasks"][-1]["sigs"] = [], []
    late["model"] = m
    late["config"] = amk.default_schedule_config(m, cus)
    sch = amk.Schedule.from_dict(late)
    assert sch.validate()[0] == 0
    assert sch.multistep_check()[0] == amk.ERR_UNSUPPORTED
    dev_w = amk.upload_model(m, w)
    kv, logits = amk.alloc_state(m)
    eng = amk.Engine(sch, dev_w, kv, logits)
    toks = synth.tokens(2, 4, wl.vocab)
    orc = oracle.Model(wl, w)
    kv_o = orc.new_kv()
    for p, tok in enumerate(toks):
        rel, mab, ok = compare(gpu_step(eng, int(tok), p), orc.step(kv_o, int(tok), p))
        assert rel <= 1e-2 and mab <= 2e-2 and ok
    out = torch.zeros(4, dtype=torch.int32, device="cuda")
    expect_status(amk.ERR_UNSUPPORTED, eng.decode_steps, int(toks[-1]), len(toks), 2, out)
    eng.close()
    sch.close()
    # a NOP declaring a logits write after an LM-head task: the gate accepts
    # it, the engine does not
    lm = s["queues"][q][-1]
    wacc = [a for a in s["tasks"][lm]["acc"] if a[1] == amk.ACCESS_WRITE][0]
    nop = _append(s, {"type": amk.TASK_NOP, "p": [0] * 8, "waits": [], "sigs": [], "acc": [wacc]}, q)
    nop["model"] = m
    nop["config"] = amk.default_schedule_config(m, cus)
    sch = amk.Schedule.from_dict(nop)
    assert sch.validate()[0] == 0
    expect_status(amk.ERR_UNSUPPORTED, amk.Engine, sch, dev_w, kv, logits)
    sch.close()
    orc.close()
    log("engine: late QKV copy decodes single steps, refuses multi-step; NOP with accesses refused")


def test_empty_launch_changes_nothing():
    """amk_engine_launch_empty runs the decode kernel with every queue empty:
    the logits of the previous step stay bit-identical, and the next steps
    still match the oracle (no position, counter or tag moved)."""
    import torch
    wl = synth.get("tiny")
    w = synth.model_weights(wl, seed=1, gains="random")
    toks = synth.tokens(2, 12, wl.vocab)
    eng = make_engine(wl, w)
    orc = oracle.Model(wl, w)
    kv_o = orc.new_kv()
    for pos in range(6):
        g = gpu_step(eng, int(toks[pos]), pos)
        orc.step(kv_o, int(toks[pos]), pos)
    before = eng.logits.clone()
    for _ in range(3):
        eng.launch_empty()
    torch.cuda.synchronize()
    eng.check()
    assert torch.equal(before, eng.logits)
    for pos in range(6, 12):
        g = gpu_step(eng, int(toks[pos]), pos)
        o = orc.step(kv_o, int(toks[pos]), pos)
        rel, mab, ok = compare(g, o)
        assert rel <= REL_L2 and mab <= MAX_ABS and ok, (pos, rel, mab)
    orc.close()
    eng.close()


def test_last_position_and_rewind_long_splits():
    """The position-major attention layout at the cache's end: a two-layer
    decoder with a 300-position cache and 2 splits per kv head decodes up to
    position 299 (splits of 150 positions, the last block of each ragged),
    then rewinds to position 262 and decodes a different continuation; every
    step from position 255 on matches the oracle."""
    wl = synth.get("tiny").with_(name="tiny_end_long", max_ctx=300, prompt_len=256, decode_steps=44)
    w = synth.model_weights(wl, seed=1, gains="random")
    n = wl.max_ctx
    toks = synth.tokens(4, n, wl.vocab)
    alt = synth.tokens(5, 8, wl.vocab)
    eng = make_engine(wl, w, {"attn_splits": 2})
    orc = oracle.Model(wl, w)
    kv_o = orc.new_kv()
    worst = 0.0
    for p in range(n):
        g = gpu_step(eng, int(toks[p]), p)
        o = orc.step(kv_o, int(toks[p]), p)
        if p >= 255:
            rel, mab, same = compare(g, o)
            worst = max(worst, rel)
            assert rel <= REL_L2 and mab <= MAX_ABS and same, (p, rel, mab)
    r = 262
    kv_o[:, :, :, r:, :] = 0
    for i, tok in enumerate(alt):
        g = gpu_step(eng, int(tok), r + i)
        o = orc.step(kv_o, int(tok), r + i)
        rel, mab, same = compare(g, o)
        worst = max(worst, rel)
        assert rel <= REL_L2 and mab <= MAX_ABS and same, (r + i, rel, mab)
    log(f"tiny, 300-position cache, 2 splits: to pos {n - 1} and rewound to {r}: worst relL2 {worst:.2e}")
    orc.close()
    eng.close()
