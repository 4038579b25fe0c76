"""amk_engine_create_noalloc through the C ABI: an engine whose device state
lives in the library's static scratch, checked against an engine from
amk_engine_create (logits bit-identical at every step, and the oracle's
parity bar) on two creations in a row, the second with a smaller model; an
engine whose state would not fit is refused before the scratch is touched.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_common import REL_L2, MAX_ABS, compare, device_cus, log

pytestmark = pytest.mark.gpu


def _engine(wl, w, noalloc):
    import persistent_megakernel_wg_amd as amk
    m = amk.ModelConfig.from_workload(wl)
    cfg = amk.default_schedule_config(m, device_cus())
    sched = amk.Schedule.build(m, cfg)
    assert sched.validate()[0] == 0
    dev_w = amk.upload_model(m, w)
    kv, logits = amk.alloc_state(m)
    return amk.Engine(sched, dev_w, kv, logits, noalloc=noalloc)


def _run_pair(wl, steps):
    """Both engines over the same teacher-forced tokens: every step's logits
    bit-identical, and the noalloc engine within the oracle parity bar."""
    import torch
    w = synth.model_weights(wl, seed=1, gains="random")
    ref = _engine(wl, w, noalloc=False)
    eng = _engine(wl, w, noalloc=True)
    orc = oracle.Model(wl, w)
    kv_o = orc.new_kv()
    toks = synth.tokens(2, steps, wl.vocab)
    worst = 0.0
    for pos, tok in enumerate(toks):
        ref.decode_step(int(tok), pos)
        eng.decode_step(int(tok), pos)
        torch.cuda.synchronize()
        ref.check()
        eng.check()
        a = ref.logits.cpu().numpy()
        b = eng.logits.cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"{wl.name} step {pos}"
        o = orc.step(kv_o, int(tok), pos)
        rel, mab, ok = compare(b.astype(np.float64), o)
        assert rel <= REL_L2 and mab <= MAX_ABS and ok, (wl.name, pos, rel, mab)
        worst = max(worst, rel)
    orc.close()
    ref.close()
    log(f"{wl.name}: {steps} steps, noalloc == allocated bit for bit, worst relL2 vs oracle {worst:.2e}")
    return eng


def test_noalloc_matches_allocated_engine_twice():
    import persistent_megakernel_wg_amd as amk
    import torch
    big = synth.get("tiny")
    small = big.with_(name="tiny_small", n_layers=1, hidden=128, ffn=344, vocab=1024, n_heads=2,
                      n_kv_heads=1, max_ctx=32)
    first = _run_pair(big, 24)
    second = _run_pair(small, 16)
    # the second creation took the scratch over: the first engine refuses to run
    with pytest.raises(amk.AmkError) as ei:
        first.decode_step(1, 24)
    assert ei.value.status == amk.ERR_INVALID_ARG
    with pytest.raises(amk.AmkError) as ei:
        first.check()
    assert ei.value.status == amk.ERR_INVALID_ARG
    first.close()
    # tracing would allocate: refused on a noalloc engine
    with pytest.raises(amk.AmkError) as ei:
        second.set_trace(True)
    assert ei.value.status == amk.ERR_UNSUPPORTED
    # a model whose engine state exceeds the scratch is refused before
    # anything is written: the live engine keeps decoding correctly
    # (the 8192-position int4 model with 64 attention splits per kv head:
    # its engine state is about 126 MB, beyond the 96 MiB scratch)
    huge = synth.get("8b_int4")
    m = amk.ModelConfig.from_workload(huge)
    cfg = amk.default_schedule_config(m, device_cus())
    cfg.attn_splits = 64
    sched = amk.Schedule.build(m, cfg)
    dummy = [torch.zeros(256, dtype=torch.uint8, device="cuda") for _ in range(amk.packed_count(m))]
    kv = torch.zeros(256, dtype=torch.int16, device="cuda")
    logits = torch.zeros(16, dtype=torch.float32, device="cuda")
    with pytest.raises(amk.AmkError) as ei:
        amk.Engine(sched, dummy, kv, logits, noalloc=True)
    assert ei.value.status == amk.ERR_UNSUPPORTED and "bytes of device scratch" in str(ei.value)
    sched.close()
    w = synth.model_weights(small, seed=1, gains="random")
    orc = oracle.Model(small, w)
    kv_o = orc.new_kv()
    toks = synth.tokens(2, 17, small.vocab)
    for pos, tok in enumerate(toks):
        o = orc.step(kv_o, int(tok), pos)
    second.decode_step(int(toks[16]), 16)
    torch.cuda.synchronize()
    second.check()
    rel, mab, ok = compare(second.logits.cpu().numpy().astype(np.float64), o)
    assert rel <= REL_L2 and mab <= MAX_ABS and ok
    orc.close()
    second.close()
    # the largest engine state among the workloads here, the int4 model's
    # with its default 28 splits per kv head, fits: created (and destroyed)
    # without a launch
    cfg = amk.default_schedule_config(m, device_cus())
    sched = amk.Schedule.build(m, cfg)
    fits = amk.Engine(sched, dummy, kv, logits, noalloc=True)
    fits.close()
    sched.close()
    log("noalloc: takeover refused the earlier engine, oversize refused, live engine intact, "
        "the default int4 engine fits")
