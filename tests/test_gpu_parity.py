"""Logits parity of the HIP decode path against the oracle (runs on MI355X).

Every test drives the C ABI through the binding (amk_build_schedule ->
amk_engine_create -> amk_decode_step) and compares the logits of each step
with the oracle on the same seeded weights and teacher-forced tokens.
"""
import numpy as np
import pytest

import synth
from tests.gpu_common import check_run, log, teacher_forced

pytestmark = pytest.mark.gpu


def test_tiny_full_protocol():
    """Tiny decoder: 16-token prompt + 32 decode steps, every step compared."""
    wl = synth.get("tiny")
    w = synth.model_weights(wl, seed=1)
    toks = synth.tokens(2, wl.prompt_len + wl.decode_steps, wl.vocab)
    log(f"tiny: {len(toks)} steps")
    res, eng, kv_o = teacher_forced(wl, w, toks)
    agree, rel, mab = check_run(res, min_argmax=1.0)
    log(f"tiny: argmax {agree:.3f} worst relL2 {rel:.2e} worst maxabs {mab:.2e}")
    # the KV cache rows written by the GPU match the oracle's within bf16 rounding
    kv_g = eng.kv_cache.cpu().numpy().view(np.uint16).reshape(kv_o.shape)
    n = len(toks)
    g = (kv_g[..., :n, :].astype(np.uint32) << 16).view(np.float32)
    o = (kv_o[..., :n, :].astype(np.uint32) << 16).view(np.float32)
    assert np.allclose(g, o, rtol=2 ** -7, atol=1e-6)


def test_1b_tied_short_and_long():
    """~1B decoder with tied embeddings (head_dim 64, 4 query heads per kv
    head): an 8-token prompt + 8 decode steps, then 3 decode steps after a
    seeded 128-row KV prefix; every step compared."""
    wl = synth.get("1b")
    w = synth.model_weights(wl, seed=1)
    toks = synth.tokens(2, 16, wl.vocab)
    res, eng, _ = teacher_forced(wl, w, toks)
    del eng
    agree, rel, mab = check_run(res, min_argmax=1.0)
    log(f"1b short: argmax {agree:.3f} worst relL2 {rel:.2e} worst maxabs {mab:.2e}")
    P = wl.prompt_len
    kvp = synth.kv_prefix(wl, P, seed=3)
    toks = synth.tokens(2, P + 3, wl.vocab)[P:]
    res, eng, _ = teacher_forced(wl, w, toks, kv_prefix=kvp, start=P)
    del eng
    _free()
    agree, rel, mab = check_run(res, min_argmax=1.0)
    log(f"1b long: argmax {agree:.3f} worst relL2 {rel:.2e} worst maxabs {mab:.2e}")


@pytest.fixture(scope="module")
def w8b():
    """Seeded bf16 weights of the 8B shape; the int8 / int4 workloads quantise
    these same tensors (both sides quantise with their own code)."""
    wl = synth.get("8b")
    log("generating 8b weights")
    return synth.model_weights(wl, seed=1)


def _free():
    import gc

    import torch
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["8b", "8b_int8", "8b_int4"])
def test_full_size_short_prompt(name, w8b):
    """Full-size model, launch configuration of the bench: a 3-token prompt
    and 3 decode steps, every step compared with the oracle."""
    wl = synth.get(name)
    toks = synth.tokens(2, 6, wl.vocab)
    res, eng, _ = teacher_forced(wl, w8b, toks)
    del eng
    _free()
    agree, rel, mab = check_run(res, min_argmax=1.0, wl=wl)
    log(f"{name} short: argmax {agree:.3f} worst relL2 {rel:.2e} worst maxabs {mab:.2e}")


def test_full_size_random_gains(w8b):
    """8B bf16 shape with N(1, 0.25^2) bf16 RMSNorm gains at the attention,
    MLP and final norms (the other weights as in the bench): a 3-token
    prompt and 5 decode steps, every step compared with the oracle."""
    wl = synth.get("8b")
    w = dict(w8b)
    w.update(synth.random_gains(wl, seed=1))
    toks = synth.tokens(2, 8, wl.vocab)
    res, eng, _ = teacher_forced(wl, w, toks)
    del eng
    _free()
    agree, rel, mab = check_run(res, min_argmax=1.0, wl=wl)
    log(f"8b random gains: argmax {agree:.3f} worst relL2 {rel:.2e} worst maxabs {mab:.2e}")


@pytest.mark.parametrize("name", ["8b", "8b_int8", "8b_int4"])
def test_full_size_long_context(name, w8b):
    """Full-size model after the workload's prompt length (1024 positions; 8192
    for int4): the KV cache holds seeded rows 0..P-1 (same bytes on both
    sides), then 2 decode steps."""
    wl = synth.get(name)
    P = wl.prompt_len
    kvp = synth.kv_prefix(wl, P, seed=3)
    toks = synth.tokens(2, P + 2, wl.vocab)[P:]
    res, eng, _ = teacher_forced(wl, w8b, toks, kv_prefix=kvp, start=P)
    del eng
    _free()
    agree, rel, mab = check_run(res, min_argmax=1.0, wl=wl)
    log(f"{name} long: argmax {agree:.3f} worst relL2 {rel:.2e} worst maxabs {mab:.2e}")


@pytest.mark.parametrize("sched", [{"prefetch_kb": -1}, {"prefetch_kb": 4}, {"poll_mode": 1}, {"poll_mode": 2},
                                   {"poll_mode": 0}, {"poll_mode": 2, "pipeline_depth": 16},
                                   {"poll_mode": 2, "sync_mode": 0},
                                   {"sync_mode": 0}, {"sync_mode": 0, "poll_mode": 1},
                                   {"sync_mode": 0, "release_mode": 1}, {"sync_mode": 0, "attn_splits": 3},
                                   {"release_mode": 1}, {"pipeline_depth": 4}, {"pipeline_depth": 16},
                                   {"cu_policy": 1}, {"attn_splits": 3}, {"merge_place": 1},
                                   {"sync_mode": 1}, {"sync_mode": 2}, {"sync_mode": 1, "attn_splits": 3},
                                   {"sync_mode": 1, "prefetch_kb": -1, "prefetch_attn_kb": -1},
                                   {"poll_mode": 3}, {"poll_mode": 3, "sync_mode": 0},
                                   {"poll_mode": 3, "sync_mode": 2}, {"poll_mode": 3, "sync_mode": 0, "release_mode": 1},
                                   {"poll_mode": 3, "release_mode": 1}, {"poll_mode": 3, "prefetch_kb": 4},
                                   {"poll_mode": 3, "attn_splits": 3}, {"poll_mode": 3, "pipeline_depth": 16},
                                   {"poll_mode": 3, "prefetch_kb": -1, "prefetch_attn_kb": -1}],
                         ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
def test_schedule_knobs_keep_parity(sched):
    """Every ScheduleConfig knob the kernel reads, on the tiny decoder's full
    protocol (ragged rows, several tiles per queue): same parity bar."""
    wl = synth.get("tiny")
    w = synth.model_weights(wl, seed=1)
    toks = synth.tokens(2, wl.prompt_len + wl.decode_steps, wl.vocab)
    res, eng, _ = teacher_forced(wl, w, toks, sched=sched)
    del eng
    agree, rel, mab = check_run(res, min_argmax=1.0)
    log(f"tiny {sched}: argmax {agree:.3f} worst relL2 {rel:.2e} worst maxabs {mab:.2e}")


def test_tuner_keeps_only_safe_agreeing_faster_configs():
    """The schedule tuner on the tiny decoder with a three-knob space and the
    oracle's logits of its check steps as the CPU reference: the library
    default and every kept candidate passed the gate and matched both the
    CPU reference and the default schedule's logits; a reference that is
    off (scaled logits) makes the tuner refuse to start."""
    from oracle.reference import check_step_logits
    from persistent_megakernel_wg_amd import tune
    wl = synth.get("tiny")
    ref = check_step_logits(wl, synth.model_weights(wl, seed=1), 3)
    res = tune.tune(wl, steps=8, space=[("attn_splits", [1, 2]), ("pipeline_depth", [4, 16]), ("sync_mode", [0])],
                    reference=ref)
    assert res["cpu_reference"]
    h0 = res["history"][0]
    assert h0["kept"] and h0["cpu_ok"] and h0["cpu_rel_l2"] <= 1e-2
    measured = [h for h in res["history"][1:] if "error" not in h]
    assert measured and all("cpu_rel_l2" in h for h in measured)
    for h in res["history"][1:]:
        if h.get("kept"):
            assert h["parity"] and h["cpu_ok"] and h["cpu_rel_l2"] <= 1e-2
    log(f"tuner tiny: best {res['best']} {res['ms']:.4f} ms vs {res['reference_ms']:.4f} ms; "
        f"cpu relL2 of candidates {[round(h['cpu_rel_l2'], 9) for h in measured]}")
    with pytest.raises(RuntimeError, match="CPU reference"):
        tune.tune(wl, steps=4, space=[], xcd_rounds=0, reference=[r * 1.1 for r in ref])


@pytest.mark.parametrize("name", ["8b", "8b_int4"])
def test_tagged_sync_is_bit_identical(name, w8b):
    """sync_mode 1 and 2 (tagged activations) run the same arithmetic as the
    counter protocol: logits bit-identical over a few steps after a seeded
    KV prefix, at full size."""
    import torch

    import persistent_megakernel_wg_amd as amk
    from tests.gpu_common import device_cus
    wl = synth.get(name)
    m = amk.ModelConfig.from_workload(wl)
    dev_w = amk.upload_model(m, w8b)
    P = 100
    kvp = torch.from_numpy(synth.kv_prefix(wl, P, seed=3).view(np.int16).reshape(-1)).cuda()
    toks = synth.tokens(2, P + 4, wl.vocab)[P:]
    outs = []
    for mode in (0, 1, 2):
        cfg = amk.default_schedule_config(m, device_cus())
        cfg.sync_mode = mode
        sched = amk.Schedule.build(m, cfg)
        kv, logits = amk.alloc_state(m)
        kv.copy_(kvp)
        eng = amk.Engine(sched, dev_w, kv, logits)
        eng.set_kv_length(P)
        got = []
        for i, tok in enumerate(toks):
            eng.decode_step(int(tok), P + i)
            torch.cuda.synchronize()
            eng.check()
            got.append(logits.cpu().numpy().copy())
        outs.append(np.stack(got))
        eng.close()
        sched.close()
        del kv, logits
    for k in (1, 2):
        assert np.array_equal(outs[0].view(np.uint32), outs[k].view(np.uint32)), k
    log(f"{name}: sync_mode 1 and 2 bit-identical to sync_mode 0 over {len(toks)} steps")
