"""Shared helpers of the GPU tests: run the HIP path and the oracle on the
same seeded inputs and compare logits with the parity criteria.

Parity bar (per decode step): relative L2 error <= 1e-2 and max |g - o| <=
2e-2 * max |o|; over a run, argmax agreement >= 99 %.
"""
import sys

import numpy as np

import oracle
import synth

REL_L2 = 1e-2
MAX_ABS = 2e-2
ARGMAX = 0.99


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def device_cus():
    import torch
    return torch.cuda.get_device_properties(0).multi_processor_count


def make_engine(wl, weights, sched_overrides=None):
    import persistent_megakernel_wg_amd as amk
    m = amk.ModelConfig.from_workload(wl)
    cfg = amk.default_schedule_config(m, device_cus())
    for k, v in (sched_overrides or {}).items():
        setattr(cfg, k, v)
    sched = amk.Schedule.build(m, cfg)
    assert sched.validate()[0] == 0
    dev_w = amk.upload_model(m, weights)
    kv, logits = amk.alloc_state(m)
    eng = amk.Engine(sched, dev_w, kv, logits)
    return eng


def gpu_step(eng, token, pos):
    import torch
    eng.decode_step(token, pos)
    torch.cuda.synchronize()
    eng.check()
    return eng.logits.cpu().numpy().astype(np.float64)


def compare(got, want):
    """(rel_l2, max_abs_ratio, argmax_equal)"""
    err = got - want
    rel = float(np.linalg.norm(err) / np.linalg.norm(want))
    mab = float(np.max(np.abs(err)) / np.max(np.abs(want)))
    return rel, mab, int(np.argmax(got)) == int(np.argmax(want))


def check_run(results, min_argmax=ARGMAX):
    agree = sum(r[2] for r in results) / len(results)
    worst_rel = max(r[0] for r in results)
    worst_abs = max(r[1] for r in results)
    assert worst_rel <= REL_L2, f"relL2 {worst_rel:.3e} > {REL_L2}"
    assert worst_abs <= MAX_ABS, f"max-abs ratio {worst_abs:.3e} > {MAX_ABS}"
    assert agree >= min_argmax, f"argmax agreement {agree:.3f} < {min_argmax}"
    return agree, worst_rel, worst_abs


def teacher_forced(wl, weights, toks, compare_from=0, kv_prefix=None, start=0, sched=None):
    """Run positions start.. over toks on both sides; compare steps >= compare_from."""
    eng = make_engine(wl, weights, sched)
    orc = oracle.Model(wl, weights)
    kv_o = orc.new_kv() if kv_prefix is None else kv_prefix.copy()
    if kv_prefix is not None:
        import torch
        eng.kv_cache.copy_(torch.from_numpy(kv_prefix.view(np.int16).reshape(-1)))
        eng.set_kv_length(start)
    results = []
    for i, tok in enumerate(toks):
        pos = start + i
        g = gpu_step(eng, tok, pos)
        o = orc.step(kv_o, tok, pos)
        if pos >= compare_from:
            results.append(compare(g, o))
    return results, eng, kv_o
