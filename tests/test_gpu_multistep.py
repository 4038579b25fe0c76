"""Greedy multi-step decode in one launch (amk_decode_steps) on MI355X: the
device-side argmax and token feedback give the same tokens and bit-identical
logits as one launch per step with the argmax taken on the host, and the
oracle, decoding greedily on its own from the same prompt, chooses the same
tokens and agrees on the last step's logits."""
import numpy as np
import pytest

import oracle
import persistent_megakernel_wg_amd as amk
import synth
from tests.gpu_common import bars, compare, device_cus, log

pytestmark = pytest.mark.gpu


def _engine(wl, w, **sched):
    m = amk.ModelConfig.from_workload(wl)
    cfg = amk.default_schedule_config(m, device_cus())
    for k, v in sched.items():
        setattr(cfg, k, v)
    s = amk.Schedule.build(m, cfg)
    kv, logits = amk.alloc_state(m)
    return amk.Engine(s, amk.upload_model(m, w), kv, logits), s


def _host_loop(eng, tok, pos, n):
    import torch
    toks = []
    for i in range(n):
        eng.decode_step(tok, pos + i)
        torch.cuda.synchronize()
        eng.check()
        lg = eng.logits.cpu().numpy()
        tok = int(np.argmax(lg))  # first index of the max: lowest on ties
        toks.append(tok)
    return toks, lg.copy()


def _oracle_greedy(wl, w, prompt, p0, n, kv_prefix=None):
    """The oracle's own greedy decode: prompt[:p0] (or a KV prefix of p0
    rows) then n steps starting from prompt[p0], each next token the argmax
    of the oracle's logits (lowest index on ties).  (tokens, last logits)."""
    orc = oracle.Model(wl, w)
    kv = orc.new_kv() if kv_prefix is None else kv_prefix.copy()
    if kv_prefix is None:
        for i in range(p0):
            orc.step(kv, int(prompt[i]), i)
    tok, toks = int(prompt[p0]), []
    for i in range(n):
        o = orc.step(kv, tok, p0 + i)
        tok = int(np.argmax(o))
        toks.append(tok)
    orc.close()
    return toks, o


@pytest.mark.parametrize("sync_mode,long_splits", [(1, False), (0, False), (1, True)],
                         ids=["tagged", "counters", "tagged-long-splits"])
def test_multistep_matches_host_loop_and_oracle(sync_mode, long_splits):
    """long_splits: a 300-position cache, 2 attention splits per kv head and
    a 257-token prompt, so every greedy step (positions 256..275) takes the
    position-major attention layout (splits of 128+ positions)."""
    import torch
    wl = synth.get("tiny")
    sched = {"sync_mode": sync_mode}
    plen = 8
    if long_splits:
        wl = wl.with_(name="tiny_ms_long", max_ctx=300, prompt_len=256, decode_steps=40)
        sched["attn_splits"] = 2
        plen = 257
    w = synth.model_weights(wl, seed=1)
    prompt = synth.tokens(2, plen, wl.vocab)
    n = 20
    a, sa = _engine(wl, w, **sched)
    b, sb = _engine(wl, w, **sched)
    for i, t in enumerate(prompt[:-1]):
        a.decode_step(int(t), i)
        b.decode_step(int(t), i)
    p0 = len(prompt) - 1
    host_toks, host_logits = _host_loop(a, int(prompt[-1]), p0, n)
    out = torch.zeros(n, dtype=torch.int32, device="cuda")
    b.decode_steps(int(prompt[-1]), p0, n, out)
    torch.cuda.synchronize()
    b.check()
    dev_toks = out.cpu().numpy().tolist()
    assert dev_toks == host_toks, (dev_toks, host_toks)
    assert np.array_equal(b.logits.cpu().numpy().view(np.uint32), host_logits.view(np.uint32))
    # the oracle decodes greedily on its own from the same prompt
    orc_toks, o = _oracle_greedy(wl, w, prompt, p0, n)
    assert orc_toks == dev_toks, (orc_toks, dev_toks)
    rel, mab, same = compare(host_logits.astype(np.float64), o, bars(wl)[2])
    assert rel <= bars(wl)[0] and mab <= bars(wl)[1] and same, (rel, mab)
    log(f"multistep {wl.name} sync_mode {sync_mode}: {n} tokens identical to the host loop and the oracle, "
        f"final relL2 {rel:.2e}")
    for e, s in ((a, sa), (b, sb)):
        e.close()
        s.close()


def test_multistep_full_size_and_errors():
    """8B bf16 after a seeded 1024-row KV prefix: 8 greedy steps in one launch
    equal 8 single-step launches; argument errors are refused on the host."""
    import torch
    wl = synth.get("8b")
    w = synth.model_weights(wl, seed=1)
    P = 1024
    kvp_host = synth.kv_prefix(wl, P, seed=3)
    kvp = torch.from_numpy(kvp_host.view(np.int16).reshape(-1)).cuda()
    a, sa = _engine(wl, w)
    b, sb = _engine(wl, w)
    for e in (a, b):
        e.kv_cache.copy_(kvp)
        e.set_kv_length(P)
    n = 8
    host_toks, host_logits = _host_loop(a, 7, P, n)
    out = torch.zeros(n, dtype=torch.int32, device="cuda")
    b.decode_steps(7, P, n, out)
    torch.cuda.synchronize()
    b.check()
    assert out.cpu().numpy().tolist() == host_toks
    assert np.array_equal(b.logits.cpu().numpy().view(np.uint32), host_logits.view(np.uint32))
    # the oracle's own greedy decode after the same KV prefix: same tokens,
    # and the last step's logits within the parity bar
    orc_toks, o = _oracle_greedy(wl, w, np.array([0] * P + [7]), P, n, kv_prefix=kvp_host)
    del w, kvp_host
    assert orc_toks == host_toks, (orc_toks, host_toks)
    rel, mab, same = compare(host_logits.astype(np.float64), o)
    assert rel <= bars(wl)[0] and mab <= bars(wl)[1] and same, (rel, mab)
    for args, code in (((7, P, 0, out), amk.ERR_OUT_OF_RANGE), ((7, wl.max_ctx - 2, 4, out), amk.ERR_OUT_OF_RANGE),
                       ((7, P + n + 1, 2, out), amk.ERR_INVALID_ARG)):
        with pytest.raises(amk.AmkError) as e:
            b.decode_steps(*args)
        assert e.value.status == code
    log(f"8b: {n} greedy steps in one launch match the host loop and the oracle: {host_toks}, "
        f"last-step relL2 {rel:.2e}")
    for e, s in ((a, sa), (b, sb)):
        e.close()
        s.close()


def test_region_stats_account_for_the_traced_launch():
    """amk_engine_region_stats: task counts per type match the schedule, every
    duration is non-negative, and the critical-path shares of the types add
    up to the traced launch's length (first wait begin to last signal)."""
    import torch
    wl = synth.get("tiny")
    w = synth.model_weights(wl, seed=1)
    eng, sched = _engine(wl, w)
    with pytest.raises(amk.AmkError):
        eng.region_stats()  # tracing never enabled
    eng.decode_step(3, 0)
    torch.cuda.synchronize()
    eng.check()
    untraced = eng.logits.cpu().numpy().copy()
    eng.set_trace(True)
    eng.decode_step(3, 0)  # the same step again (rewind), traced
    torch.cuda.synchronize()
    eng.check()
    # timing does not change what is timed: the traced launch's logits are
    # bit-identical to the untraced launch's
    assert np.array_equal(eng.logits.cpu().numpy().view(np.uint32), untraced.view(np.uint32))
    view = sched.view()
    stats = eng.region_stats()
    counts = {}
    for t in view["tasks"]:
        counts[amk.TASK_NAMES[t["type"]]] = counts.get(amk.TASK_NAMES[t["type"]], 0) + 1
    assert {k: v["n_tasks"] for k, v in stats.items()} == counts
    for v in stats.values():
        assert min(v["wait_us"], v["work_us"], v["signal_us"], v["span_us"]) >= 0.0
    st, khz = eng.read_trace(len(view["tasks"]))
    span = (int(st[:, 3].max()) - int(st[:, 0].min())) * 1e3 / khz
    total = sum(v["span_us"] for v in stats.values())
    assert abs(total - span) <= 1e-6 * span + 1e-3, (total, span)
    log(f"region stats: {total:.1f} us over {len(stats)} task types")
    eng.close()
    sched.close()


def test_multistep_to_the_last_position_and_single_step_equivalence():
    """Tiny decoder: greedy steps up to the last cache position in one launch
    equal the host loop; a one-step multi-step launch equals decode_step."""
    import torch
    wl = synth.get("tiny")
    w = synth.model_weights(wl, seed=1)
    a, sa = _engine(wl, w)
    b, sb = _engine(wl, w)
    p0 = 4
    for i in range(p0):
        a.decode_step(i + 1, i)
        b.decode_step(i + 1, i)
    n = wl.max_ctx - p0
    host_toks, host_logits = _host_loop(a, 9, p0, n)
    out = torch.zeros(n, dtype=torch.int32, device="cuda")
    b.decode_steps(9, p0, n, out)
    torch.cuda.synchronize()
    b.check()
    assert out.cpu().numpy().tolist() == host_toks
    assert np.array_equal(b.logits.cpu().numpy().view(np.uint32), host_logits.view(np.uint32))
    # the oracle's own greedy decode from the same prompt (1, 2, 3, 4, then 9)
    orc_toks, o = _oracle_greedy(wl, w, np.array([1, 2, 3, 4, 9]), p0, n)
    assert orc_toks == host_toks, (orc_toks, host_toks)
    rel, mab, same = compare(host_logits.astype(np.float64), o)
    assert rel <= bars(wl)[0] and mab <= bars(wl)[1] and same, (rel, mab)
    # rewind and take one step through each entry point
    one = torch.zeros(1, dtype=torch.int32, device="cuda")
    a.decode_step(5, p0)
    b.decode_steps(5, p0, 1, one)
    torch.cuda.synchronize()
    a.check()
    b.check()
    la, lb = a.logits.cpu().numpy(), b.logits.cpu().numpy()
    assert np.array_equal(la.view(np.uint32), lb.view(np.uint32))
    assert int(one.cpu()[0]) == int(np.argmax(la))
    for e, s in ((a, sa), (b, sb)):
        e.close()
        s.close()
