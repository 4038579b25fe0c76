"""Host side of the C ABI (no GPU): every function include/amk.h declares is
exported by libamk.so; packing and quantisation are bit-identical to the
oracle's quantisers; configuration and argument errors return the documented
status codes with a message."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import persistent_megakernel_wg_amd as amk
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "amk.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(amk_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 20
    lib = ctypes.CDLL(amk.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert set(names) <= set(amk.EXPORTED) | set(names)


def test_status_strings():
    lib = ctypes.CDLL(amk.LIB_PATH)
    lib.amk_status_string.restype = ctypes.c_char_p
    for code, name in [(0, b"AMK_OK"), (-1, b"AMK_ERR_INVALID_ARG"), (-2, b"AMK_ERR_UNSUPPORTED"),
                       (-3, b"AMK_ERR_UNSAFE_SCHEDULE"), (-4, b"AMK_ERR_OUT_OF_RANGE"), (-5, b"AMK_ERR_HIP"),
                       (-6, b"AMK_ERR_NOMEM"), (-7, b"AMK_ERR_TIMEOUT")]:
        assert lib.amk_status_string(code) == name


def small_workload(wfmt, tied=False):
    return synth.get("tiny").with_(n_layers=2, hidden=256, ffn=512, vocab=384, wfmt=wfmt, tied=tied,
                                   max_ctx=64, act_bf16=wfmt == "int8")


# canonical ids of the projections inside packed tensor k
def projections(wl, k):
    L = wl.n_layers
    if k == 0:
        return [0]
    if k == 1:
        return [1 + 9 * L]
    if k == 2:
        return [0 if wl.tied else 2 + 9 * L]
    l, sub = divmod(k - 3, 6)
    return {0: [1 + 9 * l], 1: [1 + 9 * l + 1, 1 + 9 * l + 2, 1 + 9 * l + 3], 2: [1 + 9 * l + 4],
            3: [1 + 9 * l + 5], 4: [1 + 9 * l + 6, 1 + 9 * l + 7], 5: [1 + 9 * l + 8]}[sub]


QUANTISED_SUBS = (1, 2, 4, 5)


@pytest.mark.parametrize("wfmt,tied", [("bf16", False), ("bf16", True), ("int8", False), ("int4", False)])
def test_pack_unpack_matches_oracle_quantisers(wfmt, tied):
    wl = small_workload(wfmt, tied)
    m = amk.ModelConfig.from_workload(wl)
    w = synth.model_weights(wl, seed=5)
    n = amk.packed_count(m)
    assert n == 3 + 6 * wl.n_layers
    for k in range(n):
        packed = amk.pack_tensor(m, k, w)
        assert packed.nbytes == amk.packed_bytes(m, k)
        quantised = wfmt != "bf16" and (k == 2 or (k >= 3 and (k - 3) % 6 in QUANTISED_SUBS))
        for cid in projections(wl, k):
            W = w[cid]
            R, C = W.shape if W.ndim == 2 else (1, W.size)
            q, s, z = amk.unpack_tensor(m, k, cid, packed, R, C)
            if not quantised:
                assert np.array_equal(q.reshape(-1), W.reshape(-1))
            elif wfmt == "int8":
                oq, os_ = oracle.quant_int8(W)
                assert np.array_equal(q, oq), (k, cid)
                assert np.array_equal(s.view(np.uint32), os_.view(np.uint32)), (k, cid)
            else:
                op, osc, oz = oracle.quant_int4(W)
                assert np.array_equal(q, op), (k, cid)
                assert np.array_equal(s, osc) and np.array_equal(z, oz), (k, cid)


def test_packed_sizes_follow_the_formats():
    for wfmt, per in (("bf16", lambda r, c: r * c * 2), ("int8", lambda r, c: r * c + 4 * r),
                      ("int4", lambda r, c: r * c // 2 + r * (c // 128) * 4)):
        wl = small_workload(wfmt)
        m = amk.ModelConfig.from_workload(wl)
        H, F = wl.hidden, wl.ffn
        qkv = (wl.n_heads + 2 * wl.n_kv_heads) * wl.head_dim
        assert amk.packed_bytes(m, 3 + 1) == per(qkv, H)
        assert amk.packed_bytes(m, 3 + 2) == per(H, wl.n_heads * wl.head_dim)
        assert amk.packed_bytes(m, 3 + 4) == per(2 * F, H)
        assert amk.packed_bytes(m, 3 + 5) == per(H, F)
        assert amk.packed_bytes(m, 2) == per(wl.vocab, H)
        assert amk.packed_bytes(m, 0) == wl.vocab * H * 2    # embedding stays bf16
        assert amk.packed_bytes(m, 3) == H * 2               # norms stay bf16
    m = amk.ModelConfig.from_workload(small_workload("bf16"))
    assert amk.kv_bytes(m) == m.n_layers * 2 * m.n_kv_heads * m.max_ctx * m.head_dim * 2


def expect_status(code, fn, *args):
    with pytest.raises(amk.AmkError) as e:
        fn(*args)
    assert e.value.status == code, (e.value.status, str(e.value))
    assert str(e.value)


def test_unsupported_and_invalid_models():
    base = amk.ModelConfig.from_workload(small_workload("bf16"))
    cfg = amk.default_schedule_config(base, 8)

    def variant(**kw):
        m = amk.ModelConfig.from_workload(small_workload("bf16"))
        for k, v in kw.items():
            setattr(m, k, v)
        return m
    expect_status(amk.ERR_UNSUPPORTED, amk.Schedule.build, variant(attn_bias=1), cfg)
    expect_status(amk.ERR_UNSUPPORTED, amk.Schedule.build, variant(mlp_bias=1), cfg)
    expect_status(amk.ERR_UNSUPPORTED, amk.Schedule.build, variant(n_heads=3, n_kv_heads=2), cfg)
    expect_status(amk.ERR_UNSUPPORTED, amk.Schedule.build, variant(head_dim=63), cfg)
    expect_status(amk.ERR_INVALID_ARG, amk.Schedule.build, variant(hidden=0), cfg)
    expect_status(amk.ERR_INVALID_ARG, amk.Schedule.build, variant(n_layers=-1), cfg)
    expect_status(amk.ERR_UNSUPPORTED, amk.Schedule.build, variant(wfmt=2, hidden=200), cfg)


def test_invalid_schedule_configs():
    m = amk.ModelConfig.from_workload(small_workload("bf16"))
    for field, value, code in [("pipeline_depth", 5, amk.ERR_UNSUPPORTED), ("attn_splits", 300, amk.ERR_UNSUPPORTED),
                               ("cu_policy", 2, amk.ERR_UNSUPPORTED), ("fuse_flags", 0x3, amk.ERR_UNSUPPORTED),
                               ("wg_threads", 256, amk.ERR_UNSUPPORTED), ("num_cus", 0, amk.ERR_INVALID_ARG),
                               ("poll_mode", 4, amk.ERR_UNSUPPORTED), ("release_mode", 3, amk.ERR_UNSUPPORTED)]:
        c = amk.default_schedule_config(m, 8)
        setattr(c, field, value)
        expect_status(code, amk.Schedule.build, m, c)


def test_default_config_resolves_every_field():
    m = amk.ModelConfig.from_workload(synth.get("8b"))
    c = amk.default_schedule_config(m, 256)
    d = c.as_dict()
    assert d["num_cus"] == 256 and d["wg_threads"] == 512 and d["pipeline_depth"] in (4, 8, 16)
    assert all(d[k] == 256 for k in ("tiles_qkv", "tiles_o", "tiles_gateup", "tiles_down", "tiles_lm"))
    assert d["attn_splits"] == 3 * 256 // (4 * 8) and d["prefetch_kb"] == 64
    assert d["sync_mode"] == 1 and d["merge_place"] == 0 and d["prefetch_attn_kb"] == 1024 and d["poll_mode"] == 2


def test_packed_ids_out_of_range():
    m = amk.ModelConfig.from_workload(small_workload("int8"))
    expect_status(amk.ERR_OUT_OF_RANGE, amk.packed_bytes, m, 3 + 6 * m.n_layers)
    expect_status(amk.ERR_OUT_OF_RANGE, amk.packed_bytes, m, -1)


def test_from_desc_rejects_malformed_arrays():
    s = {"n_counters": 0, "buffers": [(16, 2)], "tasks": [{"type": 0, "cu": 0, "p": [], "waits": [], "sigs": [],
                                                             "acc": [(0, 2, 0, 16)]}], "queues": [[0]]}
    sch = amk.Schedule.from_dict(s)
    assert sch.validate() == (0, -1, -1, -1)
    sch.close()
    bad = dict(s, n_counters=-1)
    expect_status(amk.ERR_INVALID_ARG, amk.Schedule.from_dict, bad)


def test_lowering_is_deterministic_and_safe_at_full_size():
    for name in ("1b", "8b", "8b_int4"):
        m = amk.ModelConfig.from_workload(synth.get(name))
        c = amk.default_schedule_config(m, 256)
        a, b = amk.Schedule.build(m, c), amk.Schedule.build(m, c)
        assert a.validate() == (0, -1, -1, -1)
        va, vb = a.view(), b.view()
        assert va["tasks"] == vb["tasks"] and va["queues"] == vb["queues"]
        a.close()
        b.close()


def test_xcd_weights_shift_rows_and_stay_safe():
    m = amk.ModelConfig.from_workload(synth.get("8b"))
    c = amk.default_schedule_config(m, 256)
    base = amk.Schedule.build(m, c).view()
    for x in range(8):
        c.xcd_weight[2][x] = 900 if x % 2 else 1100   # gate/up
        c.xcd_weight[4][x] = 900 if x % 2 else 1100   # LM head
    sch = amk.Schedule.build(m, c)
    assert sch.validate() == (0, -1, -1, -1)
    v = sch.view()
    for ty, lo, hi in ((5, 1, 2), (7, 0, 1)):  # gate/up units, LM-head rows
        rows = {}
        for t in v["tasks"]:
            if t["type"] == ty and (ty == 7 or t["p"][0] == 0):
                rows[t["cu"]] = t["p"][hi] - t["p"][lo]
        even = np.mean([r for cu, r in rows.items() if cu % 2 == 0])
        odd = np.mean([r for cu, r in rows.items() if cu % 2 == 1])
        assert abs(even / odd - 1100 / 900) < 0.03, (ty, even, odd)
    # the other phases keep the even split
    qkv = {t["cu"]: t["p"][2] - t["p"][1] for t in v["tasks"] if t["type"] == 1 and t["p"][0] == 0}
    assert max(qkv.values()) - min(qkv.values()) <= 1
    assert len(base["tasks"]) == len(v["tasks"])
    c.xcd_weight[3][3] = 50
    expect_status(amk.ERR_INVALID_ARG, amk.Schedule.build, m, c)


def test_merge_tasks_avoid_attention_queues():
    m = amk.ModelConfig.from_workload(synth.get("8b"))
    for place, disjoint in ((0, True), (1, False)):
        c = amk.default_schedule_config(m, 256)
        c.merge_place = place
        s = amk.Schedule.build(m, c)
        assert s.validate() == (0, -1, -1, -1)
        v = s.view()
        for layer in (0, 31):
            att = {t["cu"] for t in v["tasks"] if t["type"] == 2 and t["p"][0] == layer}
            mer = [t["cu"] for t in v["tasks"] if t["type"] == 3 and t["p"][0] == layer]
            assert len(mer) == m.n_heads and len(set(mer)) == m.n_heads
            assert (not (att & set(mer))) == disjoint
        s.close()
    c = amk.default_schedule_config(m, 256)
    c.merge_place = 2
    expect_status(amk.ERR_UNSUPPORTED, amk.Schedule.build, m, c)
    c = amk.default_schedule_config(m, 256)
    c.prefetch_attn_kb = -2
    expect_status(amk.ERR_INVALID_ARG, amk.Schedule.build, m, c)


def test_sync_mode_limits():
    m = amk.ModelConfig.from_workload(synth.get("8b"))
    for mode, splits, code in ((3, 24, amk.ERR_UNSUPPORTED), (1, 65, amk.ERR_UNSUPPORTED),
                               (2, 65, amk.ERR_UNSUPPORTED), (-1, 24, amk.ERR_UNSUPPORTED)):
        c = amk.default_schedule_config(m, 256)
        c.sync_mode, c.attn_splits = mode, splits
        expect_status(code, amk.Schedule.build, m, c)
    for mode in (0, 1, 2):
        c = amk.default_schedule_config(m, 256)
        c.sync_mode, c.attn_splits = mode, 64
        s = amk.Schedule.build(m, c)
        assert s.validate() == (0, -1, -1, -1)
        s.close()
    # with DMA waves (poll_mode 3), 384 threads read a merge's partials:
    # tagged modes need attn_splits * head_dim <= 6144 (48 splits at 128)
    for mode, splits, ok in ((1, 48, True), (1, 49, False), (2, 49, False), (0, 49, True)):
        c = amk.default_schedule_config(m, 256)
        c.sync_mode, c.attn_splits, c.poll_mode = mode, splits, 3
        if ok:
            s = amk.Schedule.build(m, c)
            assert s.validate() == (0, -1, -1, -1)
            s.close()
        else:
            expect_status(amk.ERR_UNSUPPORTED, amk.Schedule.build, m, c)
    # the default falls back to counters where the split count is too large
    c = amk.default_schedule_config(amk.ModelConfig.from_workload(synth.get("8b").with_(n_kv_heads=1, n_heads=16)), 256)
    assert c.sync_mode == 0


def test_defaults_follow_format_and_context():
    """Automatic schedule fields: 64 KB prefetch and half of the ring issued
    after the wait for bf16 weights at hidden >= 4096, no prefetch and the
    polling wave's ring after the wait otherwise; a 4-deep ring for int4
    weights, 8 otherwise; 3/4 of the queues run attention splits (8 per kv
    head up to a 512-position cache; past 4096 positions, as many as leave
    one split-free queue per query head)."""
    for name, splits, pf, poll, depth in (("8b", 24, 64, 2, 8), ("8b_int8", 24, -1, 1, 8), ("8b_int4", 28, -1, 1, 4),
                                          ("1b", 8, -1, 1, 8), ("tiny", 8, -1, 1, 8)):
        m = amk.ModelConfig.from_workload(synth.get(name))
        d = amk.default_schedule_config(m, 256).as_dict()
        assert (d["attn_splits"], d["prefetch_kb"], d["poll_mode"], d["pipeline_depth"]) == (splits, pf, poll, depth), name


@pytest.mark.parametrize("ncu,nq,nkv", [(256, 32, 8), (304, 64, 8), (80, 32, 8), (64, 16, 4), (40, 32, 8),
                                        (24, 32, 8), (16, 4, 2), (8, 4, 2)])
def test_long_context_default_splits_leave_a_queue_per_merge(ncu, nq, nkv):
    """Past 4096 positions the automatic split count is
    max(1, (num_cus - n_heads) / n_kv_heads): the lowering passes the gate,
    no merge shares a queue with an attention split of its layer, and every
    merge has a queue of its own whenever the queues suffice."""
    wl = synth.get("tiny").with_(n_heads=nq, n_kv_heads=nkv, hidden=nq * 64, max_ctx=8192)
    m = amk.ModelConfig.from_workload(wl)
    cfg = amk.default_schedule_config(m, ncu)
    assert cfg.attn_splits == max(1, (ncu - nq) // nkv)
    s = amk.Schedule.build(m, cfg)
    try:
        assert s.validate()[0] == 0
        v = s.view()
        for layer in range(wl.n_layers):
            attn_q = {t["cu"] for t in v["tasks"] if t["type"] == 2 and t["p"][0] == layer}
            merge_q = [t["cu"] for t in v["tasks"] if t["type"] == 3 and t["p"][0] == layer]
            assert len(attn_q) == cfg.attn_splits * nkv
            assert not attn_q & set(merge_q)
            if ncu - cfg.attn_splits * nkv >= nq:
                assert len(set(merge_q)) == len(merge_q) == nq
    finally:
        s.close()
