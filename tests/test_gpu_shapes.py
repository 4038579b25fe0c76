"""Parity of the HIP path on shapes and inputs the seeded workloads do not
reach: non-unit RMSNorm gains at all three norm sites (attention, MLP,
final), and attention group shapes that take the other lane layouts and
the multi-pass head loop (head_dim 64 / 128 / 256, 1 to 16 query heads per
kv head).  Every step is compared with the oracle on the same seeded inputs.
"""
import pytest

import synth
from tests.gpu_common import check_run, log, teacher_forced

pytestmark = pytest.mark.gpu


def test_tiny_random_gains_full_protocol():
    """Tiny decoder with N(1, 0.25^2) bf16 gains: 16-token prompt + 32 decode
    steps, every step compared (a gain read at a wrong index, or not applied,
    fails this)."""
    wl = synth.get("tiny")
    w = synth.model_weights(wl, seed=1, gains="random")
    toks = synth.tokens(2, wl.prompt_len + wl.decode_steps, wl.vocab)
    res, eng, _ = teacher_forced(wl, w, toks)
    del eng
    agree, rel, mab = check_run(res, min_argmax=1.0)
    log(f"tiny random gains: argmax {agree:.3f} worst relL2 {rel:.2e} worst maxabs {mab:.2e}")


# (head_dim, query heads, kv heads): heads per pass = min(pow2 >= group, 512 / head_dim)
SHAPES = [
    (64, 16, 2),    # group 8: one pass of 8 heads, 8 lanes per row
    (64, 32, 2),    # group 16: two passes of 8
    (64, 6, 1),     # group 6: one pass of 8 with two idle head slots
    (128, 16, 2),   # group 8: two passes of 4
    (128, 4, 4),    # group 1 (multi-head attention)
    (256, 8, 2),    # group 4: two passes of 2, 32 lanes per row
    (256, 2, 2),    # group 1 at head_dim 256
]


@pytest.mark.parametrize("hd,nq,nkv", SHAPES, ids=lambda v: str(v))
def test_attention_group_shapes(hd, nq, nkv):
    """A two-layer decoder (hidden 256, FFN 688, vocab 4096) with the given
    attention shape and random gains: 24-token prompt + 16 decode steps at a
    64-position cache, every step compared; the library's defaults keep the
    LDS prefetch off at this size, so the LDS holds exactly what the tasks
    use."""
    wl = synth.get("tiny").with_(name=f"attn_{hd}_{nq}_{nkv}", n_heads=nq, n_kv_heads=nkv,
                                 head_dim=hd, prompt_len=24, decode_steps=16, max_ctx=64)
    w = synth.model_weights(wl, seed=1, gains="random")
    toks = synth.tokens(2, wl.prompt_len + wl.decode_steps, wl.vocab)
    res, eng, _ = teacher_forced(wl, w, toks)
    del eng
    agree, rel, mab = check_run(res, min_argmax=1.0)
    log(f"{wl.name}: argmax {agree:.3f} worst relL2 {rel:.2e} worst maxabs {mab:.2e}")


# (weight format, bf16 projection inputs)
QUANT = [("int8", False), ("int8", True), ("int4", False), ("int4", True)]


@pytest.mark.parametrize("wfmt,act_bf16", QUANT, ids=lambda v: str(v))
def test_tiny_quantised_formats(wfmt, act_bf16):
    """The int8 and int4 GEMV bodies on a two-layer decoder (hidden 256, FFN
    768 so that every int4 row holds whole groups of 128, random gains): 24-token
    prompt + 16 decode steps, every step compared with the oracle, which
    dequantises the same packed codes.  With bf16 projection inputs the int4
    body's remainder terms are zero, so both of its input paths are taken."""
    wl = synth.get("tiny").with_(name=f"tiny_{wfmt}_{'a16' if act_bf16 else 'a32'}", wfmt=wfmt,
                                 act_bf16=act_bf16, ffn=768, prompt_len=24, decode_steps=16, max_ctx=64)
    w = synth.model_weights(wl, seed=1, gains="random")
    toks = synth.tokens(2, wl.prompt_len + wl.decode_steps, wl.vocab)
    res, eng, _ = teacher_forced(wl, w, toks)
    del eng
    agree, rel, mab = check_run(res, min_argmax=1.0, wl=wl)
    log(f"{wl.name}: argmax {agree:.3f} worst relL2 {rel:.2e} worst maxabs {mab:.2e}")


@pytest.mark.parametrize("hd,nq,nkv", SHAPES, ids=lambda v: str(v))
def test_attention_group_shapes_long_splits(hd, nq, nkv):
    """The position-major attention layout (splits of 128 positions or more)
    on every group shape: a two-layer decoder with a 384-position cache and
    2 attention splits per kv head, 290-token prompt + 6 decode steps (splits
    of 145..148 positions), every decode step compared with the oracle; the
    prompt's steps take the head-major layout and build the cache on both
    sides."""
    wl = synth.get("tiny").with_(name=f"attnL_{hd}_{nq}_{nkv}", n_heads=nq, n_kv_heads=nkv,
                                 head_dim=hd, prompt_len=290, decode_steps=6, max_ctx=384)
    w = synth.model_weights(wl, seed=1, gains="random")
    toks = synth.tokens(2, wl.prompt_len + wl.decode_steps, wl.vocab)
    res, eng, _ = teacher_forced(wl, w, toks, compare_from=255, sched={"attn_splits": 2})
    del eng
    agree, rel, mab = check_run(res, min_argmax=1.0)
    log(f"{wl.name}: {len(res)} steps compared, argmax {agree:.3f} worst relL2 {rel:.2e} worst maxabs {mab:.2e}")


@pytest.mark.parametrize("sched", [{"sync_mode": 0}, {"poll_mode": 3}, {"poll_mode": 3, "sync_mode": 0},
                                   {"sync_mode": 2}], ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
def test_attention_long_splits_under_schedule_knobs(sched):
    """The position-major attention layout under the counter protocol (q and
    the row at pos read after the acquire) and with DMA waves (positions on
    waves 0..5, input reads by the input threads only): hd 128, 8 query heads
    per kv head (two passes), 2 splits of 145+ positions."""
    wl = synth.get("tiny").with_(name="attnL_knobs", n_heads=16, n_kv_heads=2, head_dim=128,
                                 prompt_len=290, decode_steps=6, max_ctx=384)
    w = synth.model_weights(wl, seed=1, gains="random")
    toks = synth.tokens(2, wl.prompt_len + wl.decode_steps, wl.vocab)
    res, eng, _ = teacher_forced(wl, w, toks, compare_from=255, sched=dict(sched, attn_splits=2))
    del eng
    agree, rel, mab = check_run(res, min_argmax=1.0)
    log(f"{wl.name} {sched}: {len(res)} steps, argmax {agree:.3f} worst relL2 {rel:.2e} worst maxabs {mab:.2e}")
