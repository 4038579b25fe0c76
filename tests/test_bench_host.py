"""bench.py host logic (no GPU): the refusal of more than one GPU, and the
algorithmic bytes of a decode step behind the floor fraction and the
roofline, checked against the byte count of each stored tensor written out
from the model shapes and the weight formats' definitions (bf16: 2 bytes a
weight; int8: a byte a weight plus a 4-byte scale per output row; int4 g128:
half a byte a weight plus a 2-byte scale and a 2-byte zero per group of 128
inputs; a tied LM head reads the bf16 embedding table)."""
import os
import subprocess
import sys

import pytest

import persistent_megakernel_wg_amd as amk
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)


def expected_step_bytes(wl, pos):
    H, F, L, V = wl.hidden, wl.ffn, wl.n_layers, wl.vocab
    nq, nkv, hd = wl.n_heads, wl.n_kv_heads, wl.head_dim

    def proj(rows, k):
        if wl.wfmt == "bf16":
            return rows * k * 2
        if wl.wfmt == "int8":
            return rows * k + rows * 4
        assert wl.wfmt == "int4"
        return rows * k // 2 + rows * (k // 128) * 4

    layer = (2 * H * 2                      # attention and MLP norm gains
             + proj((nq + 2 * nkv) * hd, H)  # q, k, v
             + proj(H, nq * hd)              # o
             + proj(2 * F, H)                # gate, up
             + proj(H, F))                   # down
    lm_head = V * H * 2 if wl.tied else proj(V, H)
    weights = L * layer + H * 2 + lm_head    # + final norm gain
    kv = L * 2 * nkv * hd * 2 * (pos + 1)    # K and V rows of positions 0..pos, bf16
    return weights + 2 * H + kv + 4 * V      # + one embedding row, fp32 logits


@pytest.mark.parametrize("name", ["8b", "8b_int8", "8b_int4", "1b", "tiny"])
def test_step_bytes_match_the_tensor_definitions(name):
    wl = synth.get(name)
    m = amk.ModelConfig.from_workload(wl)
    for pos in (0, wl.prompt_len, wl.max_ctx - 1):
        assert bench.step_bytes(amk, m, pos) == expected_step_bytes(wl, pos), (name, pos)


def test_weight_bytes_per_token_of_the_quantised_workloads():
    """The per-token weight bytes of the ~8B shapes: 15.01 GB in bf16, 7.51 GB
    in int8 (0.50x) and 3.99 GB in int4 g128 (0.27x)."""
    got = {}
    for name in ("8b", "8b_int8", "8b_int4"):
        wl = synth.get(name)
        got[name] = expected_step_bytes(wl, -1) - 2 * wl.hidden - 4 * wl.vocab
    assert round(got["8b"] / 1e9, 2) == 15.01
    assert round(got["8b_int8"] / 1e9, 2) == 7.51
    assert round(got["8b_int4"] / 1e9, 2) == 3.99
