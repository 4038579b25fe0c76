"""bench.py host logic (no GPU): the refusal of more than one GPU, and the
algorithmic bytes of a decode step behind the floor fraction and the
roofline, checked against the byte count of each stored tensor written out
from the model shapes and the weight formats' definitions (bf16: 2 bytes a
weight; int8: a byte a weight plus a 4-byte scale per output row; int4 g128:
half a byte a weight plus a 2-byte scale and a 2-byte zero per group of 128
inputs; a tied LM head reads the bf16 embedding table); and the HBM traffic
per launch computed from rocprofv3 counter tables (synthetic ones here)."""
import json
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


def _counter_csv(path, rows):
    with open(path, "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for i, (kernel, counter, value) in enumerate(rows):
            f.write(f'{i},"{kernel}",{counter},{value}\n')


def test_traffic_from_counters(tmp_path, monkeypatch):
    """HBM bytes per launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch):
    the median over the decode kernel's dispatches, the near-empty
    empty-queue launches left out, each counter scaled by the known bytes of
    a device copy over what the same counter reads for it; a stored summary
    is used only while the kernel source is the one it was taken on."""
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    k = "void amk::amk_vm<8, 0, false>(amk::VmParams)"
    copy = "__amd_rocclr_copyBuffer"
    kib = bench.COPY_BYTES / 1024.0
    _counter_csv(tmp_path / "f.csv", [(k, "FETCH_SIZE", 1000.0), (k, "FETCH_SIZE", 1010.0), (k, "FETCH_SIZE", 990.0),
                                      (k, "FETCH_SIZE", 5.0), ("other_kernel", "FETCH_SIZE", 1e6)])
    _counter_csv(tmp_path / "w.csv", [(k, "WRITE_SIZE", 100.0), (k, "WRITE_SIZE", 101.0), (k, "WRITE_SIZE", 100.0),
                                      (k, "WRITE_SIZE", 0.1)])
    _counter_csv(tmp_path / "cf.csv", [(copy, "FETCH_SIZE", kib * 1.05)] * 5)
    _counter_csv(tmp_path / "cw.csv", [(copy, "WRITE_SIZE", kib * 0.98)] * 5)
    out = bench.traffic_from("unit", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                             str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv"))
    want = 1000.0 * 1024 / 1.05 + 100.0 * 1024 / 0.98
    assert out["dispatches"]["kernel_fetch"] == 3 and out["dispatches"]["kernel_write"] == 3
    assert out["bytes_per_launch"] == pytest.approx(want, rel=1e-12)
    assert bench.load_traffic("unit", 0) == pytest.approx(want, rel=1e-12)
    stale = json.loads((tmp_path / "traffic_amk_vm_unit.json").read_text())
    stale["kernel_sha256_16"] = "0" * 16
    (tmp_path / "traffic_amk_vm_unit.json").write_text(json.dumps(stale))
    assert bench.load_traffic("unit", 0) is None
    assert bench.load_traffic("absent", 0) is None
