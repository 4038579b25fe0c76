"""Batch-1 decode benchmark of the persistent megakernel on one MI355X.

One "step" is one decode step of the whole model (one cooperative launch):
token in, logits out, KV row written.  The workload is the ~8B Llama-shaped
bf16 decoder (32 layers, hidden 4096, 32/8 heads x 128, FFN 14336, vocab
128256) with a 1024-token prompt already in the KV cache and 256 decode
steps, on seeded random N(0, 0.02) weights (synthetic data; no checkpoint).

Reported: decode tokens/s (value), per-step latency, and the fraction of the
latency floor t_min(p) = B(p) / 8.0e12 B/s, where B(p) = every stored weight
byte (projections, scales, norms, LM head) + one embedding row + the KV
bytes of positions 0..p + the fp32 logits.  The `roofline` object gives the
achieved algorithmic GB/s of the single kernel (amk_vm) per launch, timed
with HIP events on the launch stream.  `cpu_baseline` times the oracle on a
bounded sample of the same workload on this host's cores.  Also on the line:
`stream_read` (a plain streaming read of the largest weight tensor on the
same device, the measured bandwidth ceiling), `launch_overhead_us` (the same
cooperative kernel launched with every queue empty), `counter_protocol` (the
same positions with the pages' counter protocol instead of the default
tagged activations) and, with --multistep, `multistep` (the same positions
as one greedy multi-step launch).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 8b]

Helpers for the committed profiles (see the command line in each summary):
  --no-launch-overhead    skip the empty-queue launches (under a profiler they
                          would be dispatches of the same kernel)
  --prompt-kv synthetic   fill the prompt's KV rows with seeded values instead
                          of running the prompt through the kernel (decode
                          time does not depend on KV values); used under the
                          counter profiler so that only the measured launches run
  --probe copy            copy a 1 GiB device buffer 5 times with torch's copy_
                          (the runtime's device-to-device copy kernel: the
                          known-size kernel that calibrates FETCH_SIZE and
                          WRITE_SIZE), then exit
  --traffic-from F W CF CW  read rocprofv3 counter CSVs (FETCH_SIZE and
                          WRITE_SIZE of a bench run, then of a copy probe run)
                          and write profiles/traffic_amk_vm_<workload>.json
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12  # bytes/s, MI355X published HBM3E bandwidth
PROFILES = os.path.join(ROOT, "profiles")
# sources of the decode kernel and its engine (the traffic summary is tied to them)
KERNEL_SRCS = [os.path.join(ROOT, "persistent_megakernel_wg_amd", "csrc", f)
               for f in ("vm.h", "vm_inst.hip", "vm.hip")]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def step_bytes(amk, model, pos):
    """Algorithmic bytes of the decode step at position pos (see module doc)."""
    H, V, L = model.hidden, model.vocab, model.n_layers
    n = amk.packed_count(model)
    weights = sum(amk.packed_bytes(model, k) for k in range(1, n))  # all but the embedding table
    emb_row = 2 * H
    kv = L * 2 * model.n_kv_heads * model.head_dim * 2 * (pos + 1)
    return weights + emb_row + kv + 4 * V


def kernel_hash():
    h = hashlib.sha256()
    for p in KERNEL_SRCS:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload, nsteps_bytes):
    """HBM traffic per launch from the committed rocprofv3 counter summary,
    or None when absent or taken on a different kernel source."""
    path = os.path.join(PROFILES, f"traffic_amk_vm_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_sha256_16") != kernel_hash():
        return None
    return t.get("bytes_per_launch")


COPY_BYTES = 1 << 30


def _counter_rows(path, counter):
    """(kernel name, value) per dispatch of one counter from a rocprofv3
    counter_collection CSV."""
    import csv
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") == counter:
                rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def traffic_from(workload, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv):
    """HBM bytes per launch of the megakernel from FETCH_SIZE / WRITE_SIZE
    (KiB per dispatch), each scaled by the ratio of known bytes to counted
    bytes of a plain device copy of COPY_BYTES (read COPY_BYTES, write
    COPY_BYTES)."""
    def med(rows, pat):
        v = [x for k, x in rows if pat in k]
        assert v, f"no dispatch of a kernel matching {pat!r}"
        return float(np.median(v)), len(v)
    copy_pat = "copyBuffer"  # the runtime's device-to-device copy kernel behind torch's copy_
    cf, ncf = med(_counter_rows(copy_fetch_csv, "FETCH_SIZE"), copy_pat)
    cw, ncw = med(_counter_rows(copy_write_csv, "WRITE_SIZE"), copy_pat)
    # decode-step dispatches only: an empty-queue launch of the same kernel
    # (the launch-overhead measurement) reads next to nothing
    def steps_only(rows):
        big = max(v for k, v in rows if "amk_vm" in k)
        return [(k, v) for k, v in rows if v >= 0.01 * big]
    kf, nkf = med(steps_only(_counter_rows(fetch_csv, "FETCH_SIZE")), "amk_vm")
    kw, nkw = med(steps_only(_counter_rows(write_csv, "WRITE_SIZE")), "amk_vm")
    fscale = COPY_BYTES / (cf * 1024.0)
    wscale = COPY_BYTES / (cw * 1024.0)
    out = {"workload": workload, "kernel_sha256_16": kernel_hash(),
           "fetch_kib_per_launch": kf, "write_kib_per_launch": kw,
           "copy_fetch_kib": cf, "copy_write_kib": cw, "copy_bytes": COPY_BYTES,
           "fetch_scale": fscale, "write_scale": wscale,
           "dispatches": {"kernel_fetch": nkf, "kernel_write": nkw, "copy_fetch": ncf, "copy_write": ncw},
           "bytes_per_launch": kf * 1024.0 * fscale + kw * 1024.0 * wscale}
    path = os.path.join(PROFILES, f"traffic_amk_vm_{workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    return out


def cpu_baseline(wl, weights, budget_s=20.0, max_steps=8):
    """Oracle decode steps at the prompt's context length on this host."""
    import oracle
    kvp = None
    m = oracle.Model(wl, weights)
    kv = m.new_kv()
    P = wl.prompt_len
    # the prompt's KV rows: synthetic (oracle cost does not depend on values)
    import synth
    if P > 0:
        kvp = synth.kv_prefix(wl, P, seed=3)
        kv[...] = kvp
    toks = synth.tokens(2, P + max_steps, wl.vocab)[P:]
    times = []
    t_start = time.time()
    for i, tok in enumerate(toks):
        t0 = time.time()
        m.step(kv, int(tok), P + i)
        times.append(time.time() - t0)
        if time.time() - t_start > budget_s:
            break
    m.close()
    per = float(np.mean(times))
    cpu = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": 1.0 / per, "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "cpu_model": cpu, "host_cpus": os.cpu_count(),
            "sample": f"{len(times)} decode steps at positions {P}..{P + len(times) - 1} of the "
                      f"{wl.name} workload (prompt KV rows filled with seeded values), "
                      f"{per * 1e3:.0f} ms/step, double-precision C++ oracle with OpenMP over output rows"}


def analyse_trace(view, stamps, khz):
    """Wait share and per-join latency of one traced launch.

    stamps[i] = (wait begin, wait end, work end, signal end) of task i."""
    us = 1e3 / khz
    st = stamps.astype(np.int64)
    t0 = st[:, 0].min()
    st = (st - t0) * us
    wait = st[:, 1] - st[:, 0]
    work = st[:, 2] - st[:, 1]
    sig = st[:, 3] - st[:, 2]
    tasks = view["tasks"]
    types = np.array([t["type"] for t in tasks])
    names = ["NOP", "QKV", "ATTN", "MERGE", "OPROJ", "GATEUP", "DOWN", "LMHEAD"]
    per_type = {}
    for ty in sorted(set(types.tolist())):
        m = types == ty
        per_type[names[ty]] = {"n": int(m.sum()), "wait_us": float(wait[m].mean()),
                               "work_us": float(work[m].mean()), "signal_us": float(sig[m].mean())}
    # join latency: last producer's signal end -> consumers' wait end
    prod = {}
    for i, t in enumerate(tasks):
        for c in t["sigs"]:
            prod.setdefault(c, []).append(i)
    lat_first, lat_med = [], []
    cons = {}
    for i, t in enumerate(tasks):
        for c, _ in t["waits"]:
            cons.setdefault(c, []).append(i)
    for c, ws in cons.items():
        last = max(st[p, 3] for p in prod[c])
        wake = np.array([st[w, 1] for w in ws])
        lat_first.append(wake.min() - last)
        lat_med.append(np.median(wake) - last)
    span = float(st[:, 3].max())
    return {"span_us": span, "wait_share": float(wait.sum() / (st[:, 3] - st[:, 0]).sum()),
            "join_latency_us": {"first_waiter_mean": float(np.mean(lat_first)),
                                "median_waiter_mean": float(np.mean(lat_med))},
            "per_type": per_type}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed decode steps (default: workload's)")
    ap.add_argument("--warmup", type=int, default=8, help="untimed decode steps after the prompt")
    ap.add_argument("--workload", default="8b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--depth", type=int, default=0, help="pipeline_depth override")
    ap.add_argument("--sched", default="", help="schedule overrides k=v,k=v")
    ap.add_argument("--trace", default="", help="after timing, trace 2 steps and write the analysis here")
    ap.add_argument("--prompt-kv", choices=("decode", "synthetic"), default="decode")
    ap.add_argument("--probe", choices=("", "copy"), default="")
    ap.add_argument("--no-counter-protocol", action="store_true",
                    help="skip timing the same positions with the counter protocol (sync_mode 0)")
    ap.add_argument("--no-launch-overhead", action="store_true",
                    help="skip the empty-queue launches (profiler runs: they are dispatches of the same kernel)")
    ap.add_argument("--multistep", action="store_true",
                    help="also time the same positions as one greedy multi-step launch")
    ap.add_argument("--traffic-from", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"))
    args = ap.parse_args()
    if args.traffic_from:
        print(json.dumps(traffic_from(args.workload, *args.traffic_from)))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the decode path is a "
              "single-GPU persistent kernel; multi-GPU sharding is a design note, not built.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.probe == "copy":
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"probe": "copy", "bytes": COPY_BYTES, "launches": 5}))
        return

    import persistent_megakernel_wg_amd as amk
    import synth

    wl = synth.get(args.workload)
    steps = args.steps if args.steps is not None else wl.decode_steps
    assert torch.cuda.is_available(), "bench needs a GPU"
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    model = amk.ModelConfig.from_workload(wl)
    cfg = amk.default_schedule_config(model, cus)
    if args.depth:
        cfg.pipeline_depth = args.depth
    for kv_ in filter(None, args.sched.split(",")):
        k, v = kv_.split("=")
        setattr(cfg, k, int(v))
    sched = amk.Schedule.build(model, cfg)
    verdict = sched.validate()
    assert verdict[0] == 0, verdict

    t0 = time.time()
    weights = synth.model_weights(wl, seed=1)
    log(f"generated {wl.name} weights in {time.time() - t0:.1f}s")
    t0 = time.time()
    dev_w = amk.upload_model(model, weights, device=dev)
    log(f"packed + uploaded in {time.time() - t0:.1f}s "
        f"({sum(w.numel() for w in dev_w) / 1e9:.2f} GB on device)")
    kv, logits = amk.alloc_state(model, device=dev)
    eng = amk.Engine(sched, dev_w, kv, logits)
    toks = synth.tokens(2, wl.prompt_len + steps + args.warmup, wl.vocab)
    stream = torch.cuda.current_stream()

    # prompt: teacher-forced decode steps (untimed), or seeded KV rows
    t0 = time.time()
    if args.prompt_kv == "synthetic":
        kvp = synth.kv_prefix(wl, wl.prompt_len, seed=3)
        kv.copy_(torch.from_numpy(kvp.view(np.int16).reshape(-1)).to(dev))
        del kvp
        eng.set_kv_length(wl.prompt_len)
    else:
        for p in range(wl.prompt_len):
            eng.decode_step(int(toks[p]), p, stream)
    torch.cuda.synchronize()
    eng.check()
    log(f"prompt of {wl.prompt_len} positions ({args.prompt_kv}) in {time.time() - t0:.2f}s")
    P = wl.prompt_len
    # warmup steps, then rewind so that the timed steps see the workload's positions
    for i in range(args.warmup):
        eng.decode_step(int(toks[P + i]), P + i, stream)
    torch.cuda.synchronize()
    eng.check()

    # HIP events on the launch stream right before and after every launch:
    # their difference is the kernel's duration (the roofline's denominator)
    ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    dec = toks[P + args.warmup:]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(steps):
        ev0[i].record(stream)
        eng.decode_step(int(dec[i]), P + i, stream)
        ev1[i].record(stream)
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    eng.check()
    lat = np.array([ev0[i].elapsed_time(ev1[i]) * 1e-3 for i in range(steps)])  # seconds
    gpu_total = float(lat.sum())
    B = np.array([step_bytes(amk, model, P + i) for i in range(steps)], dtype=np.float64)
    tmin = B / HBM_PEAK
    floor_frac = float(tmin.sum() / (t_total))
    achieved = float(B.mean() / lat.mean())
    traffic = load_traffic(wl.name, B.mean())
    out = {
        "metric": "batch-1 decode tokens/s and % of weight+KV bytes / HBM-BW latency floor",
        "value": steps / t_total,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": t_total / steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.wfmt if wl.wfmt != "bf16" else "bf16",
        "data": "synthetic (seeded N(0,0.02) bf16 weights, seeded uniform tokens)",
        "config": {"workload": f"{wl.name}: {wl.n_layers} layers, hidden {wl.hidden}, "
                               f"{wl.n_heads}/{wl.n_kv_heads} heads x {wl.head_dim}, FFN {wl.ffn}, "
                               f"vocab {wl.vocab}, {wl.wfmt} weights, batch 1, "
                               f"{wl.prompt_len}-token prompt, decode positions {P}..{P + steps - 1}",
                   "batch": 1, "prompt_len": P, "decode_steps": steps,
                   "schedule": cfg.as_dict()},
        "floor_fraction": floor_frac,
        "floor_fraction_kernel": float(tmin.sum() / gpu_total),
        "t_min_ms_mean": float(tmin.mean() * 1e3),
        "kernel_ms": {"mean": float(lat.mean() * 1e3), "median": float(np.median(lat) * 1e3),
                       "p90": float(np.percentile(lat, 90) * 1e3), "min": float(lat.min() * 1e3)},
        "bytes_per_step_mean": float(B.mean()),
        "roofline": {"bound": "hbm", "achieved": achieved / 1e9, "peak": HBM_PEAK / 1e9,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK,
                     "traffic": traffic},
        "cpu_baseline": None,
    }
    # the fraction of the device's streaming-read ceiling: the largest weight
    # tensor read in the pattern that reaches the highest rate here
    # (amk_stream_read_probe: contiguous share per workgroup, 16
    # non-temporal 16-byte loads per lane in flight), best of three grids
    big = max(dev_w, key=lambda x: x.numel() * x.element_size())
    probe_out = torch.zeros(65536, device=dev)
    rates = []
    for blocks in (256, 512, 1024):
        amk.stream_read_probe(big, probe_out, blocks)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(5):
            amk.stream_read_probe(big, probe_out, blocks, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        rates.append(big.numel() * big.element_size() * 5 / (e0.elapsed_time(e1) * 1e-3))
    out["stream_read"] = {"GBps": max(rates) / 1e9, "bytes": int(big.numel() * big.element_size()),
                          "kernel_frac": achieved / max(rates)}
    # the cooperative-launch overhead of a step: the same kernel, grid, LDS
    # and parameters with every queue empty (amk_engine_launch_empty),
    # back to back on the launch stream
    if not args.no_launch_overhead:
        for _ in range(4):
            eng.launch_empty(stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(64):
            eng.launch_empty(stream)
        e1.record(stream)
        torch.cuda.synchronize()
        eng.check()
        out["launch_overhead_us"] = e0.elapsed_time(e1) * 1e3 / 64
    if not args.no_counter_protocol and cfg.sync_mode != 0:
        # the same positions with the pages' counter protocol (sync_mode 0):
        # same DAG, every edge a monotonic counter (wait -> dispatch ->
        # signal) instead of a tagged activation word
        c0 = amk.ScheduleConfig.from_buffer_copy(cfg)
        c0.sync_mode = 0
        s0 = amk.Schedule.build(model, c0)
        assert s0.validate()[0] == 0
        kv0, lg0 = amk.alloc_state(model, device=dev)
        kv0.copy_(kv)
        e_c = amk.Engine(s0, dev_w, kv0, lg0)
        e_c.set_kv_length(P)
        for i in range(args.warmup):
            e_c.decode_step(int(toks[P + i]), P + i, stream)
        torch.cuda.synchronize()
        e_c.check()
        m0, m1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        m0.record(stream)
        for i in range(steps):
            e_c.decode_step(int(dec[i]), P + i, stream)
        m1.record(stream)
        torch.cuda.synchronize()
        e_c.check()
        ms = m0.elapsed_time(m1) / steps
        out["counter_protocol"] = {"sync_mode": 0, "ms_per_step": ms, "tokens_per_s": 1e3 / ms,
                                   "floor_fraction": float(tmin.mean() / (ms * 1e-3))}
        log(f"counter protocol (sync_mode 0): {ms:.4f} ms/step")
        e_c.close()
        s0.close()
        del e_c, kv0, lg0
    if args.multistep:
        # the same positions decoded greedily in ONE launch (amk_decode_steps):
        # the token of every step is fed back on the device
        out_tok = torch.zeros(steps, dtype=torch.int32, device=dev)
        eng.decode_steps(int(dec[0]), P, steps, out_tok, stream)  # warm-up launch
        torch.cuda.synchronize()
        eng.check()
        m0, m1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        m0.record(stream)
        eng.decode_steps(int(dec[0]), P, steps, out_tok, stream)
        m1.record(stream)
        torch.cuda.synchronize()
        eng.check()
        ms = m0.elapsed_time(m1)
        out["multistep"] = {"launches": 1, "steps": steps, "ms_per_step": ms / steps,
                            "tokens_per_s": steps / (ms * 1e-3),
                            "floor_fraction": float(tmin.sum() / (ms * 1e-3))}
        log(f"multistep: {steps} greedy steps in one launch, {ms / steps:.4f} ms/step")
    if args.trace:
        eng.set_trace(True)
        for i in range(2):
            eng.decode_step(int(dec[i]), P + i, stream)
        torch.cuda.synchronize()
        eng.check()
        eng.set_trace(False)
        view = sched.view()
        stamps, khz = eng.read_trace(len(view["tasks"]))
        tr = analyse_trace(view, stamps, khz)
        tr["regions"] = eng.region_stats()  # per task type, from the library (amk_engine_region_stats)
        with open(args.trace, "w") as f:
            json.dump(tr, f, indent=1)
        out["trace"] = {k: tr[k] for k in ("span_us", "wait_share", "join_latency_us")}
        out["trace"]["critical_path_us"] = {k: round(v["span_us"], 1) for k, v in tr["regions"].items()}
        log(f"trace: {json.dumps(tr)}")
    # release every HIP resource before the process ends: the engine, the
    # schedule and the device tensors are freed here, in order, not by
    # finalizers at interpreter exit (a profiler may have detached by then)
    eng.close()
    sched.close()
    del eng, dev_w, kv, logits, probe_out, big
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        t0 = time.time()
        out["cpu_baseline"] = cpu_baseline(wl, weights, budget_s=args.cpu_budget)
        log(f"cpu baseline in {time.time() - t0:.1f}s")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
