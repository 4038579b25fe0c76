"""Deterministic schedule tuner: the AutoMegaKernel summary's autoresearch
loop ("Methodology", the autonomous research loop: propose a ScheduleConfig
change, check it against a reference, measure latency, keep or revert)
without the agent.  Candidates are proposed by coordinate descent over the
knobs of ScheduleConfig in a fixed order; every candidate must

  1. lower and pass the static safety gate (amk_validate; the engine refuses
     unsafe schedules anyway),
  2. reproduce, on a few decode steps after the workload's seeded prompt
     KV rows, the logits of a CPU reference (the oracle's logits for the
     same seeded inputs, handed in by the caller: tune(reference=...) or
     --reference FILE, written by oracle/reference.py) within the parity
     bar, and the logits of the library-default schedule on the GPU,
  3. be faster than the best so far by more than `min_gain` (median
     kernel time over `steps` timed decode steps).

Without a CPU reference only the GPU-default check applies, and the result
says so ("cpu_reference": false).  The parity bar is the workload's: 1e-2
relative L2 and 2e-2 max-abs, or 4e-2 for both on models with bf16
projection inputs (their measured conditioning).

After the knobs, the per-phase XCD weights are fitted from traced steps
(tasks of an XCD that ends late get proportionally fewer rows) and kept
under the same three conditions.

Usage (one GPU):  python -m persistent_megakernel_wg_amd.tune --workload 8b --out best.json
"""
import argparse
import json
import sys
import time

import numpy as np

# knob -> candidate values, tried in this order
SPACE = [
    ("attn_splits", [8, 16, 24, 32, 48]),
    ("pipeline_depth", [4, 8, 16]),
    ("prefetch_kb", [-1, 64, 96, 128, 160]),
    ("poll_mode", [0, 1]),
    ("cu_policy", [0, 1]),
    ("release_mode", [0, 1]),
    ("sync_mode", [0, 1, 2]),
    ("merge_place", [0, 1]),
    ("prefetch_attn_kb", [-1, 64, 128]),
]

REL_L2 = 1e-2
MAX_ABS = 2e-2
ACT_BF16_TOL = 4e-2


def bar(wl):
    """(relative L2, max-abs ratio) bar of the workload's check steps."""
    return (ACT_BF16_TOL, ACT_BF16_TOL) if wl.act_bf16 else (REL_L2, MAX_ABS)


def check_tokens(wl, warmup=8, steps=48, check_steps=3):
    """(prompt length, tokens of the check steps): the check steps decode at
    positions P .. P + check_steps - 1 after P seeded KV rows (seed 3), with
    the seeded tokens (seed 2) that follow the prompt."""
    import synth
    P = wl.prompt_len
    return P, synth.tokens(2, P + warmup + steps + check_steps, wl.vocab)[P:P + check_steps]


def log(msg):
    print(f"[tune] {msg}", file=sys.stderr, flush=True)


def apply(cfg, overrides):
    for k, v in overrides.items():
        if isinstance(v, list):
            arr = getattr(cfg, k)
            for i, x in enumerate(v):
                if isinstance(x, list):
                    for j, y in enumerate(x):
                        arr[i][j] = y
                else:
                    arr[i] = x
        else:
            setattr(cfg, k, v)
    return cfg


class Bench:
    """Runs candidate schedules of one workload on shared device buffers."""

    def __init__(self, wl, steps=32, warmup=8, check_steps=3):
        import torch

        import persistent_megakernel_wg_amd as amk
        import synth
        self.torch, self.amk = torch, amk
        self.wl = wl
        self.model = amk.ModelConfig.from_workload(wl)
        self.cus = torch.cuda.get_device_properties(0).multi_processor_count
        w = synth.model_weights(wl, seed=1)
        self.dev_w = amk.upload_model(self.model, w)
        del w
        self.kv, self.logits = amk.alloc_state(self.model)
        P = wl.prompt_len
        self.P = P
        self.kvp = torch.from_numpy(synth.kv_prefix(wl, P, seed=3).view(np.int16).reshape(-1)).to(self.kv.device)
        self.toks = synth.tokens(2, P + warmup + steps + check_steps, wl.vocab)[P:]
        self.steps, self.warmup, self.check_steps = steps, warmup, check_steps
        self.reference = None

    def config(self, overrides):
        return apply(self.amk.default_schedule_config(self.model, self.cus), overrides)

    def run(self, overrides):
        """(median kernel ms, logits of the check steps) or raises."""
        torch, amk = self.torch, self.amk
        sched = amk.Schedule.build(self.model, self.config(overrides))
        code = sched.validate()
        if code[0] != 0:
            raise RuntimeError(f"rejected by the safety gate: {code}")
        eng = amk.Engine(sched, self.dev_w, self.kv, self.logits)
        s = torch.cuda.current_stream()
        try:
            self.kv.copy_(self.kvp)
            eng.set_kv_length(self.P)
            out = []
            for i in range(self.check_steps):
                eng.decode_step(int(self.toks[i]), self.P + i, s)
                torch.cuda.synchronize()
                eng.check()
                out.append(self.logits.cpu().numpy().astype(np.float64))
            for i in range(self.warmup):
                eng.decode_step(int(self.toks[i]), self.P + i, s)
            e0 = [torch.cuda.Event(enable_timing=True) for _ in range(self.steps)]
            e1 = [torch.cuda.Event(enable_timing=True) for _ in range(self.steps)]
            for i in range(self.steps):
                e0[i].record(s)
                eng.decode_step(int(self.toks[i]), self.P + i, s)
                e1[i].record(s)
            torch.cuda.synchronize()
            eng.check()
            ms = float(np.median([e0[i].elapsed_time(e1[i]) for i in range(self.steps)]))
        finally:
            eng.close()
            sched.close()
        return ms, out

    def xcd_imbalance(self, overrides, nsteps=4):
        """Per GEMV phase and XCD, from traced decode steps: the mean offset
        of a task's end from the median end of its phase, and its mean
        duration from input staged to end (microseconds).  [5][8] each."""
        torch, amk = self.torch, self.amk
        sched = amk.Schedule.build(self.model, self.config(overrides))
        eng = amk.Engine(sched, self.dev_w, self.kv, self.logits)
        s = torch.cuda.current_stream()
        tasks = sched.view()["tasks"]
        ty = np.array([t["type"] for t in tasks])
        cu = np.array([t["cu"] for t in tasks])
        layer = np.array([t["p"][0] if t["type"] != 7 else -1 for t in tasks])
        off = np.zeros((5, 8))
        dur = np.zeros((5, 8))
        cnt = np.zeros((5, 8))
        try:
            self.kv.copy_(self.kvp)
            eng.set_kv_length(self.P)
            for i in range(2):
                eng.decode_step(int(self.toks[i]), self.P + i, s)
            eng.set_trace(True)
            for i in range(nsteps):
                eng.decode_step(int(self.toks[i]), self.P + i, s)
                torch.cuda.synchronize()
                eng.check()
                st, khz = eng.read_trace(len(tasks))
                st = st.astype(np.float64) * (1e3 / khz)
                for ph, tt in enumerate((1, 4, 5, 6, 7)):
                    layers = [-1] if tt == 7 else range(1, self.model.n_layers - 1)
                    for l in layers:
                        m = (ty == tt) & (layer == l)
                        if not m.any():
                            continue
                        end = st[m, 3]
                        x = cu[m] % 8
                        np.add.at(off[ph], x, end - np.median(end))
                        np.add.at(dur[ph], x, st[m, 3] - st[m, 1])
                        np.add.at(cnt[ph], x, 1)
        finally:
            eng.set_trace(False)
            eng.close()
            sched.close()
        cnt = np.maximum(cnt, 1)
        return off / cnt, dur / cnt

    def agrees(self, out, ref=None):
        """(within the bar on every check step, worst relative L2) against
        `ref` (default: the library-default schedule's logits)."""
        rl, ml = bar(self.wl)
        worst = 0.0
        ok = True
        for g, o in zip(out, self.reference if ref is None else ref):
            rel = float(np.linalg.norm(g - o) / np.linalg.norm(o))
            mab = float(np.max(np.abs(g - o)) / np.max(np.abs(o)))
            worst = max(worst, rel)
            ok = ok and rel <= rl and mab <= ml
        return ok, worst


def tune(wl, min_gain=0.005, steps=48, space=SPACE, xcd_rounds=2, reference=None):
    """reference: the CPU reference logits of the check steps (a sequence of
    `check_steps` fp64 arrays of the vocabulary size, see check_tokens) or
    None."""
    b = Bench(wl, steps=steps)
    if reference is not None:
        reference = [np.asarray(r, dtype=np.float64) for r in reference]
        assert len(reference) == b.check_steps and all(r.shape == (wl.vocab,) for r in reference)
    default = b.config({})
    best = {}
    best_ms, b.reference = b.run(best)
    log(f"reference (library default) {best_ms:.4f} ms")
    entry = {"overrides": {}, "ms": best_ms, "kept": True}
    if reference is not None:
        ok, rel = b.agrees(b.reference, reference)
        entry.update(cpu_ok=ok, cpu_rel_l2=rel)
        log(f"library default vs the CPU reference: worst relL2 {rel:.2e} {'ok' if ok else 'FAIL'}")
        if not ok:
            raise RuntimeError(f"the library-default schedule misses the CPU reference (relL2 {rel:.2e})")
    history = [entry]

    def judge(cand, ms, out):
        """history entry of a measured candidate and whether it is kept"""
        ok, rel = b.agrees(out)
        e = {"overrides": cand, "ms": ms, "parity": ok, "gpu_rel_l2": rel}
        if reference is not None:
            cok, crel = b.agrees(out, reference)
            e.update(cpu_ok=cok, cpu_rel_l2=crel)
            ok = ok and cok
        e["kept"] = ok and ms < best_ms * (1 - min_gain)
        return e
    for knob, values in space:
        for v in values:
            cand = dict(best)
            cand[knob] = v
            current = best.get(knob, getattr(default, knob))
            if v == current:
                continue
            try:
                ms, out = b.run(cand)
            except Exception as e:  # unsafe or unsupported: reverted
                history.append({"overrides": cand, "error": str(e), "kept": False})
                log(f"{cand}: {e}")
                continue
            e = judge(cand, ms, out)
            history.append(e)
            log(f"{cand}: {ms:.4f} ms gpu relL2 {e['gpu_rel_l2']:.2e}"
                f"{' cpu relL2 %.2e' % e['cpu_rel_l2'] if 'cpu_rel_l2' in e else ''}{' KEEP' if e['kept'] else ''}")
            if e["kept"]:
                best, best_ms = cand, ms
    # per-phase XCD weights: shorten the tasks of XCDs that end late and
    # lengthen those that end early, in proportion to their durations
    for rnd in range(xcd_rounds):
        off, dur = b.xcd_imbalance(best)
        cur = np.array([list(r) for r in b.config(best).xcd_weight], dtype=np.float64)
        new = cur * np.clip((dur - (off - off.mean(axis=1, keepdims=True))) / np.maximum(dur, 1e-3), 0.7, 1.3)
        new = np.clip(np.round(new / new.mean(axis=1, keepdims=True) * 1000), 100, 10000).astype(int)
        cand = dict(best)
        cand["xcd_weight"] = new.tolist()
        log(f"xcd end offsets (us) per phase: {np.round(off, 2).tolist()}")
        try:
            ms, out = b.run(cand)
        except Exception as e:
            history.append({"overrides": cand, "error": str(e), "kept": False})
            break
        e = judge(cand, ms, out)
        history.append(e)
        log(f"xcd weights round {rnd}: {ms:.4f} ms{' KEEP' if e['kept'] else ''}")
        if not e["kept"]:
            break
        best, best_ms = cand, ms
    # re-measure the winner against the reference, interleaved
    ref, win = [], []
    for _ in range(2):
        ref.append(b.run({})[0])
        win.append(b.run(best)[0])
    return {"workload": wl.name, "best": best, "ms": float(np.median(win)), "reference_ms": float(np.median(ref)),
            "cpu_reference": reference is not None, "history": history}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="8b")
    ap.add_argument("--out", default="")
    ap.add_argument("--steps", type=int, default=48)
    ap.add_argument("--min-gain", type=float, default=0.005)
    ap.add_argument("--reference", default="",
                    help="npz with 'logits' [check steps][vocab]: the CPU reference of the check steps")
    args = ap.parse_args()
    import synth
    ref = None
    if args.reference:
        with np.load(args.reference, allow_pickle=False) as z:
            ref = list(z["logits"])
    t0 = time.time()
    res = tune(synth.get(args.workload), args.min_gain, args.steps, reference=ref)
    res["seconds"] = time.time() - t0
    text = json.dumps(res, indent=1)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    print(json.dumps({k: res[k] for k in ("workload", "best", "ms", "reference_ms", "seconds")}))


if __name__ == "__main__":
    main()
