"""CPU reference logits for the schedule tuner's check steps (test
infrastructure: the oracle's logits written to a file the tuner reads with
--reference; the tuner never runs the oracle itself).

The check steps follow the tuner's protocol: P = the workload's prompt
length seeded KV rows (seed 3), then decode steps at positions P, P + 1, ...
taking the seeded tokens (seed 2) that follow the prompt; weights seed 1.

Usage: python -m oracle.reference --workload 8b --steps 3 --out ref_8b.npz
"""
import argparse
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def check_step_logits(wl, weights, steps=3):
    """Oracle logits (fp64) of the first `steps` check steps of workload wl."""
    import oracle
    import synth
    P = wl.prompt_len
    toks = synth.tokens(2, P + steps, wl.vocab)[P:]
    m = oracle.Model(wl, weights)
    kv = m.new_kv()
    if P:
        kv[...] = synth.kv_prefix(wl, P, seed=3)
    out = [m.step(kv, int(t), P + i).copy() for i, t in enumerate(toks)]
    m.close()
    return out


def main():
    import synth
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="8b")
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--out", required=True)
    a = ap.parse_args()
    wl = synth.get(a.workload)
    ref = check_step_logits(wl, synth.model_weights(wl, seed=1), a.steps)
    np.savez(a.out, logits=np.stack(ref), workload=wl.name)
    print(f"wrote {a.out}: {len(ref)} check steps of {wl.name}")


if __name__ == "__main__":
    main()
