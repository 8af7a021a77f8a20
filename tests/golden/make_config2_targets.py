"""Write config2_targets.txt: the 4096 target ids of the Qwen3-8B-shaped forward workload.

Each row's target is drawn from softmax(z) of the oracle's fp64 logits z = h W^T / 0.7 over
the real vocabulary (151669 ids), by inverse CDF in ascending-id order with the row's seeded
U(0,1). Calls only the oracle and the seeded input generators. Takes about a minute and
~8 GB of memory.

    python tests/golden/make_config2_targets.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth   # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "config2_targets.txt")


def main():
    base = synth.config2_base()
    Vr, tau = base["real_vocab"], base["temperature"]
    h = oracle.bf16_to_f64(base["hidden"])
    w = oracle.bf16_to_f64(synth.full_weight()[:Vr])
    u = synth.config2_uniforms()
    targets = np.empty(base["T"], dtype=np.int64)
    for r0 in range(0, base["T"], 256):
        z = oracle.logits(h[r0:r0 + 256], w, None, tau)
        lse, _ = oracle.softmax_stats(z)
        p = np.exp(z - lse[:, None])
        for i in range(z.shape[0]):
            targets[r0 + i] = synth.inverse_cdf(p[i], u[r0 + i])
        print(f"rows {r0}..{r0 + z.shape[0] - 1} done", flush=True)
    with open(OUT, "w") as f:
        f.write("# config-2 targets (T=4096): ids sampled from the fp64 oracle softmax, tau=0.7,\n")
        f.write("# real vocab 151669; written by tests/golden/make_config2_targets.py\n")
        for t in targets:
            f.write(f"{int(t)}\n")


if __name__ == "__main__":
    main()
