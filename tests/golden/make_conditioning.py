"""Write tests/golden/conditioning.json: per-(b, n) sensitivity of the exact
float64 dynamics of each full-size workload.

For every unit, oracle.tangent_growth pushes a tangent through the
linearisation of Eq. (10)-(11) of the M²RNN review along the float64
trajectory and returns the largest finite-time amplification of a
perturbation.  Units with small amplification are reproducible in fp32 over
the whole sequence; units with large amplification are not (no fp32
evaluation, on any hardware, stays within a fixed absolute tolerance of the
float64 trajectory there).  Calls only oracle/ and the input generator.

Usage: python tests/golden/make_conditioning.py [workload ...]
"""
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from m2rnn_inputs import WORKLOAD_ORDER, WORKLOADS, make_inputs  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "conditioning.json")


def main(names):
    data = json.load(open(OUT)) if os.path.exists(OUT) else {}
    for name in names:
        wl = WORKLOADS[name]
        t0 = time.time()
        inp = make_inputs(wl, with_dy=False)
        f = oracle.gates(wl.gate, inp.logit, inp.alpha, inp.beta)
        # shared q/k (the review's section 2.4 layout): value head n reads q/k
        # head n // (N / NQ); the tangent pass takes one q/k row per value head
        rep = wl.N // wl.qk_heads
        k = np.repeat(inp.k, rep, axis=2)
        q = np.repeat(inp.q, rep, axis=2)
        G = oracle.tangent_growth(k, inp.v, q, f, inp.W)
        data[name] = {"B": wl.B, "N": wl.N, "T": wl.T, "seed": wl.seed,
                      "growth": [[float(x) for x in row] for row in G]}
        print(f"{name}: growth quantiles {np.quantile(G, [0, 0.25, 0.5, 0.75, 1])} "
              f"({time.time() - t0:.0f} s)", flush=True)
        json.dump(data, open(OUT, "w"), indent=1)


if __name__ == "__main__":
    main(sys.argv[1:] or WORKLOAD_ORDER + ["multi_value_k64_v16"])
