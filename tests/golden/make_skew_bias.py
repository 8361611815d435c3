"""Write c2_skew_bias.json: the router bias of the skewed verify workload.

The workload is a T=8 speculative-verify batch (launch post "Edge0-145B: Frontier
AI Capabilities on Your Own Computer", Under the Hood, Scheduling paragraph) with
skewed routing: 60 % of the 80 top-10 picks fall in 2 of the 8 groups.  The pages
give no mechanism, so the stated reading is a constant fp32 bias beta on every
expert of groups 0 and 1.  For each (seed, layer) this script bisects beta with the
oracle's router until exactly 48 of the 80 picks land in those groups, and stores
the float32 midpoint of the interval of betas that give 48 (so that the choice does
not sit on a boundary).

Calls only oracle/ and the input generator.  Run from the repository root:
    python tests/golden/make_skew_bias.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle.layer import route  # noqa: E402

TARGET = 48
SEEDS = (0, 1, 2)
LAYERS = (0, 1, 2, 3)


def count_in_hot(x, wr, beta, D):
    bias = np.zeros(D.n_experts, dtype=np.float32)
    bias[: 2 * D.experts_per_group] = np.float32(beta)
    idx = route(x, wr, bias, D.top_k)["idx"]
    return int(np.sum(idx < 2 * D.experts_per_group))


def first_reaching(x, wr, D, target, lo=0.0, hi=8.0, iters=40):
    """Smallest beta (to bisection precision) with count >= target."""
    assert count_in_hot(x, wr, hi, D) >= target
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if count_in_hot(x, wr, mid, D) >= target:
            hi = mid
        else:
            lo = mid
    return hi


def main():
    D = synth.config(2).dims
    entries = []
    for seed in SEEDS:
        x = synth.make_activations(2, seed)
        for layer in LAYERS:
            wr, _ = synth.make_router(2, seed, layer, with_skew=False)
            b48 = first_reaching(x, wr, D, TARGET)
            b49 = first_reaching(x, wr, D, TARGET + 1)
            beta = float(np.float32(0.5 * (b48 + b49)))
            c = count_in_hot(x, wr, beta, D)
            assert c == TARGET, (seed, layer, c)
            entries.append({"seed": seed, "layer": layer, "beta": beta,
                            "interval": [b48, b49], "picks_in_groups_0_1": c})
            print(seed, layer, beta, (b48, b49), flush=True)
    out = {"description": "fp32 router bias on experts 0..127 of the T=8 skewed verify "
                          "workload; 48 of 80 top-10 picks land in groups 0-1",
           "generator": "synth.make_activations(2, seed), synth.make_router(2, seed, layer)",
           "entries": entries}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c2_skew_bias.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
