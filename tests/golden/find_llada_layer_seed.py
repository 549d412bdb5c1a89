"""Find the first seed of the LLaDA-8B-shaped single-layer workload whose oracle scores keep every
token more than 1e-4 away from the top-128 boundary (the midpoint of the 128th and 129th scores),
and write it to llada_layer_seed.json. Calls only the oracle and the seeded generators.

    python tests/golden/find_llada_layer_seed.py [start_seed]
"""
import json
import os
import sys
import time

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle as O  # noqa: E402
from synth import workloads as W  # noqa: E402


def margin_of(seed: int):
    dims = W.LLADA_LAYER
    h_prev, h_cur, large, lg, _ = W.layer_inputs(dims, W.LLADA_LARGE, seed)
    dec = lambda t: O.decode_bf16(t.view(torch.uint16).numpy())  # noqa: E731
    score, _, _ = O.saliency(dec(h_cur[0]), dec(h_prev[0]), dec(lg[0]), 0.5, O.DELTA_L1N)
    s = np.sort(score.astype(np.float64))[::-1]
    k = W.LLADA_TOPK
    thr = 0.5 * (s[k - 1] + s[k])
    return float(np.min(np.abs(score.astype(np.float64) - thr))), float(thr)


def main():
    seed = int(sys.argv[1]) if len(sys.argv) > 1 else 20261203
    while True:
        t = time.time()
        m, thr = margin_of(seed)
        print(f"seed {seed}: margin {m:.3e} threshold {thr:.6f} ({time.time() - t:.1f}s)")
        if m > 1e-4:
            break
        seed += 1
    out = {"workload": "llada_layer", "seed": seed, "topk": W.LLADA_TOPK, "margin": m,
           "threshold_midpoint": thr,
           "rule": "every oracle score is more than 1e-4 from the midpoint of the 128th and "
                   "129th largest scores",
           "script": "tests/golden/find_llada_layer_seed.py (oracle + synth only)"}
    with open(os.path.join(HERE, "llada_layer_seed.json"), "w") as f:
        json.dump(out, f, indent=2)
    print(out)


if __name__ == "__main__":
    main()
