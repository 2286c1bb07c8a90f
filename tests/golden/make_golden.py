"""Write tests/golden/tiny_oracle.json from the oracle alone.

The pages print no worked example for this layer, so this fixture is a
regression record of the oracle's own output on the tiny seeded workload
(hidden 256, 16 experts top-2 + shared, FFN 128, 4 tokens, seed 0).  Run:
    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import moe_synth as ms  # noqa: E402
import oracle  # noqa: E402


def main():
    cfg = ms.CONFIGS["tiny"]
    r = oracle.forward(cfg, ms.make_inputs(cfg))
    g = {
        "workload": "tiny: H=256 E=16 k=2 F=128 T=4 seed 0, learned router with bias, Q8 experts + Q8 shared",
        "ids": r["ids"].tolist(),
        "w": [[float(v) for v in row] for row in r["w"]],
        "out_head": r["out"][:, :8].tolist(),
        "out_sum": float(np.sum(r["out"].astype(np.float64))),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.json")
    with open(path, "w") as f:
        json.dump(g, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
