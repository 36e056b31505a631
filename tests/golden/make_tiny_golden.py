"""Write tiny_oracle.json from the seeded generator and the oracle only."""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import adafuse as O  # noqa: E402
from weight_merge_amd import synth  # noqa: E402
from weight_merge_amd.configs import TINY  # noqa: E402

SEED = 0
ROWS = [0, 1, 17, 63, 64, 128, 200, 255]
COLS = [0, 3, 8, 64, 127, 128, 254, 255]


def build():
    h, R = synth.router_inputs(TINY, SEED)
    st = synth.make_stack(TINY, SEED)
    idx, g = O.pregate(h.double().numpy(), R.double().numpy(), TINY.k, TINY.renorm)
    layers = []
    for l, p, _ in st.items():
        W = st.W[l][p].double().numpy()
        merged = O.merge(W, st.A[l][p].double().numpy(), st.B[l][p].double().numpy(), idx, g, TINY.scale)
        layers.append({"layer": l, "proj": p,
                       "samples": [[r, c, float(merged[r, c])] for r in ROWS for c in COLS],
                       "sum": float(merged.sum()), "abs_sum": float(np.abs(merged).sum())})
    return {"config": TINY.name, "seed": SEED, "idx": idx.tolist(), "gate": [float(v) for v in g],
            "logits": [float(v) for v in O.router_logits(h.double().numpy(), R.double().numpy())],
            "layers": layers}


if __name__ == "__main__":
    with open(os.path.join(HERE, "tiny_oracle.json"), "w") as f:
        json.dump(build(), f, indent=1)
    print("wrote tiny_oracle.json")
