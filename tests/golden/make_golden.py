"""Writes tests/golden/tiny_workload.json from the float64 oracle only.

The tiny workload is T=4, H=256, E=8, k=2, I=512 with the seeded generators
of moe_inputs.  The fixture freezes the oracle's routing, tile table (BM=16)
and a fixed sample of outputs so that any later change to the oracle's
arithmetic shows up as a diff.  Run: python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from moe_inputs import make_workload  # noqa: E402

SAMPLE = [(0, 0), (0, 255), (1, 17), (2, 128), (3, 3), (3, 200)]


def main():
    inp = make_workload(0)
    res = oracle.moe_layer(inp, BM=16)
    doc = {
        "what": "oracle output for the tiny MoE workload (T=4,H=256,E=8,k=2,I=512), BM=16",
        "written_by": "tests/golden/make_golden.py (calls only oracle/ and moe_inputs)",
        "topk_ids": res["topk_ids"].tolist(),
        "topk_weights": [[float(v) for v in r] for r in res["topk_weights"]],
        "expert_offsets": res["expert_offsets"].tolist(),
        "sorted_ids": res["sorted_ids"].tolist(),
        "tiles": res["tiles"].tolist(),
        "num_tiles": res["num_tiles"],
        "out_samples": [[t, h, float(res["out"][t, h])] for t, h in SAMPLE],
        "out_l2": float(np.linalg.norm(res["out"])),
    }
    with open(os.path.join(HERE, "tiny_workload.json"), "w") as f:
        json.dump(doc, f, indent=1)


if __name__ == "__main__":
    main()
