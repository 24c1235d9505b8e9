"""The oracle still reproduces its frozen tiny-workload fixture (CPU only)."""
import json
import os

import numpy as np

import oracle
from moe_inputs import make_workload

GOLD = os.path.join(os.path.dirname(__file__), "golden", "tiny_workload.json")


def test_tiny_workload_fixture():
    with open(GOLD) as f:
        g = json.load(f)
    res = oracle.moe_layer(make_workload(0), BM=16)
    assert res["topk_ids"].tolist() == g["topk_ids"]
    np.testing.assert_allclose(res["topk_weights"], g["topk_weights"], rtol=1e-14, atol=0)
    assert res["expert_offsets"].tolist() == g["expert_offsets"]
    assert res["sorted_ids"].tolist() == g["sorted_ids"]
    assert res["tiles"].tolist() == g["tiles"] and res["num_tiles"] == g["num_tiles"]
    for t, h, v in g["out_samples"]:
        assert abs(res["out"][t, h] - v) <= 1e-12 * max(1.0, abs(v))
    assert abs(np.linalg.norm(res["out"]) - g["out_l2"]) <= 1e-12 * g["out_l2"]
