"""GPU parity of the two other MoE families' shapes at the sizes the
benchmark times (workloads 5 and 6, 128 tokens each): the Mixtral-8x7B-shaped
layer (8 experts, top-2, hidden 4096, FFN 14336) and the DeepSeek-V3-shaped
layer with sigmoid gating (256 experts, top-8, hidden 7168, expert FFN 2048;
the triton-kernels README's MoE dispatch benchmark names these families).
Both the separate entry points (canonical weights) and the benchmark's own
configuration (MoeLayer, blocked weights) are compared with the float64
oracle on every token, so every expert the routing touches is checked.  The
oracle decodes every touched expert once: about 20 s for the first layer and
about 2 minutes for the second (252 of 256 experts touched), with a progress
line every 16 experts.
"""
import numpy as np
import pytest
import torch

import mxfp4_grouped_expert_amd as moe
from moe_inputs import make_workload

from gpu_helpers import (assert_out_close, check_all, log, oracle_layer, to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    moe.load()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wid", [5, 6])
def test_other_family_at_bench_shape(wid):
    inp = make_workload(wid)
    T, k, E = inp["T"], inp["k"], inp["E"]
    BM = moe.pick_bm(T, k, E)
    ref = oracle_layer(inp, BM)
    touched = np.unique(ref["topk_ids"])
    log(f"workload {wid}: {touched.size} of {E} experts touched")
    check_all(inp, BM, ref=ref)
    d = to_device(inp)
    layer = moe.MoeLayer(d["w_router"], d["bias"], d["w13_q"], d["w13_s"], d["w2_q"], d["w2_s"],
                         k, gating=inp["gating"]).plan(T)
    assert layer.BM == BM
    log(f"bench configuration, workload {wid}: MoeLayer (layout blocked, BM {BM})")
    out = layer(d["x"]).float().cpu().numpy().astype(np.float64)
    np.testing.assert_array_equal(layer.topk_ids.cpu().numpy(), ref["topk_ids"])
    np.testing.assert_allclose(layer.topk_weights.cpu().numpy(), ref["topk_weights"], rtol=0,
                               atol=1e-6)
    assert len(ref["tokens"]) == T
    assert_out_close(out, ref["out"], f"bench configuration, workload {wid}")
