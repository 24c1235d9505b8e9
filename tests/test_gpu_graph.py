"""GPU: graph replay and the step entry points give bit-identical results.

A captured layer call is replayed several times with unrelated eager work and
synchronisations in between; every replay must equal the eager result bit for
bit.  The three step entry points (moe_gateup_swiglu, moe_down, moe_combine)
must reproduce moe_forward exactly.
"""
import numpy as np
import pytest
import torch

import mxfp4_grouped_expert_amd as moe
from moe_inputs import make_random, make_workload

from gpu_helpers import log, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    moe.load()


def _layer(inp):
    d = to_device(inp)
    layer = moe.MoeLayer(d["w_router"], d["bias"], d["w13_q"], d["w13_s"], d["w2_q"], d["w2_s"],
                         inp["k"]).plan(inp["T"])
    return d, layer


@pytest.mark.parametrize("wid", [0, 2])
def test_graph_replays_match_eager(wid):
    inp = make_workload(wid)
    d, layer = _layer(inp)
    x = d["x"]
    log(f"graph replay, workload {wid}: eager reference")
    ref = layer(x).clone()
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            layer(x)
    torch.cuda.synchronize()
    other = make_random(T=inp["T"], H=inp["H"], E=inp["E"], k=inp["k"], I=inp["I"], seed=9)
    x_other = torch.from_numpy(other["x"].view(np.int16)).cuda()
    for rep in range(4):
        log(f"graph replay {rep}")
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        got = layer.out.clone()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"replay {rep}"
        # unrelated eager work between replays: a different batch through the
        # same buffers, plus a plain torch op
        layer(x_other)
        _ = (x_other.float() * 2).sum()
        torch.cuda.synchronize()


# One token takes the fused down + combine launch inside moe_forward; it must
# match the separate entry points bit for bit.
STEP_CASES = [(37, 320, 6, 3, 224), (1, 320, 6, 3, 224), (1, 2880, 8, 4, 2880), (1, 64, 1, 1, 32)]


@pytest.mark.parametrize("case", STEP_CASES, ids=lambda c: "T{}_H{}_E{}_k{}_I{}".format(*c))
def test_step_entry_points_equal_forward(case):
    T, H, E, k, I = case
    inp = make_random(T=T, H=H, E=E, k=k, I=I, seed=21 + T, router_std=0.3)
    d = to_device(inp)
    k, E, BM = inp["k"], inp["E"], 16
    log("step entry points vs moe_forward")
    ids, wts, _ = moe.moe_route(d["x"], d["w_router"], None, k)
    off, srt, tiles, nt = moe.moe_build_tiles(ids, E, BM)
    full = moe.moe_forward(d["x"], d["w13_q"], d["w13_s"], d["w2_q"], d["w2_s"], wts, srt, tiles,
                           nt, BM)
    h = moe.moe_gateup_swiglu(d["x"], d["w13_q"], d["w13_s"], srt, tiles, nt, k, BM)
    y = moe.moe_down(h, d["w2_q"], d["w2_s"], srt, tiles, nt, inp["T"], k, BM)
    out = moe.moe_combine(y, wts)
    torch.cuda.synchronize()
    assert torch.equal(full.view(torch.int16), out.view(torch.int16))
