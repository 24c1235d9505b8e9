"""GPU: sigmoid gating on every routing path, and the two layers shaped like
the triton-kernels README's MoE dispatch benchmark (Mixtral-8x7B-shaped:
8 experts, top-2, hidden 4096, FFN 14336; DeepSeek-V3-shaped: sigmoid
gating, hidden 7168, expert FFN 2048, top-8, here with 16 experts), against
the float64 oracle at the usual bar.  Both of those shapes have a reduction
length above one register chunk (K > 3072), so they also cover the
multi-chunk form of the row-tile GEMMs.
"""
import numpy as np
import pytest
import torch

import mxfp4_grouped_expert_amd as moe
from moe_inputs import make_random

from gpu_helpers import check_all, log, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    moe.load()


SIGMOID_CASES = [
    # T, H, E, k, I, bias, router_std, BM
    (1, 320, 6, 3, 224, False, 0.3, 16),
    (5, 256, 33, 4, 128, True, 0.3, 16),
    (64, 256, 33, 4, 512, True, 0.3, 16),
    (1100, 64, 40, 2, 32, False, 0.5, 128),   # fp64-MFMA logits, 128-row GEMMs
    (300, 128, 256, 8, 64, False, 1.0, 128),  # E and k at their maxima
]


@pytest.mark.parametrize("case", SIGMOID_CASES, ids=lambda c: "T{}_H{}_E{}_k{}_I{}".format(*c[:5]))
def test_sigmoid_layer_matches_oracle(case):
    T, H, E, k, I, bias, std, BM = case
    inp = make_random(T=T, H=H, E=E, k=k, I=I, seed=50 + T + E, router_bias=bias,
                      router_std=std, gating="sigmoid")
    check_all(inp, BM)


@pytest.mark.parametrize("T", [1, 5, 16])
def test_sigmoid_route_tiles_equals_route(T):
    inp = make_random(T=T, H=256, E=24, k=4, I=64, seed=60 + T, router_bias=True,
                      router_std=0.3, gating="sigmoid")
    d = to_device(inp)
    BM = moe.pick_bm(T, 4, 24)
    log(f"sigmoid route_tiles T={T}")
    ids, wts, logits = moe.moe_route(d["x"], d["w_router"], d["bias"], 4, want_logits=True,
                                     gating="sigmoid")
    off, srt, tiles, nt = moe.moe_build_tiles(ids, 24, BM)
    f = moe.moe_route_tiles(d["x"], d["w_router"], d["bias"], 4, BM, want_logits=True,
                            gating="sigmoid")
    soft = moe.moe_route(d["x"], d["w_router"], d["bias"], 4, gating="softmax")
    torch.cuda.synchronize()
    assert torch.equal(f[0], ids) and torch.equal(f[1].view(torch.int32), wts.view(torch.int32))
    assert torch.equal(f[2].view(torch.int64), logits.view(torch.int64))
    n = int(nt.item())
    assert torch.equal(f[3], off) and torch.equal(f[4], srt) and int(f[6].item()) == n
    assert torch.equal(f[5][:n], tiles[:n])
    assert torch.equal(soft[0], ids) and not torch.equal(soft[1], wts)


@pytest.mark.parametrize("gating", ["sigmoid"])
def test_sigmoid_one_launch_equals_separate_launches(gating):
    inp = make_random(T=1, H=2880, E=32, k=4, I=2880, seed=71, router_std=0.3, gating=gating)
    d = to_device(inp)
    BM = moe.pick_bm(1, 4, 32)
    log("sigmoid one-token layer")
    ids, wts, logits, off, srt, tiles, nt = moe.moe_route_tiles(
        d["x"], d["w_router"], None, 4, BM, want_logits=True, gating=gating)
    want = moe.moe_forward(d["x"], d["w13_q"], d["w13_s"], d["w2_q"], d["w2_s"], wts, srt, tiles,
                           nt, BM)
    got = moe.moe_layer_one_token(d["x"], d["w_router"], None, d["w13_q"], d["w13_s"], d["w2_q"],
                                  d["w2_s"], 4, BM, want_logits=True, gating=gating)
    torch.cuda.synchronize()
    assert torch.equal(got[0].view(torch.int16), want.view(torch.int16))
    assert torch.equal(got[1], ids) and torch.equal(got[2].view(torch.int32), wts.view(torch.int32))


def test_mixtral_shaped_layer():
    inp = make_random(T=8, H=4096, E=8, k=2, I=14336, seed=81, router_std=0.02)
    check_all(inp, 16)


def test_deepseek_v3_shaped_layer_sigmoid():
    inp = make_random(T=8, H=7168, E=16, k=8, I=2048, seed=82, router_std=0.02,
                      gating="sigmoid")
    check_all(inp, 16)
