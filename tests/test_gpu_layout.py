"""GPU: the blocked weight layout (moe_repack_weights and layout arguments).

The repack must produce exactly the oracle's blocked layout, byte for byte,
and every entry point that reads packed codes must give bit-identical
outputs for the canonical codes and their blocked copy (the layouts differ
only in where the bytes sit; every kernel runs the same arithmetic on the
same values in the same order).  The shapes cover the one-token kernels,
the row-tile kernels at every pass size, several K chunks, ragged K tails
and the large-tile (prefill) kernel.
"""
import numpy as np
import pytest
import torch

import mxfp4_grouped_expert_amd as moe
import oracle
from moe_inputs import make_random

from gpu_helpers import assert_out_close, log, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    moe.load()


@pytest.mark.parametrize("shape", [(1, 16, 16), (3, 64, 48), (2, 5760, 1440), (4, 2880, 1440),
                                   (1, 48, 2048)])
def test_repack_matches_oracle(shape):
    rng = np.random.default_rng(sum(shape))
    q = rng.integers(0, 256, size=shape, dtype=np.uint8)
    log(f"repack {shape}")
    got = moe.moe_repack_weights(torch.from_numpy(q).cuda())
    torch.cuda.synchronize()
    assert got.shape == q.shape
    np.testing.assert_array_equal(got.cpu().numpy(), oracle.blocked_from_canonical(q))


def _blocked(d):
    b = dict(d)
    b["w13_q"] = moe.moe_repack_weights(d["w13_q"])
    b["w2_q"] = moe.moe_repack_weights(d["w2_q"])
    return b


# (T, H, I, E, k): one token (exchange gate/up, fused down + combine), small
# ragged shapes, 16-row passes with 4 blocks per workgroup, one-row passes at
# 128 experts, the large-tile kernel, and K > 3072 (several chunks) on each
# GEMM
FORWARD = [(1, 2880, 2880, 32, 4), (5, 320, 224, 6, 3), (64, 2880, 2880, 32, 4),
           (16, 256, 256, 128, 4), (512, 256, 192, 4, 2), (8, 4096, 512, 8, 2),
           (8, 512, 3584, 4, 2)]


@pytest.mark.parametrize("case", FORWARD, ids=lambda c: "T{}_H{}_I{}_E{}_k{}".format(*c))
def test_forward_blocked_equals_canonical(case):
    T, H, I, E, k = case
    inp = make_random(T=T, H=H, E=E, k=k, I=I, seed=700 + T + E)
    d = to_device(inp)
    b = _blocked(d)
    BM = moe.pick_bm(T, k, E)
    ids, wts, _ = moe.moe_route(d["x"], d["w_router"], d["bias"], k)
    off, srt, tiles, nt = moe.moe_build_tiles(ids, E, BM)
    log(f"forward T={T} H={H} I={I} E={E} k={k}: canonical")
    want = moe.moe_forward(d["x"], d["w13_q"], d["w13_s"], d["w2_q"], d["w2_s"], wts, srt, tiles,
                           nt, BM)
    log(f"forward T={T} H={H} I={I} E={E} k={k}: blocked")
    got = moe.moe_forward(b["x"], b["w13_q"], b["w13_s"], b["w2_q"], b["w2_s"], wts, srt, tiles,
                          nt, BM, layout="blocked")
    h_c = moe.moe_gateup_swiglu(d["x"], d["w13_q"], d["w13_s"], srt, tiles, nt, k, BM)
    h_b = moe.moe_gateup_swiglu(b["x"], b["w13_q"], b["w13_s"], srt, tiles, nt, k, BM,
                                layout="blocked")
    y_c = moe.moe_down(h_c, d["w2_q"], d["w2_s"], srt, tiles, nt, T, k, BM)
    y_b = moe.moe_down(h_c, b["w2_q"], b["w2_s"], srt, tiles, nt, T, k, BM, layout="blocked")
    torch.cuda.synchronize()
    n = int(nt.item())
    rows = srt.numel()
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))
    if n:
        assert torch.equal(h_b[:rows].view(torch.int16), h_c[:rows].view(torch.int16))
        assert torch.equal(y_b.view(torch.int32), y_c.view(torch.int32))


def test_blocked_forward_matches_oracle():
    inp = make_random(T=5, H=320, E=6, k=3, I=224, seed=41)
    d = _blocked(to_device(inp))
    BM = moe.pick_bm(5, 3, 6)
    ids, wts, _ = moe.moe_route(d["x"], d["w_router"], d["bias"], 3)
    off, srt, tiles, nt = moe.moe_build_tiles(ids, 6, BM)
    log("blocked forward vs oracle")
    out = moe.moe_forward(d["x"], d["w13_q"], d["w13_s"], d["w2_q"], d["w2_s"], wts, srt, tiles,
                          nt, BM, layout="blocked")
    torch.cuda.synchronize()
    r = oracle.moe_layer(inp, BM=BM)
    assert_out_close(out.float().cpu().numpy().astype(np.float64), r["out"])


@pytest.mark.parametrize("case", [(2880, 2880, 32, 4), (320, 224, 6, 3), (3072, 3072, 8, 2),
                                  (128, 96, 256, 8)],
                         ids=lambda c: "H{}_I{}_E{}_k{}".format(*c))
def test_one_token_blocked_equals_canonical(case):
    H, I, E, k = case
    inp = make_random(T=1, H=H, E=E, k=k, I=I, seed=900 + E, router_std=0.3)
    d = to_device(inp)
    b = _blocked(d)
    BM = moe.pick_bm(1, k, E)
    ws_c = moe.zeroed_layer_one_token_workspace(H, I, E, k, d["x"].device)
    ws_b = moe.zeroed_layer_one_token_workspace(H, I, E, k, d["x"].device)
    for call in range(2):
        log(f"one-token layer H={H} I={I} E={E} k={k}: canonical and blocked, call {call}")
        want = moe.moe_layer_one_token(d["x"], d["w_router"], d["bias"], d["w13_q"], d["w13_s"],
                                       d["w2_q"], d["w2_s"], k, BM, workspace=ws_c)
        got = moe.moe_layer_one_token(b["x"], b["w_router"], b["bias"], b["w13_q"], b["w13_s"],
                                      b["w2_q"], b["w2_s"], k, BM, workspace=ws_b,
                                      layout="blocked")
        torch.cuda.synchronize()
        assert torch.equal(got[0].view(torch.int16), want[0].view(torch.int16)), f"call {call}"
        assert torch.equal(got[1], want[1]) and torch.equal(got[2], want[2])
        head = ws_b[:12].cpu().numpy().view(np.int32)
        assert (int(head[1]), int(head[2])) == (call + 1, 0)


@pytest.mark.parametrize("T", [1, 64])
def test_layer_blocked_equals_canonical(T):
    inp = make_random(T=T, H=2880, E=32, k=4, I=2880, seed=55)
    d = to_device(inp)
    args = (d["w_router"], d["bias"], d["w13_q"], d["w13_s"], d["w2_q"], d["w2_s"], 4)
    canon = moe.MoeLayer(*args, layout="canonical").plan(T)
    blk = moe.MoeLayer(*args, layout="blocked").plan(T)
    log(f"MoeLayer T={T}: canonical and blocked")
    want = canon(d["x"]).clone()
    got = blk(d["x"])
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))
    assert torch.equal(blk.w13_q.cpu(), torch.from_numpy(
        oracle.blocked_from_canonical(inp["w13_q"])))
