"""GPU: the one-token layer in one launch (moe_layer_one_token).

Every output must equal moe_route_tiles + moe_forward bit for bit on every
call and graph replay (the workspace's counters and flags carry over from
call to call), each call must advance the workspace's call count by one and
leave its error word zero, and the output must meet the parity bar against
the float64 oracle.
"""
import numpy as np
import pytest
import torch

import mxfp4_grouped_expert_amd as moe
import oracle
from moe_inputs import make_random, make_workload

from gpu_helpers import assert_out_close, log, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    moe.load()


def _unfused(d, k, BM):
    ids, wts, logits, off, srt, tiles, nt = moe.moe_route_tiles(d["x"], d["w_router"], d["bias"],
                                                                k, BM, want_logits=True)
    out = moe.moe_forward(d["x"], d["w13_q"], d["w13_s"], d["w2_q"], d["w2_s"], wts, srt, tiles,
                          nt, BM)
    return out, ids, wts, logits, off, srt, tiles, nt


def _fused(d, k, BM, ws):
    return moe.moe_layer_one_token(d["x"], d["w_router"], d["bias"], d["w13_q"], d["w13_s"],
                                   d["w2_q"], d["w2_s"], k, BM, want_logits=True, workspace=ws)


def _assert_same(got, want, what):
    names = ("out", "topk_ids", "topk_weights", "logits", "expert_offsets", "sorted_ids")
    for name, g, w in zip(names, got[:6], want[:6]):
        assert torch.equal(g.view(torch.uint8), w.view(torch.uint8)), f"{what}: {name} differs"
    n = int(want[7].item())
    assert int(got[7].item()) == n, f"{what}: num_tiles differs"
    assert torch.equal(got[6][:n], want[6][:n]), f"{what}: tiles differ"


def _calls_and_error(ws):
    """(completed calls, error word) from the head of the sync region."""
    head = ws[:12].cpu().numpy().view(np.int32)
    return int(head[1]), int(head[2])


# (H, I, E, k, bias): the gpt-oss-20b shape, 128 experts (two per lane in
# the top-k), odd small shapes, one expert, 256 experts with k = 8, the
# largest H and I, and router biases
CASES = [(2880, 2880, 32, 4, False), (256, 256, 128, 4, False), (320, 224, 6, 3, False),
         (64, 32, 1, 1, False), (128, 96, 256, 8, True), (3072, 3072, 8, 2, True)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "H{}_I{}_E{}_k{}_b{}".format(*c))
def test_one_launch_equals_separate_launches(case):
    H, I, E, k, bias = case
    inp = make_random(T=1, H=H, E=E, k=k, I=I, seed=300 + E + k, router_bias=bias,
                      router_std=0.3)
    d = to_device(inp)
    BM = moe.pick_bm(1, k, E)
    log(f"one-token layer H={H} I={I} E={E} k={k}: separate launches")
    want = _unfused(d, k, BM)
    ws = moe.zeroed_layer_one_token_workspace(H, I, E, k, d["x"].device)
    for call in range(3):
        log(f"one-token layer H={H} I={I} E={E} k={k}: one launch, call {call}")
        got = _fused(d, k, BM, ws)
        torch.cuda.synchronize()
        _assert_same(got, want, f"call {call}")
        assert _calls_and_error(ws) == (call + 1, 0), f"call {call}: counters"


@pytest.mark.parametrize("wid", [1])
def test_one_launch_matches_oracle(wid):
    inp = make_workload(wid)
    d = to_device(inp)
    k, E, H, I = inp["k"], inp["E"], inp["H"], inp["I"]
    BM = moe.pick_bm(1, k, E)
    ws = moe.zeroed_layer_one_token_workspace(H, I, E, k, d["x"].device)
    log(f"one-token layer, workload {wid}: one launch")
    out, ids, wts, _, off, srt, tiles, nt = _fused(d, k, BM, ws)
    torch.cuda.synchronize()
    log(f"one-token layer, workload {wid}: oracle")
    r = oracle.moe_layer(inp, BM=BM)
    np.testing.assert_array_equal(ids.cpu().numpy(), r["topk_ids"])
    np.testing.assert_allclose(wts.cpu().numpy(), r["topk_weights"], rtol=0, atol=1e-6)
    np.testing.assert_array_equal(off.cpu().numpy(), r["expert_offsets"])
    np.testing.assert_array_equal(srt.cpu().numpy(), r["sorted_ids"])
    n = int(nt.item())
    assert n == r["num_tiles"]
    np.testing.assert_array_equal(tiles[:n].cpu().numpy(), r["tiles"])
    assert_out_close(out.float().cpu().numpy().astype(np.float64)[r["tokens"]], r["out"])


def test_layer_graph_replays_one_launch():
    """The layer at T = 1 runs as one launch; replays of a captured call with
    other calls between them stay bit-identical and count every call."""
    inp = make_workload(1)
    d = to_device(inp)
    layer = moe.MoeLayer(d["w_router"], d["bias"], d["w13_q"], d["w13_s"], d["w2_q"], d["w2_s"],
                         inp["k"]).plan(1)
    assert layer.one_launch
    x = d["x"]
    log("one-token layer graph: eager reference")
    ref = layer(x).clone()
    sep = moe.MoeLayer(d["w_router"], d["bias"], d["w13_q"], d["w13_s"], d["w2_q"], d["w2_s"],
                       inp["k"]).plan(1, one_launch=False)
    assert torch.equal(sep(x).view(torch.int16), ref.view(torch.int16))
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            layer(x)
    torch.cuda.synchronize()
    other = make_random(T=1, H=inp["H"], E=inp["E"], k=inp["k"], I=inp["I"], seed=11)
    x_other = torch.from_numpy(other["x"].view(np.int16)).cuda()
    calls, err = _calls_and_error(layer.one_ws)
    assert err == 0
    for rep in range(4):
        log(f"one-token layer graph replay {rep}")
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(layer.out.view(torch.int16), ref.view(torch.int16)), f"replay {rep}"
        layer(x_other)
        torch.cuda.synchronize()
        assert _calls_and_error(layer.one_ws) == (calls + 2 * (rep + 1), 0)


def test_bounded_wait_gives_up_reports_and_recovers():
    """With the poll bound lowered to zero re-polls (the sync region's int at
    byte 12 set to 1 from the host) a wait that finds its data not yet there
    gives up at once: the call still completes, its error word is set, and
    after the sync region is zeroed the next call is exact again."""
    H, I, E, k = 256, 256, 16, 4
    inp = make_random(T=1, H=H, E=E, k=k, I=I, seed=77)
    d = to_device(inp)
    BM = moe.pick_bm(1, k, E)
    want = _unfused(d, k, BM)
    ws = moe.zeroed_layer_one_token_workspace(H, I, E, k, d["x"].device)
    ws[12:16].view(torch.int32).fill_(1)
    log("one-token layer: poll bound 0")
    _fused(d, k, BM, ws)
    torch.cuda.synchronize()
    calls, err = _calls_and_error(ws)
    assert calls == 1 and err == 1, (calls, err)
    ws.zero_()
    log("one-token layer: normal bound after zeroing")
    got = _fused(d, k, BM, ws)
    torch.cuda.synchronize()
    _assert_same(got, want, "after recovery")
    assert _calls_and_error(ws) == (1, 0)
