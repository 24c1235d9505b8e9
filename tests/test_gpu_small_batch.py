"""GPU: the small-batch layer in one launch (moe_layer_small_batch, 2..4 tokens).

Every output must equal moe_route_tiles + moe_forward (blocked codes) bit
for bit on every call and graph replay (the workspace's counters and
published words carry over from call to call, also across batch sizes),
each call must advance the workspace's call count by one and leave its error
word zero, the output must meet the parity bar against the float64 oracle,
and MoeLayer must take this path for 2..4 tokens when asked to.
"""
import numpy as np
import pytest
import torch

import mxfp4_grouped_expert_amd as moe
import oracle
from moe_inputs import make_activations, make_random, make_weights

from gpu_helpers import assert_out_close, log, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    moe.load()


def _blocked(d):
    b = dict(d)
    b["w13_q"] = moe.moe_repack_weights(d["w13_q"])
    b["w2_q"] = moe.moe_repack_weights(d["w2_q"])
    return b


def _unfused(d, k, BM, gating="softmax"):
    ids, wts, logits, off, srt, tiles, nt = moe.moe_route_tiles(
        d["x"], d["w_router"], d["bias"], k, BM, want_logits=True, gating=gating)
    out = moe.moe_forward(d["x"], d["w13_q"], d["w13_s"], d["w2_q"], d["w2_s"], wts, srt, tiles,
                          nt, BM, layout="blocked")
    return out, ids, wts, logits, off, srt, tiles, nt


def _fused(d, k, BM, ws, gating="softmax"):
    return moe.moe_layer_small_batch(d["x"], d["w_router"], d["bias"], d["w13_q"], d["w13_s"],
                                     d["w2_q"], d["w2_s"], k, BM, want_logits=True, workspace=ws,
                                     gating=gating)


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


# (T, H, I, E, k, bias, std, gating): the gpt-oss-20b shape at 2, 3 and 4
# tokens (with a flat router and a skewed one, so that experts get several
# rows), 128 experts, odd small shapes, one expert (one tile of T rows),
# 256 experts with k = 8, the largest H and I, and sigmoid gating
CASES = [(2, 2880, 2880, 32, 4, False, 0.02, "softmax"),
         (3, 2880, 2880, 32, 4, True, 0.02, "softmax"),
         (4, 2880, 2880, 32, 4, False, 0.02, "softmax"),
         (4, 2880, 2880, 32, 4, True, 0.5, "softmax"),
         (4, 256, 256, 128, 4, False, 0.3, "softmax"),
         (3, 320, 224, 6, 3, False, 0.3, "softmax"),
         (4, 64, 32, 1, 1, False, 0.3, "softmax"),
         (2, 128, 96, 256, 8, True, 0.3, "softmax"),
         (2, 3072, 3072, 8, 2, True, 0.3, "softmax"),
         (4, 512, 256, 16, 4, True, 0.3, "sigmoid")]


def _case_input(case):
    T, H, I, E, k, bias, std, gating = case
    inp = make_random(T=T, H=H, E=E, k=k, I=I, seed=500 + T + E + k, router_bias=bias,
                      router_std=std)
    inp["gating"] = gating
    return inp


@pytest.mark.parametrize("case", CASES, ids=lambda c: "T{}_H{}_I{}_E{}_k{}_b{}_s{}_{}".format(*c))
def test_small_batch_equals_separate_launches(case):
    T, H, I, E, k, bias, std, gating = case
    d = _blocked(to_device(_case_input(case)))
    BM = moe.pick_bm(T, k, E)
    log(f"small-batch layer {case}: separate launches")
    want = _unfused(d, k, BM, gating)
    ws = moe.zeroed_layer_small_batch_workspace(T, H, I, E, k, d["x"].device)
    for call in range(3):
        log(f"small-batch layer {case}: one launch, call {call}")
        got = _fused(d, k, BM, ws, gating)
        torch.cuda.synchronize()
        _assert_same(got, want, f"call {call}")
        assert _calls_and_error(ws) == (call + 1, 0), f"call {call}: counters"
    n = int(want[7].item())
    rows = want[6][:n, 2].cpu().numpy()
    log(f"small-batch layer {case}: {n} tiles, rows {sorted(rows.tolist(), reverse=True)}")


def test_one_workspace_across_batch_sizes():
    """One workspace serves calls of 4, 2, 3 and 4 tokens in a row (the
    partial buffers are cleared for any shape, the plan words are stamped)."""
    H = I = 2880
    E, k = 32, 4
    w = make_weights(E, H, I, 20)
    ws = None
    for call, T in enumerate((4, 2, 3, 4)):
        inp = dict(T=T, H=H, E=E, k=k, I=I, gating="softmax")
        inp.update(make_activations(T, H, E, [900 + call, 2], call % 2 == 1, 0.3))
        inp.update(w)
        d = _blocked(to_device(inp))
        BM = moe.pick_bm(T, k, E)
        if ws is None:
            ws = moe.zeroed_layer_small_batch_workspace(4, H, I, E, k, d["x"].device)
        log(f"small-batch layer: call {call}, T={T}")
        want = _unfused(d, k, BM)
        got = _fused(d, k, BM, ws)
        torch.cuda.synchronize()
        _assert_same(got, want, f"call {call} (T={T})")
        assert _calls_and_error(ws) == (call + 1, 0)


@pytest.mark.parametrize("T", [2, 4])
def test_small_batch_matches_oracle(T):
    inp = dict(T=T, H=2880, E=32, k=4, I=2880, gating="softmax")
    inp.update(make_activations(T, 2880, 32, [T, 7], False))
    inp.update(make_weights(32, 2880, 2880, 20))
    d = _blocked(to_device(inp))
    k, E = inp["k"], inp["E"]
    BM = moe.pick_bm(T, k, E)
    ws = moe.zeroed_layer_small_batch_workspace(T, 2880, 2880, E, k, d["x"].device)
    log(f"small-batch layer T={T}: one launch")
    out, ids, wts, _, off, srt, tiles, nt = _fused(d, k, BM, ws)
    torch.cuda.synchronize()
    log(f"small-batch layer T={T}: oracle")
    r = oracle.moe_layer(inp, BM=BM)
    np.testing.assert_array_equal(ids.cpu().numpy(), r["topk_ids"])
    np.testing.assert_allclose(wts.cpu().numpy(), r["topk_weights"], rtol=0, atol=1e-6)
    np.testing.assert_array_equal(off.cpu().numpy(), r["expert_offsets"])
    np.testing.assert_array_equal(srt.cpu().numpy(), r["sorted_ids"])
    n = int(nt.item())
    assert n == r["num_tiles"]
    np.testing.assert_array_equal(tiles[:n].cpu().numpy(), r["tiles"])
    assert_out_close(out.float().cpu().numpy().astype(np.float64)[r["tokens"]], r["out"],
                     f"small-batch layer T={T}")


def test_layer_takes_small_batch_launch_and_replays():
    """MoeLayer runs 2..4 tokens as one launch when asked to; replays of a
    captured call with other calls between them stay bit-identical to the
    separate launches and count every call."""
    T, H, I, E, k = 3, 2880, 2880, 32, 4
    inp = dict(T=T, H=H, E=E, k=k, I=I, gating="softmax")
    inp.update(make_activations(T, H, E, [33, 2], True, 0.3))
    inp.update(make_weights(E, H, I, 20))
    d = to_device(inp)
    layer = moe.MoeLayer(d["w_router"], d["bias"], d["w13_q"], d["w13_s"], d["w2_q"], d["w2_s"],
                         k).plan(T, small_batch=True)
    assert layer.small_launch
    x = d["x"]
    log("small-batch layer graph: eager reference")
    ref = layer(x).clone()
    sep = moe.MoeLayer(d["w_router"], d["bias"], d["w13_q"], d["w13_s"], d["w2_q"], d["w2_s"],
                       k).plan(T)
    assert not sep.small_launch
    assert torch.equal(sep(x).view(torch.int16), ref.view(torch.int16))
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            layer(x)
    torch.cuda.synchronize()
    other = make_activations(T, H, E, [34, 2], True, 0.3)
    x_other = torch.from_numpy(other["x"].view(np.int16)).cuda()
    calls, err = _calls_and_error(layer.small_ws)
    assert err == 0
    for rep in range(4):
        log(f"small-batch layer graph replay {rep}")
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(layer.out.view(torch.int16), ref.view(torch.int16)), f"replay {rep}"
        layer(x_other)
        torch.cuda.synchronize()
        assert _calls_and_error(layer.small_ws) == (calls + 2 * (rep + 1), 0)


def test_small_batch_bounded_wait_gives_up_reports_and_recovers():
    """With the poll bound lowered to zero re-polls (the sync region's int at
    byte 12 set to 1 from the host) a wait that finds its data not yet there
    gives up at once: the call still completes, its error word is set, and
    after the sync region is zeroed the next call is exact again."""
    T, H, I, E, k = 3, 256, 256, 16, 4
    d = _blocked(to_device(make_random(T=T, H=H, E=E, k=k, I=I, seed=78)))
    BM = moe.pick_bm(T, k, E)
    want = _unfused(d, k, BM)
    ws = moe.zeroed_layer_small_batch_workspace(T, H, I, E, k, d["x"].device)
    ws[12:16].view(torch.int32).fill_(1)
    log("small-batch layer: poll bound 0")
    _fused(d, k, BM, ws)
    torch.cuda.synchronize()
    calls, err = _calls_and_error(ws)
    assert calls == 1 and err == 1, (calls, err)
    ws.zero_()
    log("small-batch layer: normal bound after zeroing")
    got = _fused(d, k, BM, ws)
    torch.cuda.synchronize()
    _assert_same(got, want, "after recovery")
    assert _calls_and_error(ws) == (1, 0)
