"""GPU: the fused decode routing entry point (moe_route_tiles).

Its outputs must be bit-identical to moe_route + moe_build_tiles and match
the oracle (bit-exact ids and tables, weights within 1e-6) on both of its
kernels (one tail workgroup up to 16 tokens; the token relay from 17 to 64);
its sync block must return to zero after every call, so one workspace
serves calls of different sizes in a row and under graph replay.
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


def _router_inputs(inp):
    x = torch.from_numpy(np.ascontiguousarray(inp["x"]).view(np.int16)).cuda()
    wr = torch.from_numpy(inp["w_router"]).cuda()
    b = None if inp.get("bias") is None else torch.from_numpy(inp["bias"]).cuda()
    return x, wr, b


def _workload(wid):
    return make_workload(wid, weights=False)


def _random(T, H, E, k, bias, std, seed, gating="softmax"):
    from moe_inputs import make_activations
    inp = dict(T=T, H=H, E=E, k=k, name=f"rand_T{T}_H{H}_E{E}_k{k}", gating=gating)
    inp.update(make_activations(T, H, E, [2000 + seed, 2], bias, std))
    return inp


CASES = {
    "tiny": lambda: _workload(0),
    "20b_T1": lambda: _workload(1),
    "E1_k1": lambda: _random(1, 64, 1, 1, False, 0.02, 1),
    "T16_E33_k3_bias": lambda: _random(16, 160, 33, 3, True, 0.3, 2),
    "T16_E8_k8": lambda: _random(16, 96, 8, 8, False, 0.5, 3),
    "T3_E256_k8": lambda: _random(3, 2880, 256, 8, True, 0.02, 4),
    "T2_E32_k4": lambda: _random(2, 2880, 32, 4, False, 0.02, 15),
    "T5_E32_k4_bias": lambda: _random(5, 2880, 32, 4, True, 0.3, 16),
    "T16_E128_k4_H2880": lambda: _random(16, 2880, 128, 4, False, 0.02, 7),
    # the token relay (17..64 tokens)
    "T17_E32_k4": lambda: _random(17, 2880, 32, 4, False, 0.02, 9),
    "20b_T64_biased": lambda: _workload(2),
    "120b_T64": lambda: _workload(3),
    "T33_E33_k3_bias": lambda: _random(33, 160, 33, 3, True, 0.3, 10),
    "T64_E256_k8": lambda: _random(64, 2880, 256, 8, True, 0.02, 11),
    "T40_E100_k4": lambda: _random(40, 512, 100, 4, False, 0.3, 12),
    "T48_E24_k4_sigmoid": lambda: _random(48, 256, 24, 4, True, 0.3, 13, "sigmoid"),
    "T64_E1_k1": lambda: _random(64, 64, 1, 1, False, 0.02, 14),
}


@pytest.mark.parametrize("name", list(CASES))
def test_fused_equals_separate_and_oracle(name):
    inp = CASES[name]()
    T, E, k = inp["T"], inp["E"], inp["k"]
    BM = moe.pick_bm(T, k, E)
    gating = inp.get("gating", "softmax")
    x, wr, b = _router_inputs(inp)
    log(f"route_tiles {name}: fused")
    f = moe.moe_route_tiles(x, wr, b, k, BM, want_logits=True, gating=gating)
    log(f"route_tiles {name}: separate")
    ids, wts, logits = moe.moe_route(x, wr, b, k, want_logits=True, gating=gating)
    off, srt, tiles, nt = moe.moe_build_tiles(ids, E, BM)
    torch.cuda.synchronize()
    n = int(nt.item())
    assert int(f[6].item()) == n
    for a, c in ((f[0], ids), (f[1], wts), (f[2], logits), (f[3], off), (f[4], srt),
                 (f[5][:n], tiles[:n])):
        assert torch.equal(a, c)
    ref_ids, ref_w, _ = oracle.route(inp["x"], inp["w_router"], inp.get("bias"), k, gating)
    np.testing.assert_array_equal(f[0].cpu().numpy(), ref_ids)
    np.testing.assert_allclose(f[1].cpu().numpy(), ref_w, rtol=0, atol=1e-6)
    r_off, r_srt, r_tiles, r_n = oracle.build_tiles(ref_ids, E, BM)
    assert n == r_n
    np.testing.assert_array_equal(f[3].cpu().numpy(), r_off)
    np.testing.assert_array_equal(f[4].cpu().numpy(), r_srt)
    np.testing.assert_array_equal(f[5][:n].cpu().numpy(), r_tiles)


def test_counter_returns_to_zero_across_sizes():
    inp = _random(64, 256, 32, 4, True, 0.3, 5)
    x, wr, b = _router_inputs(inp)
    ws = moe.zeroed_route_tiles_workspace(64, 256, 32, x.device)
    for T in (1, 16, 3, 64, 1, 11, 17, 40, 16, 64, 33):
        log(f"counter reuse T={T}")
        xs = x[:T].contiguous()
        BM = moe.pick_bm(T, 4, 32)
        f = moe.moe_route_tiles(xs, wr, b, 4, BM, workspace=ws)
        torch.cuda.synchronize()
        assert int(ws[:256].count_nonzero().item()) == 0, f"counter not reset after T={T}"
        ref_ids, _, _ = oracle.route(inp["x"][:T], inp["w_router"], inp["bias"], 4)
        np.testing.assert_array_equal(f[0].cpu().numpy(), ref_ids)
        r = oracle.build_tiles(ref_ids, 32, BM)
        n = int(f[6].item())
        assert n == r[3]
        np.testing.assert_array_equal(f[5][:n].cpu().numpy(), r[2])


def test_fused_graph_replays():
    inp = _random(16, 2880, 32, 4, True, 1.0, 8)
    T, E, k = inp["T"], inp["E"], inp["k"]
    BM = moe.pick_bm(T, k, E)
    x, wr, b = _router_inputs(inp)
    d = _router_inputs(_random(T, inp["H"], E, k, True, 0.3, 6))
    layer_ws = moe.zeroed_route_tiles_workspace(T, inp["H"], E, x.device)
    ref = moe.moe_route_tiles(x, wr, b, k, BM, workspace=layer_ws)
    torch.cuda.synchronize()
    ids = torch.empty_like(ref[0]); wts = torch.empty_like(ref[1])
    off = torch.empty_like(ref[3]); srt = torch.empty_like(ref[4])
    tiles = torch.empty_like(ref[5]); nt = torch.empty_like(ref[6])
    lib = moe.load()
    p = lambda t: None if t is None else __import__("ctypes").c_void_p(t.data_ptr())  # noqa: E731
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            st = lib.moe_route_tiles(p(x), p(wr), p(b), T, inp["H"], E, k, 0, BM, p(ids), p(wts),
                                     None, p(off), p(srt), p(tiles), p(nt), p(layer_ws),
                                     layer_ws.numel(),
                                     __import__("ctypes").c_void_p(stream.cuda_stream))
            assert st == 0
    torch.cuda.synchronize()
    for rep in range(4):
        log(f"fused graph replay {rep}")
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        n = int(nt.item())
        assert n == int(ref[6].item())
        for a, c in ((ids, ref[0]), (wts, ref[1]), (off, ref[3]), (srt, ref[4]),
                     (tiles[:n], ref[5][:n])):
            assert torch.equal(a, c), f"replay {rep}"
        # eager work between replays, on the same workspace
        moe.moe_route_tiles(d[0], d[1], d[2], k, BM, workspace=layer_ws)
        torch.cuda.synchronize()
        assert int(layer_ws[:256].count_nonzero().item()) == 0


@pytest.mark.parametrize("E,k", [(8, 2), (32, 4), (40, 4), (64, 8), (100, 4)])
def test_ties_on_every_routing_path(E, k):
    """Equal logits go to the lower expert on every path that selects: the
    unfused top-k (T > 16), the fused launch (one and several tokens) and the
    one-launch layer; up to 32 experts the rank count with two lanes per
    expert runs (and the one-launch layer's publishers count with the whole
    workgroup), at 40 and 64 experts the rank count with one lane per expert,
    at 100 the argmax rounds.  Rows of the router are duplicated in pairs, so
    every logit has a twin, and an all-zero router ties everything."""
    for zero in (False, True):
        inp = make_random(T=20, H=128, E=E, k=k, I=64, seed=E + k, router_std=0.5)
        wr = inp["w_router"]
        if zero:
            wr[:] = 0
        else:
            wr[1::2] = wr[0::2][: wr[1::2].shape[0]]
        x, wrd, _ = _router_inputs(inp)
        # logits by one elementwise product and sum per (token, expert), so
        # duplicated router rows give bitwise equal logits here as well
        xf = oracle.bf16_to_f64(inp["x"])
        L = (xf[:, None, :] * wr.astype(np.float64)[None, :, :]).sum(axis=2)
        ref_ids = oracle.top_k(L, k)
        ref_w = oracle.softmax_selected(L, ref_ids)
        if zero:
            assert np.all(ref_ids == np.arange(k))
        log(f"ties E={E} k={k} zero={zero}: moe_route at T=20")
        ids, wts, _ = moe.moe_route(x, wrd, None, k)
        np.testing.assert_array_equal(ids.cpu().numpy(), ref_ids)
        np.testing.assert_allclose(wts.cpu().numpy(), ref_w, rtol=0, atol=1e-6)
        for T in (1, 5, 20):
            log(f"ties E={E} k={k} zero={zero}: moe_route_tiles at T={T}")
            f = moe.moe_route_tiles(x[:T].contiguous(), wrd, None, k, moe.pick_bm(T, k, E))
            np.testing.assert_array_equal(f[0].cpu().numpy(), ref_ids[:T])
            np.testing.assert_allclose(f[1].cpu().numpy(), ref_w[:T], rtol=0, atol=1e-6)
        d = {key: torch.from_numpy(np.ascontiguousarray(inp[key])).cuda()
             for key in ("w13_q", "w13_s", "w2_q", "w2_s")}
        log(f"ties E={E} k={k} zero={zero}: one-launch layer")
        o = moe.moe_layer_one_token(x[:1].contiguous(), wrd, None, d["w13_q"], d["w13_s"],
                                    d["w2_q"], d["w2_s"], k, moe.pick_bm(1, k, E),
                                    layout="canonical")
        torch.cuda.synchronize()
        np.testing.assert_array_equal(o[1].cpu().numpy(), ref_ids[:1])
        np.testing.assert_allclose(o[2].cpu().numpy(), ref_w[:1], rtol=0, atol=1e-6)


@pytest.mark.parametrize("T", [2, 5, 16, 64])
def test_layer_output_with_one_launch_routing(T):
    """The whole layer with routing and tiles in one launch (moe_route_tiles:
    one tail workgroup up to 16 tokens, the relay at 64) gives the same
    output, bit for bit, as with moe_route + moe_build_tiles, and meets the
    oracle bar."""
    inp = make_random(T=T, H=512, E=32, k=4, I=512, seed=50 + T, router_bias=True,
                      router_std=0.3)
    d = to_device(inp)
    k, E = inp["k"], inp["E"]
    BM = moe.pick_bm(T, k, E)
    log(f"layer with one-launch routing T={T}")
    f = moe.moe_route_tiles(d["x"], d["w_router"], d["bias"], k, BM)
    out_f = moe.moe_forward(d["x"], d["w13_q"], d["w13_s"], d["w2_q"], d["w2_s"], f[1], f[4],
                            f[5], f[6], BM)
    log(f"layer with separate routing launches T={T}")
    ids, wts, _ = moe.moe_route(d["x"], d["w_router"], d["bias"], k)
    off, srt, tiles, nt = moe.moe_build_tiles(ids, E, BM)
    out_s = moe.moe_forward(d["x"], d["w13_q"], d["w13_s"], d["w2_q"], d["w2_s"], wts, srt,
                            tiles, nt, BM)
    torch.cuda.synchronize()
    assert torch.equal(out_f.view(torch.int16), out_s.view(torch.int16))
    log(f"layer with one-launch routing T={T}: oracle")
    r = oracle.moe_layer(inp, BM=BM)
    assert_out_close(out_f.float().cpu().numpy().astype(np.float64)[r["tokens"]], r["out"])
