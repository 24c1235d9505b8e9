"""GPU parity: the HIP library against the float64 oracle (needs a gfx950 GPU).

Covers the five gpt-oss-shaped workloads (tiny; 20b decode T=1; 20b decode
T=64 with a skewed router; 120b decode T=64; 120b prefill T=4096), every
token of each, small random shapes with ragged K-block counts and
multi-chunk tile scatters, a constructed routing that gives the 128-row
matrix-core kernel every fragment count, and the method's degenerate
cases.
"""
import numpy as np
import pytest
import torch

import mxfp4_grouped_expert_amd as moe
import oracle
from moe_inputs import (identical_experts, make_activations, make_random, make_weights,
                        make_workload, WORKLOADS)

from gpu_helpers import (assert_out_close, assert_routing_equal, assert_tiles_equal, check_all,
                         log, oracle_layer, run_gpu, to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    moe.load()  # fails loudly if the HIP library is missing


@pytest.fixture(scope="module")
def w120b():
    w = WORKLOADS[3]
    return make_weights(w.E, w.H, w.I, w.model_id)


# Oracle results over every token of a workload, by (workload, BM): the
# separate-launch test and the benchmark-configuration test of a workload
# compare against the same float64 result.  At the 120b shapes the oracle's
# cost is dominated by decoding each expert once (about 40 s for all 128),
# not by the number of tokens, so every token is compared.
_ORACLE = {}


def full_oracle(inp: dict, BM: int) -> dict:
    key = (inp["wid"], BM)
    if key not in _ORACLE:
        r = oracle_layer(inp, BM)
        r.pop("y")  # [T*k, H] float64: not needed after the combine
        _ORACLE[key] = r
    return _ORACLE[key]


def workload_input(wid: int, w120b) -> dict:
    inp = make_workload(wid, weights=wid < 3)
    if wid >= 3:
        inp.update(w120b)
    return inp


# ------------------------------------------------------------- workloads --

@pytest.mark.parametrize("BM", [16, 32, 64, 128])
def test_tiny_workload(BM):
    check_all(make_workload(0), BM)


@pytest.mark.parametrize("wid", [1, 2])
def test_gptoss20b_decode(wid):
    inp = make_workload(wid)
    BM = moe.pick_bm(inp["T"], inp["k"], inp["E"])
    check_all(inp, BM, ref=full_oracle(inp, BM))


@pytest.mark.timeout(600)
def test_gptoss120b_decode_T64(w120b):
    inp = workload_input(3, w120b)
    BM = moe.pick_bm(inp["T"], inp["k"], inp["E"])
    res = check_all(inp, BM, ref=full_oracle(inp, BM))
    assert len(res["ref"]["tokens"]) == inp["T"]


@pytest.mark.timeout(600)
def test_gptoss120b_prefill_T4096(w120b):
    inp = workload_input(4, w120b)
    BM = moe.pick_bm(inp["T"], inp["k"], inp["E"])
    res = check_all(inp, BM, ref=full_oracle(inp, BM))
    # every token is compared, so every (expert, tile) pair of the table and
    # every row of each partial tile is checked
    assert len(res["ref"]["tokens"]) == inp["T"]
    tiles = res["ref"]["tiles"]
    log(f"prefill: {len(tiles)} tiles, {int((tiles[:, 2] < BM).sum())} partial, rows "
        f"{int(tiles[:, 2].min())}..{int(tiles[:, 2].max())}")
    ids = res["gpu"]["topk_ids"]
    assert all(len(set(r)) == inp["k"] for r in ids)
    assert sorted(res["gpu"]["sorted_ids"].tolist()) == list(range(inp["T"] * inp["k"]))


# The benchmark's own configuration: MoeLayer with its default plan (the
# weights repacked into the blocked layout, the single launch at T = 1, the
# fused routing up to 16 tokens), one call per workload, against the oracle
# over every token.
@pytest.mark.timeout(600)
@pytest.mark.parametrize("wid", [1, 2, 3, 4])
def test_bench_configuration_matches_oracle(wid, w120b):
    inp = workload_input(wid, w120b)
    d = to_device(inp)
    layer = moe.MoeLayer(d["w_router"], d["bias"], d["w13_q"], d["w13_s"], d["w2_q"], d["w2_s"],
                         inp["k"], gating=inp["gating"]).plan(inp["T"])
    log(f"bench configuration, workload {wid}: MoeLayer (layout blocked, BM {layer.BM})")
    out = layer(d["x"]).float().cpu().numpy().astype(np.float64)
    ids = layer.topk_ids.cpu().numpy()
    wts = layer.topk_weights.cpu().numpy()
    del layer, d
    r = full_oracle(inp, moe.pick_bm(inp["T"], inp["k"], inp["E"]))
    np.testing.assert_array_equal(ids, r["topk_ids"])
    np.testing.assert_allclose(wts, r["topk_weights"], rtol=0, atol=1e-6)
    assert len(r["tokens"]) == inp["T"]
    assert_out_close(out, r["out"], f"bench configuration, workload {wid}")


# Constructed routing for the 128-row matrix-core kernel: expert loads chosen
# so that the tiles hold every fragment count 1..8 (rows 1..128, with both
# parities of the split between a SIMD's two waves), full tiles followed by
# remainders, and a 256-row expert; partial column blocks on both GEMMs (I =
# 320: 192 + 128 gate/up columns; H = 256 of a 384-column down unit) and
# ragged K (5 stages of 64 on the down side).  The oracle side is composed of
# the oracle's own steps (tile table, per-expert FFN, combine).
MMA_COUNTS = [1, 16, 17, 33, 48, 49, 65, 80, 81, 96, 97, 112, 113, 127, 128, 129, 160, 256]


def test_mma_kernel_every_fragment_count():
    E, k, H, I = len(MMA_COUNTS), 2, 256, 320
    flat_sorted = np.repeat(np.arange(E, dtype=np.int32), MMA_COUNTS)
    N = flat_sorted.size
    assert N % k == 0 and max(MMA_COUNTS) <= N // k
    T = N // k
    ids = np.stack([flat_sorted[:T], flat_sorted[T:]], axis=1)  # distinct per token
    assert np.all(ids[:, 0] != ids[:, 1])
    rng = np.random.default_rng(2024)
    w = rng.uniform(0.1, 1.0, size=(T, k))
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    inp = make_random(T=T, H=H, E=E, k=k, I=I, seed=909)
    BM = 128
    assert T * k >= 32 * E  # the launchers pick the matrix-core kernel
    d = to_device(inp)
    ids_d = torch.from_numpy(ids.astype(np.int32)).cuda()
    off, srt, tiles, nt = moe.moe_build_tiles(ids_d, E, BM)
    for layout in ("canonical", "blocked"):
        if layout == "blocked":
            q13, q2 = moe.moe_repack_weights(d["w13_q"]), moe.moe_repack_weights(d["w2_q"])
        else:
            q13, q2 = d["w13_q"], d["w2_q"]
        log(f"matrix-core fragments, layout {layout}")
        out = moe.moe_forward(d["x"], q13, d["w13_s"], q2, d["w2_s"],
                              torch.from_numpy(w).cuda(), srt, tiles, nt, BM, layout=layout)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
        r_off, r_srt, r_tiles, r_n = oracle.build_tiles(ids, E, BM)
        assert int(nt.item()) == r_n
        np.testing.assert_array_equal(tiles[:r_n].cpu().numpy(), r_tiles)
        np.testing.assert_array_equal(srt.cpu().numpy(), r_srt)
        rows = r_tiles[:, 2]
        assert set(((rows + 15) // 16).tolist()) == set(range(1, 9))
        x64 = oracle.bf16_to_f64(inp["x"])
        y = np.zeros((T * k, H))
        for e in range(E):
            slots = r_srt[r_off[e]:r_off[e + 1]].astype(np.int64)
            y[slots] = oracle.expert_ffn(x64[slots // k], inp["w13_q"][e], inp["w13_s"][e],
                                         inp["w2_q"][e], inp["w2_s"][e])
        want = oracle.combine(y, w.astype(np.float64))
        assert_out_close(got, want, f"matrix-core fragments ({layout})")


@pytest.mark.parametrize("BM", [16, 32, 64, 128])
def test_tile_table_all_bm_at_prefill(w120b, BM):
    inp = make_workload(4, weights=False)
    log(f"prefill tile table BM={BM}")
    d = {"x": torch.from_numpy(inp["x"].view(np.int16)).cuda(),
         "w_router": torch.from_numpy(inp["w_router"]).cuda()}
    ids, wts, _ = moe.moe_route(d["x"], d["w_router"], None, inp["k"])
    off, srt, tiles, nt = moe.moe_build_tiles(ids, inp["E"], BM)
    torch.cuda.synchronize()
    ref = oracle.build_tiles(ids.cpu().numpy(), inp["E"], BM)
    n = int(nt.item())
    assert n == ref[3]
    np.testing.assert_array_equal(off.cpu().numpy(), ref[0])
    np.testing.assert_array_equal(srt.cpu().numpy(), ref[1])
    np.testing.assert_array_equal(tiles[:n].cpu().numpy(), ref[2])


# Many slots: the table is built by several workgroups, each scattering one
# range of the slots (the 16,384-slot prefill above takes 8 of them).  A
# slot count whose last range is short (100,008 slots, 49 ranges), one whose
# last workgroup gets no slots at all (160,000 slots over 64 workgroups of
# 2,560), the smallest split (4,097 slots, 3 ranges), skewed expert loads,
# and the largest expert count and top-k.
@pytest.mark.parametrize("T,k,E,BM", [(12_501, 8, 256, 128), (40_000, 4, 128, 64),
                                      (4_097, 1, 3, 16)])
def test_tile_table_many_slots(T, k, E, BM):
    rng = np.random.default_rng(T + E)
    keys = rng.random((T, E)) + np.linspace(0.0, 0.6, E)[None, :]  # skewed toward high ids
    ids_np = np.argsort(-keys, axis=1, kind="stable")[:, :k].astype(np.int32)
    log(f"tile table T={T} k={k} E={E} BM={BM} ({T * k} slots)")
    ids = torch.from_numpy(ids_np).cuda()
    off, srt, tiles, nt = moe.moe_build_tiles(ids, E, BM)
    torch.cuda.synchronize()
    ref = oracle.build_tiles(ids_np, E, BM)
    n = int(nt.item())
    assert n == ref[3]
    np.testing.assert_array_equal(off.cpu().numpy(), ref[0])
    np.testing.assert_array_equal(srt.cpu().numpy(), ref[1])
    np.testing.assert_array_equal(tiles[:n].cpu().numpy(), ref[2])


# Ids outside [0, E) are dropped from the counts and tiles and their slots
# placed after expert_offsets[E] (the library's contract for a corrupted
# routing; the method itself never produces them).  One case per builder:
# all-pairs (<= 128 slots), one workgroup, and the scatter split over
# workgroups.  Expected values: counts of the valid ids, a stable argsort of
# the bucket (invalid ids last), and the oracle's tiles of the valid ids.
@pytest.mark.parametrize("T,k,E,BM", [(50, 2, 8, 16), (300, 4, 32, 64), (2_500, 4, 128, 128)])
def test_tile_table_drops_out_of_range_ids(T, k, E, BM):
    rng = np.random.default_rng(7 * T + E)
    ids_np = rng.integers(0, E, (T, k)).astype(np.int32)
    bad = rng.random((T, k)) < 0.05
    ids_np[bad] = rng.choice(np.array([-1, E, E + 7, -1000], dtype=np.int32), int(bad.sum()))
    log(f"tile table with {int(bad.sum())} out-of-range ids, {T * k} slots")
    ids = torch.from_numpy(ids_np).cuda()
    off, srt, tiles, nt = moe.moe_build_tiles(ids, E, BM)
    torch.cuda.synchronize()
    flat = ids_np.ravel()
    valid = (flat >= 0) & (flat < E)
    nv = int(valid.sum())
    want_off = np.concatenate([[0], np.cumsum(np.bincount(flat[valid], minlength=E))])
    np.testing.assert_array_equal(off.cpu().numpy(), want_off)
    bucket = np.where(valid, flat, E)
    np.testing.assert_array_equal(srt.cpu().numpy(), np.argsort(bucket, kind="stable"))
    ref = oracle.build_tiles(flat[valid], E, BM)
    n = int(nt.item())
    assert n == ref[3] and want_off[E] == nv
    np.testing.assert_array_equal(tiles[:n].cpu().numpy(), ref[2])


# ------------------------------------------------------ random / ragged --

RANDOM_CASES = [
    # T, H, E, k, I, bias, router_std, BM
    (1, 64, 1, 1, 32, False, 0.02, 16),
    (3, 96, 2, 2, 160, True, 0.3, 16),
    (17, 544, 8, 4, 96, False, 0.3, 16),     # 17 K-blocks: ragged last step
    (64, 256, 33, 4, 512, True, 0.3, 16),
    (257, 128, 8, 2, 64, False, 0.5, 64),    # several M-blocks per tile
    (700, 64, 33, 2, 32, True, 0.5, 32),     # tile scatter over 2 chunks
    (4100, 32, 256, 8, 32, False, 1.0, 128), # E and k at their maxima, 33 chunks
    (40, 2880, 4, 4, 64, False, 0.02, 32),   # k = E: every expert used
    # large token tiles (128-row MFMA kernel): two tiles per expert, a K tail
    # (5 MX blocks), partial column blocks (224 and 160 outputs)
    (300, 160, 4, 2, 224, False, 0.3, 128),
    (512, 2880, 16, 2, 2880, True, 0.5, 128),
    (160, 96, 2, 1, 32, False, 0.3, 128),
    # the largest H and I the library accepts (65536): 22 K chunks of 3072
    # with a ragged last one, on the gate/up and on the down GEMM
    (3, 65536, 2, 2, 64, False, 0.02, 16),
    (3, 64, 2, 1, 65536, True, 0.3, 16),
    # K > 3072 with three 16-row passes per tile: two passes share each
    # chunk's weights, the third runs alone (gate/up side, then down side;
    # K = 4160 is past the 128-row kernel's scale slab)
    (70, 4160, 2, 1, 64, False, 0.3, 128),
    (70, 64, 2, 1, 4160, False, 0.3, 128),
    # the 128-row matrix-core kernel past K = 3072: K = 4096 on the gate/up
    # side (a partial column block of 32 outputs), K = 3584 on the down side
    # and K = 3136 (98 MX blocks: scale runs not 16-byte aligned) on gate/up
    (200, 4096, 4, 2, 224, False, 0.3, 128),
    (150, 3136, 4, 2, 3584, True, 0.5, 128),
]


@pytest.mark.parametrize("case", RANDOM_CASES, ids=lambda c: "T{}_H{}_E{}_k{}_I{}".format(*c[:5]))
def test_random_shapes(case):
    T, H, E, k, I, bias, std, BM = case
    inp = make_random(T=T, H=H, E=E, k=k, I=I, seed=T + H + E, router_bias=bias, router_std=std)
    check_all(inp, BM)


# Many tokens: router logits on the fp64 matrix cores (16-token workgroups,
# up to 128 experts).  A ragged last token block, an expert count that is not
# a multiple of 16, and the full 2880-wide hidden size.
ROUTER_MANY_CASES = [
    # T, H, E, k
    (1029, 2880, 128, 4),
    (1040, 160, 72, 4),
    (2048, 64, 5, 2),
]


@pytest.mark.parametrize("case", ROUTER_MANY_CASES, ids=lambda c: "T{}_H{}_E{}".format(*c[:3]))
def test_router_many_tokens_match_oracle(case):
    T, H, E, k = case
    inp = make_random(T=T, H=H, E=E, k=k, I=32, seed=T + E, router_std=0.3)
    inp["name"] = "router_many_T{}_E{}".format(T, E)
    res = check_all(inp, 128, tokens=np.arange(0, T, 97))
    ref = oracle.router_logits(inp["x"], inp["w_router"], None)
    np.testing.assert_allclose(res["gpu"]["logits"], ref, rtol=1e-13, atol=1e-12)


def test_wide_scale_range():
    T, H, E, k, I = 9, 192, 4, 2, 96
    inp = make_random(T=T, H=H, E=E, k=k, I=I, seed=5, router_std=0.3)
    inp.update(make_weights(E, H, I, 77, scale_lo=112, scale_hi=134))
    inp["name"] = "wide_scales_112_134"
    check_all(inp, 16)


# ------------------------------------------------------ degenerate cases --

def test_zero_tokens_is_a_noop():
    inp = make_random(T=1, H=64, E=4, k=2, I=32, seed=1)
    d = to_device(inp)
    x0 = d["x"][:0]
    ids, wts, _ = moe.moe_route(x0, d["w_router"], None, 2)
    off, srt, tiles, nt = moe.moe_build_tiles(ids, 4, 16)
    out = moe.moe_forward(x0, d["w13_q"], d["w13_s"], d["w2_q"], d["w2_s"], wts, srt, tiles, nt,
                          16)
    torch.cuda.synchronize()
    assert out.shape == (0, 64) and ids.shape == (0, 2)


def test_all_zero_router_ties_go_to_lower_experts():
    inp = make_random(T=5, H=64, E=6, k=3, I=32, seed=2)
    inp["w_router"] = np.zeros_like(inp["w_router"])
    inp["name"] = "zero_router"
    res = check_all(inp, 16)
    assert np.all(res["gpu"]["topk_ids"] == np.arange(3))
    np.testing.assert_allclose(res["gpu"]["topk_weights"], 1 / 3, rtol=0, atol=1e-7)


def test_identical_experts_output_independent_of_routing():
    inp = identical_experts(make_random(T=12, H=128, E=5, k=2, I=64, seed=3, router_std=0.5))
    inp["name"] = "identical_experts"
    res = check_all(inp, 16)
    one = make_random(T=12, H=128, E=5, k=2, I=64, seed=3, router_std=0.5)
    one = identical_experts(one)
    one["w_router"] = np.zeros_like(one["w_router"])
    one["name"] = "identical_experts_zero_router"
    res2 = check_all(one, 16)
    assert_out_close(res["gpu"]["out"], res2["ref"]["out"], "identical experts vs fixed routing")


def test_single_expert_k1():
    check_all(make_random(T=33, H=96, E=1, k=1, I=64, seed=4), 16)


def test_deterministic_bitwise():
    inp = make_workload(2)
    d = to_device(inp)
    log("determinism: two runs of the 20b T=64 layer")
    a = run_gpu(d, inp["k"], 16)
    b = run_gpu(d, inp["k"], 16)
    for key in ("topk_ids", "topk_weights", "logits", "sorted_ids", "tiles", "out"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)


def test_logits_match_oracle_in_fp64():
    inp = make_workload(2, weights=False)
    d = {"x": torch.from_numpy(inp["x"].view(np.int16)).cuda(),
         "w_router": torch.from_numpy(inp["w_router"]).cuda(),
         "bias": torch.from_numpy(inp["bias"]).cuda()}
    log("router logits vs float64")
    _, _, logits = moe.moe_route(d["x"], d["w_router"], d["bias"], inp["k"], want_logits=True)
    ref = oracle.router_logits(inp["x"], inp["w_router"], inp["bias"])
    np.testing.assert_allclose(logits.cpu().numpy(), ref, rtol=0, atol=1e-12)
