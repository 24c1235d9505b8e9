"""GPU: the gpt-oss expert form (moe_forward_gptoss, moe_deinterleave_rows)
against the float64 oracle.

The oracle evaluates the checkpoint's interleaved w13 rows and biases
directly; the library de-interleaves them once (moe_deinterleave_rows) and
runs every expert GEMM path with the biased, clamped SwiGLU epilogue: the
one-token down + combine, the row-tile decode kernels (one K chunk and
several), and the 128-row matrix-core kernels.  The form is the released
model's own definition, not the pages': parity here is against that
definition, and against a real checkpoint it is unpinned.
"""
import numpy as np
import pytest
import torch

import mxfp4_grouped_expert_amd as moe
import oracle
from moe_inputs import WORKLOADS, make_random, make_weights, make_workload, with_gptoss_experts

from gpu_helpers import (assert_out_close, assert_routing_equal, assert_tiles_equal, log,
                         oracle_layer, to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    moe.load()


def test_deinterleave_rows_matches_oracle_definition():
    inp = make_random(T=1, H=2880, E=3, k=1, I=96, seed=5)
    inp = with_gptoss_experts(inp, 5)
    for name, axis in (("w13_q", 1), ("w13_s", 1), ("b13", 1)):
        a = inp[name]
        got = moe.moe_deinterleave_rows(torch.from_numpy(a).cuda())
        torch.cuda.synchronize()
        want = oracle.concatenated_from_interleaved(a, axis=axis)
        log(f"deinterleave {name} {a.shape} {a.dtype}")
        np.testing.assert_array_equal(got.cpu().numpy(), want)


def run_gptoss(inp, BM, layout="canonical"):
    d = to_device(inp)
    k, E = inp["k"], inp["E"]
    ids, wts, _ = moe.moe_route(d["x"], d["w_router"], d["bias"], k, gating=d["gating"])
    off, srt, tiles, nt = moe.moe_build_tiles(ids, E, BM)
    q13 = moe.moe_deinterleave_rows(d["w13_q"])
    s13 = moe.moe_deinterleave_rows(d["w13_s"])
    b13 = None if inp["b13"] is None else moe.moe_deinterleave_rows(
        torch.from_numpy(inp["b13"]).cuda())
    b2 = None if inp["b2"] is None else torch.from_numpy(inp["b2"]).cuda()
    q2 = d["w2_q"]
    if layout == "blocked":
        q13, q2 = moe.moe_repack_weights(q13), moe.moe_repack_weights(q2)
    out = moe.moe_forward_gptoss(d["x"], q13, s13, q2, d["w2_s"], b13, b2, wts, srt, tiles, nt,
                                 BM, alpha=inp["alpha"], limit=inp["limit"], layout=layout)
    torch.cuda.synchronize()
    n = int(nt.item())
    return dict(topk_ids=ids.cpu().numpy(), topk_weights=wts.cpu().numpy(),
                expert_offsets=off.cpu().numpy(), sorted_ids=srt.cpu().numpy(),
                tiles=tiles[:n].cpu().numpy(), num_tiles=n,
                out=out.float().cpu().numpy().astype(np.float64))


GPTOSS_CASES = [
    # T, H, E, k, I, BM, note
    (1, 2880, 32, 4, 2880, 16, "one token: fused down + combine"),
    (1, 320, 6, 3, 224, 16, "one token, ragged K"),
    (5, 256, 8, 2, 512, 16, "decode row tiles"),
    (64, 2880, 33, 4, 512, 64, "decode, 4 blocks per workgroup"),
    (300, 160, 4, 2, 224, 128, "128-row matrix-core tiles, partial column blocks"),
    (512, 2880, 16, 2, 2880, 128, "matrix-core tiles at the gpt-oss width"),
    (70, 4096, 2, 1, 64, 128, "K > 3072: chunked gate/up"),
    (70, 64, 2, 1, 4096, 128, "K > 3072: chunked down"),
]


@pytest.mark.parametrize("case", GPTOSS_CASES, ids=lambda c: "T{}_H{}_E{}_k{}_I{}".format(*c[:5]))
def test_gptoss_form_matches_oracle(case):
    T, H, E, k, I, BM, note = case
    inp = make_random(T=T, H=H, E=E, k=k, I=I, seed=200 + T + E, router_std=0.3)
    inp = with_gptoss_experts(inp, T + I)
    log(f"gpt-oss form {inp['name']} BM={BM} ({note})")
    for layout in ("canonical", "blocked"):
        g = run_gptoss(inp, BM, layout)
        r = oracle.moe_layer(inp, BM=BM)
        assert_routing_equal(g, r)
        assert_tiles_equal(g, r)
        assert_out_close(g["out"], r["out"], f"gpt-oss {layout} ({note})")


def test_gptoss_form_without_biases_and_unclamped():
    inp = make_random(T=9, H=192, E=4, k=2, I=96, seed=7, router_std=0.3)
    inp = with_gptoss_experts(inp, 7)
    inp.update(b13=None, b2=None, limit=float("inf"), alpha=1.0)
    r_inp = dict(inp, b13=np.zeros((4, 192), np.float32), b2=np.zeros((4, 192), np.float32))
    g = run_gptoss(inp, 16)
    r = oracle.moe_layer(r_inp, BM=16)
    assert_out_close(g["out"], r["out"], "gpt-oss, no biases, no clamp")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("wid", [2, 4])
def test_gptoss_form_at_workload_shapes(wid):
    """The MoeLayer path (blocked weights) on the 20b T=64 and 120b T=4096
    shapes with gpt-oss biases, every token against the oracle."""
    inp = make_workload(wid, weights=False)
    w = WORKLOADS[wid]
    inp.update(make_weights(w.E, w.H, w.I, w.model_id))
    inp = with_gptoss_experts(inp, 100 + wid)
    d = to_device(inp)
    layer = moe.MoeLayer(d["w_router"], d["bias"], d["w13_q"], d["w13_s"], d["w2_q"], d["w2_s"],
                         inp["k"], activation="gptoss",
                         b13=torch.from_numpy(inp["b13"]).cuda(),
                         b2=torch.from_numpy(inp["b2"]).cuda()).plan(inp["T"])
    log(f"gpt-oss MoeLayer, workload {wid} (BM {layer.BM})")
    out = layer(d["x"]).float().cpu().numpy().astype(np.float64)
    ids = layer.topk_ids.cpu().numpy()
    del layer, d
    r = oracle_layer(inp, moe.pick_bm(inp["T"], inp["k"], inp["E"]))
    np.testing.assert_array_equal(ids, r["topk_ids"])
    assert len(r["tokens"]) == inp["T"]
    assert_out_close(out, r["out"], f"gpt-oss MoeLayer, workload {wid}")
