"""GPU: moe_forward_static_workspace (the allocation-free moe_forward) gives
the same bytes as moe_forward on consecutive calls of shrinking size, and
allocates no device memory from torch's side."""
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


def _routed(inp, d, BM):
    ids, wts, _ = moe.moe_route(d["x"], d["w_router"], d["bias"], inp["k"], gating=d["gating"])
    off, srt, tiles, nt = moe.moe_build_tiles(ids, inp["E"], BM)
    return wts, srt, tiles, nt


def test_static_workspace_equals_forward_on_calls_of_shrinking_size():
    cases = [make_workload(2),                                        # 256 slots, 20b shape
             make_random(T=5, H=256, E=8, k=2, I=512, seed=41),       # 10 slots
             make_random(T=1, H=320, E=6, k=3, I=224, seed=42)]       # one token
    for i, inp in enumerate(cases):
        T, k, E = inp["T"], inp["k"], inp["E"]
        BM = moe.pick_bm(T, k, E)
        d = to_device(inp)
        wts, srt, tiles, nt = _routed(inp, d, BM)
        for layout in ("canonical", "blocked"):
            q13, q2 = d["w13_q"], d["w2_q"]
            if layout == "blocked":
                q13, q2 = moe.moe_repack_weights(q13), moe.moe_repack_weights(q2)
            want = moe.moe_forward(d["x"], q13, d["w13_s"], q2, d["w2_s"], wts, srt, tiles, nt,
                                   BM, layout=layout)
            out = torch.full_like(want, float("nan"))
            torch.cuda.synchronize()
            before = torch.cuda.memory_stats()["allocation.all.allocated"]
            log(f"static workspace call {i} ({inp['name']}, {layout})")
            moe.moe_forward_static_workspace(d["x"], q13, d["w13_s"], q2, d["w2_s"], wts, srt,
                                             tiles, nt, BM, out, layout=layout)
            torch.cuda.synchronize()
            assert torch.cuda.memory_stats()["allocation.all.allocated"] == before
            assert torch.equal(out.view(torch.int16), want.view(torch.int16)), \
                f"call {i} ({layout}): differs from moe_forward"
        if T * E <= 64:
            ref = oracle.moe_layer(inp, BM=BM)
            assert_out_close(out.float().cpu().numpy().astype(np.float64), ref["out"],
                             f"static workspace, {inp['name']}")


def test_static_workspace_rejects_oversized_batches():
    inp = make_random(T=971, H=2880, E=1, k=1, I=2880, seed=43)
    d = to_device(inp)
    BM = 128
    wts, srt, tiles, nt = _routed(inp, d, BM)
    out = torch.empty((971, 2880), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError, match="MOE_ERR_WORKSPACE"):
        moe.moe_forward_static_workspace(d["x"], d["w13_q"], d["w13_s"], d["w2_q"], d["w2_s"],
                                         wts, srt, tiles, nt, BM, out)
