"""Shared helpers of the GPU parity tests: move seeded inputs to the device,
run the library's three calls, and compare against the float64 oracle.

Parity bar (both from the layer's acceptance criteria):
  * bit-exact topk_ids, expert_offsets, sorted_ids, tiles and num_tiles;
  * topk_weights within 1e-6 absolute;
  * out (bf16) within relative L2 <= 5e-3 and max |diff| <= 2e-2 * max|oracle|.
The max-abs bound is read relative to the output's scale: outputs of these
layers reach ~2e3 in magnitude, where one bf16 ulp alone is 8.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import mxfp4_grouped_expert_amd as moe
import oracle

REL_L2 = 5e-3
MAX_REL = 2e-2
W_ATOL = 1e-6


def log(msg: str):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_device(inp: dict, dev="cuda") -> dict:
    d = {"x": torch.from_numpy(np.ascontiguousarray(inp["x"]).view(np.int16)).to(dev),
         "w_router": torch.from_numpy(np.ascontiguousarray(inp["w_router"])).to(dev),
         "bias": None if inp.get("bias") is None else torch.from_numpy(inp["bias"]).to(dev),
         "gating": inp.get("gating", "softmax")}
    for key in ("w13_q", "w13_s", "w2_q", "w2_s"):
        d[key] = torch.from_numpy(np.ascontiguousarray(inp[key])).to(dev)
    return d


def run_gpu(d: dict, k: int, BM: int) -> dict:
    E = d["w13_q"].shape[0]
    ids, wts, logits = moe.moe_route(d["x"], d["w_router"], d["bias"], k, want_logits=True,
                                     gating=d["gating"])
    off, srt, tiles, nt = moe.moe_build_tiles(ids, E, BM)
    out = moe.moe_forward(d["x"], d["w13_q"], d["w13_s"], d["w2_q"], d["w2_s"], wts, srt, tiles,
                          nt, BM)
    torch.cuda.synchronize()
    n = int(nt.item())
    return dict(topk_ids=ids.cpu().numpy(), topk_weights=wts.cpu().numpy(),
                logits=logits.cpu().numpy(), expert_offsets=off.cpu().numpy(),
                sorted_ids=srt.cpu().numpy(), tiles=tiles[:n].cpu().numpy(), num_tiles=n,
                out=out.float().cpu().numpy().astype(np.float64))


def out_errors(got: np.ndarray, want: np.ndarray):
    diff = got - want
    rel_l2 = float(np.linalg.norm(diff) / max(np.linalg.norm(want), 1e-300))
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    scale = float(np.abs(want).max()) if want.size else 0.0
    return rel_l2, max_abs, scale


def assert_routing_equal(g: dict, r: dict):
    np.testing.assert_array_equal(g["topk_ids"], r["topk_ids"])
    np.testing.assert_allclose(g["topk_weights"], r["topk_weights"], rtol=0, atol=W_ATOL)


def assert_tiles_equal(g: dict, r: dict):
    np.testing.assert_array_equal(g["expert_offsets"], r["expert_offsets"])
    np.testing.assert_array_equal(g["sorted_ids"], r["sorted_ids"])
    assert g["num_tiles"] == r["num_tiles"]
    np.testing.assert_array_equal(g["tiles"], r["tiles"])


def assert_out_close(got: np.ndarray, want: np.ndarray, what: str = "out"):
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    rel_l2, max_abs, scale = out_errors(got, want)
    log(f"{what}: {got.shape[0]} rows relL2={rel_l2:.3e} max_abs={max_abs:.3e} "
        f"max|ref|={scale:.3e} max/scale={max_abs / max(scale, 1e-300):.3e}")
    assert rel_l2 <= REL_L2, f"{what}: relative L2 {rel_l2:.3e} > {REL_L2}"
    assert max_abs <= MAX_REL * scale, f"{what}: max abs {max_abs:.3e} > {MAX_REL} * {scale:.3e}"


def progress_logger(what: str, every: int = 16):
    """An oracle progress callback that logs every `every` experts."""
    def cb(e, E):
        if (e + 1) % every == 0 or e + 1 == E:
            log(f"{what}: oracle expert {e + 1}/{E}")
    return cb


def oracle_layer(inp: dict, BM: int, tokens=None) -> dict:
    """oracle.moe_layer with progress lines (long at the 120b shapes)."""
    what = f"{inp.get('name', '?')} BM={BM}"
    log(f"{what}: oracle over {inp['T'] if tokens is None else len(tokens)} tokens")
    return oracle.moe_layer(inp, BM=BM, tokens=tokens, progress=progress_logger(what))


def check_all(inp: dict, BM: int, tokens=None, dev="cuda", ref=None) -> dict:
    """Run the GPU path on `inp` and hold every output to the parity bar
    (against `ref`, an oracle result for the same input and BM, when given)."""
    log(f"{inp.get('name', '?')} BM={BM}: upload")
    d = to_device(inp, dev)
    log(f"{inp.get('name', '?')} BM={BM}: run")
    g = run_gpu(d, inp["k"], BM)
    del d
    r = ref if ref is not None else oracle_layer(inp, BM, tokens)
    assert_routing_equal(g, r)
    assert_tiles_equal(g, r)
    sel = r["tokens"]
    assert_out_close(g["out"][sel], r["out"])
    return dict(gpu=g, ref=r)
