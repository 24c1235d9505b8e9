"""The C-ABI library loads, exports every declared entry point, and rejects bad
arguments on the host before touching a device (CPU only: no compute calls).

Pointer arguments here are fake addresses; every call below must return an
error status during host validation, so nothing is ever dereferenced.
"""
import ctypes
import os
import re

import pytest

import mxfp4_grouped_expert_amd as moe
from mxfp4_grouped_expert_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mxfp4.h")

OK, NULL, SHAPE, ALIGN, WORKSPACE, DEVICE, OVERLAP = 0, 1, 2, 3, 4, 5, 7
P = 0x10000          # fake, 16-byte aligned "device" address (never dereferenced)
PMIS = 0x10004       # misaligned


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = B.load()
    names = _declared_functions()
    assert {"moe_route", "moe_build_tiles", "moe_forward"} <= set(names)
    for name in names:
        assert hasattr(lib, name), f"{name} declared in moe_mxfp4.h but not exported"


def test_status_strings_and_version():
    for s in range(8):
        assert moe.status_string(s).startswith("MOE_")
    assert "unknown" in moe.status_string(99)
    assert re.match(r"\d+\.\d+\.\d+", moe.version())


@pytest.mark.parametrize("T,k,E,want", [(1, 4, 32, 16), (16, 4, 32, 16), (17, 4, 32, 32),
                                        (64, 4, 32, 64), (64, 4, 128, 64), (65, 4, 128, 128),
                                        (4096, 4, 128, 128), (0, 4, 8, 16)])
def test_pick_bm_rule(T, k, E, want):
    # the smallest of 16/32/64/128 that is >= T
    assert moe.pick_bm(T, k, E) == want


@pytest.mark.parametrize("T,k,E,BM", [(1, 4, 32, 16), (64, 4, 128, 16), (4096, 4, 128, 64),
                                      (3, 2, 100, 128), (1000, 8, 3, 16)])
def test_tiles_max_is_a_tight_bound(T, k, E, BM):
    n = T * k
    tm = moe.tiles_max(T, k, E, BM)
    assert tm == min(n, -(-n // BM) + min(E, n))
    # worst case over routings: spread n slots over min(E, n) experts so each
    # has c mod BM == 1 where possible; sum of ceil(c/BM) never exceeds tm
    used = min(E, n)
    counts = [n // used + (1 if i < n % used else 0) for i in range(used)]
    assert sum(-(-c // BM) for c in counts) <= tm


def test_workspace_sizes():
    assert moe.forward_workspace_bytes(4096, 2880, 2880, 4) == (
        -(-4096 * 4 * 2880 * 2 // 256) * 256 + -(-4096 * 4 * 2880 * 4 // 256) * 256)
    assert moe.forward_workspace_bytes(0, 2880, 2880, 4) == 0
    assert moe.route_workspace_bytes(0, 2880, 32) == 0
    rb = moe.route_workspace_bytes(64, 2880, 128)
    assert rb >= 64 * 128 * 8 and rb % 256 == 0


def _route(**kw):
    a = dict(x=P, w=P, bias=None, T=4, H=256, E=8, k=2, gating=0, ids=P, wts=P, logits=None,
             ws=P, wsb=1 << 20)
    a.update(kw)
    lib = B.load()
    return lib.moe_route(a["x"], a["w"], a["bias"], a["T"], a["H"], a["E"], a["k"], a["gating"],
                         a["ids"], a["wts"], a["logits"], a["ws"], a["wsb"], None)


def _tiles(**kw):
    a = dict(ids=P, T=4, k=2, E=8, BM=16, off=P, srt=P, tiles=P, nt=P)
    a.update(kw)
    return B.load().moe_build_tiles(a["ids"], a["T"], a["k"], a["E"], a["BM"], a["off"],
                                    a["srt"], a["tiles"], a["nt"], None)


def _forward(**kw):
    a = dict(x=P, q13=P, s13=P, q2=P, s2=P, w=P, srt=P, tiles=P, nt=P, T=4, H=256, I=512, E=8,
             k=2, BM=16, layout=0, ws=P, wsb=1 << 30, out=P)
    a.update(kw)
    return B.load().moe_forward(a["x"], a["q13"], a["s13"], a["q2"], a["s2"], a["w"], a["srt"],
                                a["tiles"], a["nt"], a["T"], a["H"], a["I"], a["E"], a["k"],
                                a["BM"], a["layout"], a["ws"], a["wsb"], a["out"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(x=None), NULL), (dict(w=None), NULL), (dict(ids=None), NULL), (dict(ws=None), NULL),
    (dict(H=100), SHAPE), (dict(H=0), SHAPE), (dict(E=0), SHAPE), (dict(E=257), SHAPE),
    (dict(k=0), SHAPE), (dict(k=9, E=16), SHAPE), (dict(k=9, E=8), SHAPE), (dict(T=-1), SHAPE),
    (dict(H=65536 + 32), SHAPE), (dict(x=PMIS), ALIGN), (dict(w=PMIS), ALIGN),
    (dict(wsb=0), WORKSPACE), (dict(T=0, x=None), OK), (dict(gating=2), SHAPE),
    (dict(gating=-1), SHAPE),
])
def test_route_validation(kw, want):
    assert _route(**kw) == want


@pytest.mark.parametrize("kw,want", [
    (dict(ids=None), NULL), (dict(srt=None), NULL), (dict(tiles=None), NULL), (dict(nt=None), NULL),
    (dict(BM=8), SHAPE), (dict(BM=256), SHAPE), (dict(E=0), SHAPE), (dict(k=0), SHAPE),
    (dict(T=1 << 29, k=4), SHAPE), (dict(T=0, ids=None), OK),
])
def test_build_tiles_validation(kw, want):
    assert _tiles(**kw) == want


@pytest.mark.parametrize("kw,want", [
    (dict(x=None), NULL), (dict(q13=None), NULL), (dict(s2=None), NULL), (dict(ws=None), NULL),
    (dict(out=None), NULL), (dict(nt=None), NULL),
    (dict(H=100), SHAPE), (dict(I=48), SHAPE), (dict(k=3, E=2), SHAPE), (dict(BM=24), SHAPE),
    (dict(q13=PMIS), ALIGN), (dict(s13=PMIS), ALIGN), (dict(s2=PMIS), ALIGN),
    (dict(ws=PMIS), ALIGN), (dict(wsb=1000), WORKSPACE), (dict(T=0, x=None), OK),
    (dict(layout=2), SHAPE), (dict(layout=-1), SHAPE),
])
def test_forward_validation(kw, want):
    assert _forward(**kw) == want


def _forward_static(**kw):
    a = dict(x=P, q13=P, s13=P, q2=P, s2=P, wts=P, srt=P, tiles=P, nt=P, T=4, H=256, I=512, E=8,
             k=2, BM=16, layout=0, out=P)
    a.update(kw)
    return B.load().moe_forward_static_workspace(
        a["x"], a["q13"], a["s13"], a["q2"], a["s2"], a["wts"], a["srt"], a["tiles"], a["nt"],
        a["T"], a["H"], a["I"], a["E"], a["k"], a["BM"], a["layout"], a["out"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(x=None), NULL), (dict(q13=None), NULL), (dict(out=None), NULL), (dict(nt=None), NULL),
    (dict(H=100), SHAPE), (dict(BM=24), SHAPE), (dict(layout=2), SHAPE), (dict(s2=PMIS), ALIGN),
    (dict(T=0, x=None), OK),
    # h bf16 + y fp32 of every slot must fit the library's 16 MiB array:
    # 970 slots of 2880 x 2880 fit, 971 do not
    (dict(T=971, k=1, E=1, H=2880, I=2880, BM=128), WORKSPACE),
    (dict(T=4096, k=4, E=128, H=2880, I=2880, BM=128), WORKSPACE),
])
def test_forward_static_workspace_validation(kw, want):
    assert _forward_static(**kw) == want


def test_static_workspace_limit_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define MOE_STATIC_WORKSPACE_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == moe.STATIC_WORKSPACE_BYTES
    assert moe.forward_workspace_bytes(970, 2880, 2880, 1) <= moe.STATIC_WORKSPACE_BYTES
    assert moe.forward_workspace_bytes(971, 2880, 2880, 1) > moe.STATIC_WORKSPACE_BYTES


def _forward_gptoss(**kw):
    a = dict(x=P, q13=P, s13=P, q2=P, s2=P, b13=P, b2=None, alpha=1.702, limit=7.0, wts=P, srt=P,
             tiles=P, nt=P, T=4, H=256, I=512, E=8, k=2, BM=16, layout=0, ws=P, wsb=1 << 30, out=P)
    a.update(kw)
    return B.load().moe_forward_gptoss(
        a["x"], a["q13"], a["s13"], a["q2"], a["s2"], a["b13"], a["b2"], a["alpha"], a["limit"],
        a["wts"], a["srt"], a["tiles"], a["nt"], a["T"], a["H"], a["I"], a["E"], a["k"], a["BM"],
        a["layout"], a["ws"], a["wsb"], a["out"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(x=None), NULL), (dict(ws=None), NULL), (dict(out=None), NULL),
    (dict(H=100), SHAPE), (dict(BM=24), SHAPE), (dict(layout=2), SHAPE),
    (dict(alpha=float("nan")), SHAPE), (dict(alpha=float("inf")), SHAPE),
    (dict(limit=0.0), SHAPE), (dict(limit=-1.0), SHAPE), (dict(limit=float("nan")), SHAPE),
    (dict(q13=PMIS), ALIGN), (dict(wsb=1000), WORKSPACE), (dict(T=0, x=None), OK),
])
def test_forward_gptoss_validation(kw, want):
    assert _forward_gptoss(**kw) == want


@pytest.mark.parametrize("args,want", [
    ((P, 0, 4, 16, P + (1 << 20)), SHAPE), ((P, 2, 0, 16, P + (1 << 20)), SHAPE),
    ((P, 2, 4, 0, P + (1 << 20)), SHAPE), ((None, 2, 4, 16, P), NULL),
    ((P, 2, 4, 16, None), NULL), ((P, 2, 4, 16, P + 64), OVERLAP),
])
def test_deinterleave_rows_validation(args, want):
    assert B.load().moe_deinterleave_rows(*args, None) == want


def _route_tiles(**kw):
    a = dict(x=P, w=P, bias=None, T=4, H=256, E=8, k=2, gating=0, BM=16, ids=P, wts=P,
             logits=None, off=P, srt=P, tiles=P, nt=P, ws=P, wsb=1 << 20)
    a.update(kw)
    return B.load().moe_route_tiles(a["x"], a["w"], a["bias"], a["T"], a["H"], a["E"], a["k"],
                                    a["gating"], a["BM"], a["ids"], a["wts"], a["logits"],
                                    a["off"], a["srt"], a["tiles"], a["nt"], a["ws"], a["wsb"],
                                    None)


@pytest.mark.parametrize("kw,want", [
    (dict(x=None), NULL), (dict(tiles=None), NULL), (dict(ws=None), NULL), (dict(nt=None), NULL),
    (dict(T=65, E=128), SHAPE), (dict(T=1000, k=4, E=8), SHAPE), (dict(BM=8), SHAPE),
    (dict(H=48), SHAPE), (dict(x=PMIS), ALIGN), (dict(wsb=16), WORKSPACE), (dict(T=0, x=None), OK),
    (dict(gating=7), SHAPE),
])
def test_route_tiles_validation(kw, want):
    assert _route_tiles(**kw) == want


def test_route_tiles_limits_and_workspace():
    assert moe.route_tiles_ok(64, 256, 8) and not moe.route_tiles_ok(65, 8, 1)
    assert moe.route_tiles_workspace_bytes(1, 2880, 32) >= 256 + moe.route_workspace_bytes(1, 2880, 32) - 256


def _steps(which, **kw):
    a = dict(x=P, q=P, s=P, srt=P, tiles=P, nt=P, T=4, H=256, I=512, E=8, k=2, BM=16, layout=1,
             o=P, w=P)
    a.update(kw)
    lib = B.load()
    if which == "gateup":
        return lib.moe_gateup_swiglu(a["x"], a["q"], a["s"], a["srt"], a["tiles"], a["nt"], a["T"],
                                     a["H"], a["I"], a["E"], a["k"], a["BM"], a["layout"], a["o"],
                                     None)
    if which == "down":
        return lib.moe_down(a["x"], a["q"], a["s"], a["srt"], a["tiles"], a["nt"], a["T"], a["H"],
                            a["I"], a["E"], a["k"], a["BM"], a["layout"], a["o"], None)
    return lib.moe_combine(a["x"], a["w"], a["T"], a["H"], a["k"], a["o"], None)


@pytest.mark.parametrize("which", ["gateup", "down", "combine"])
@pytest.mark.parametrize("kw,want", [
    (dict(x=None), NULL), (dict(o=None), NULL), (dict(H=48), SHAPE), (dict(k=0), SHAPE),
    (dict(x=PMIS), ALIGN), (dict(s=PMIS), ALIGN), (dict(T=0, x=None), OK),
    (dict(layout=3), SHAPE),
])
def test_step_entry_points_validation(which, kw, want):
    if which == "combine" and ("s" in kw or "layout" in kw):
        pytest.skip("moe_combine takes no weights")
    assert _steps(which, **kw) == want


def _one_token(**kw):
    a = dict(x=P, w=P, bias=None, q13=P, s13=P, q2=P, s2=P, H=256, I=512, E=8, k=2, gating=0,
             layout=1, ids=P, wts=P, logits=None, off=P, srt=P, tiles=P, nt=P, ws=P,
             wsb=1 << 24, out=P)
    a.update(kw)
    return B.load().moe_layer_one_token(a["x"], a["w"], a["bias"], a["q13"], a["s13"], a["q2"],
                                        a["s2"], a["H"], a["I"], a["E"], a["k"], a["gating"],
                                        a["layout"], a["ids"], a["wts"], a["logits"], a["off"],
                                        a["srt"], a["tiles"], a["nt"], a["ws"], a["wsb"],
                                        a["out"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(x=None), NULL), (dict(q2=None), NULL), (dict(ws=None), NULL), (dict(out=None), NULL),
    (dict(H=48), SHAPE), (dict(I=4096), SHAPE), (dict(k=3, E=2), SHAPE), (dict(gating=2), SHAPE),
    (dict(layout=2), SHAPE), (dict(q13=PMIS), ALIGN), (dict(ws=PMIS), ALIGN),
    (dict(wsb=256), WORKSPACE),
])
def test_one_token_validation(kw, want):
    assert _one_token(**kw) == want


def _repack(**kw):
    a = dict(q=P, rows=64, K=256, qb=P + (1 << 20))
    a.update(kw)
    return B.load().moe_repack_weights(a["q"], a["rows"], a["K"], a["qb"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), NULL), (dict(qb=None), NULL), (dict(rows=0), SHAPE), (dict(rows=40), SHAPE),
    (dict(rows=-16), SHAPE), (dict(K=48), SHAPE), (dict(K=0), SHAPE), (dict(K=65536 + 32), SHAPE),
    (dict(rows=1 << 40, K=65536), SHAPE), (dict(q=PMIS), ALIGN), (dict(qb=PMIS), ALIGN),
    (dict(qb=P), OVERLAP), (dict(qb=P + 64 * 128 - 16), OVERLAP), (dict(q=P + (1 << 20) - 4096), OVERLAP),
])
def test_repack_validation(kw, want):
    assert _repack(**kw) == want


def test_layout_names():
    assert moe.LAYOUTS == {"canonical": 0, "blocked": 1}
    with pytest.raises(ValueError):
        B.layout_code("rowmajor")


def test_valid_arguments_reach_the_device_check():
    # only meaningful where no GPU is visible: a well-formed call must stop at
    # the device check (MOE_ERR_DEVICE) and never dereference the fake pointers
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible; fake pointers must not reach it")
    assert _route() == DEVICE
    assert _tiles() == DEVICE
    assert _forward() == DEVICE
    for which in ("gateup", "down", "combine"):
        assert _steps(which) == DEVICE
    assert _route_tiles() == DEVICE
    assert _one_token() == DEVICE
    assert _repack() == DEVICE


def test_binding_raises_on_error_status():
    with pytest.raises(B.MoeError):
        B._check(SHAPE, "probe")
