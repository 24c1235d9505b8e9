"""Pins for the oracle's router, top-k, softmax and tile table (CPU only).

Logits are checked against exact rational arithmetic, top-k against brute
force over all k-subsets, the softmax against scipy's full softmax followed
by renormalisation over the selected experts (the Mixtral-style gating the
triton-kernels README's fused MoE dispatch example names), and the tile
table against Python's stable sort and closed-form counts.
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

import oracle
from moe_inputs import WORKLOADS, make_random, make_workload


def _exact(v) -> Fraction:
    return Fraction(float(v))


def test_logits_match_exact_rationals():
    inp = make_random(T=3, H=64, E=5, k=2, I=32, seed=1, router_bias=True)
    L = oracle.router_logits(inp["x"], inp["w_router"], inp["bias"])
    x = oracle.bf16_to_f64(inp["x"])
    for t in range(3):
        for e in range(5):
            acc = sum(_exact(x[t, h]) * _exact(inp["w_router"][e, h]) for h in range(64))
            acc += _exact(inp["bias"][e])
            assert abs(float(acc) - L[t, e]) <= 1e-15 * max(1.0, abs(float(acc)))


def test_logits_without_bias_differ_by_bias():
    inp = make_random(T=4, H=32, E=6, k=2, I=32, seed=2, router_bias=True)
    a = oracle.router_logits(inp["x"], inp["w_router"], inp["bias"])
    b = oracle.router_logits(inp["x"], inp["w_router"], None)
    np.testing.assert_allclose(a - b, np.broadcast_to(inp["bias"].astype(np.float64), a.shape),
                               rtol=0, atol=1e-12)


def _brute_topk(row, k):
    # best k-subset by sum, ties by lexicographically smallest sorted ids;
    # then order by (-logit, id)
    best = None
    for sub in itertools.combinations(range(len(row)), k):
        key = (-sum(Fraction(float(row[i])) for i in sub), sub)
        if best is None or key < best[0]:
            best = (key, sub)
    return sorted(best[1], key=lambda e: (-row[e], e))


@pytest.mark.parametrize("seed", range(5))
def test_topk_brute_force(seed):
    rng = np.random.default_rng(seed)
    L = rng.standard_normal((6, 7))
    L[0, :] = 0.25                      # all tied
    L[1, [1, 4]] = L[1, 3]              # three-way tie
    for k in (1, 2, 3, 7):
        ids = oracle.top_k(L, k)
        for t in range(L.shape[0]):
            assert list(ids[t]) == _brute_topk(L[t], k)


def test_topk_tie_rule_and_order():
    L = np.array([[1.0, 3.0, 3.0, 0.0, 3.0]])
    assert list(oracle.top_k(L, 3)[0]) == [1, 2, 4]
    assert list(oracle.top_k(L, 4)[0]) == [1, 2, 4, 0]


def test_softmax_equals_renormalised_full_softmax():
    rng = np.random.default_rng(3)
    L = rng.standard_normal((20, 9)) * 3
    ids = oracle.top_k(L, 3)
    w = oracle.softmax_selected(L, ids)
    full = sp_softmax(L, axis=1)
    sel = np.take_along_axis(full, ids.astype(np.int64), axis=1)
    np.testing.assert_allclose(w, sel / sel.sum(axis=1, keepdims=True), rtol=1e-14, atol=0)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(np.diff(w, axis=1) <= 0)   # descending logits -> descending weights


def test_softmax_special_cases():
    L = np.random.default_rng(4).standard_normal((5, 6))
    assert np.all(oracle.softmax_selected(L, oracle.top_k(L, 1)) == 1.0)
    # all-zero router: ids 0..k-1, weights 1/k
    inp = make_random(T=4, H=32, E=6, k=3, I=32, seed=5)
    ids, w, _ = oracle.route(inp["x"], np.zeros_like(inp["w_router"]), None, 3)
    assert np.all(ids == np.arange(3)) and np.allclose(w, 1 / 3, rtol=0, atol=1e-15)


def test_sigmoid_gating_worked_example():
    # logits 0, ln 3, -ln 3: sigmoids 1/2, 3/4, 1/4; top-2 are experts 1 and 0,
    # weights (3/4, 1/2) / (5/4) = (0.6, 0.4)
    L = np.array([[0.0, np.log(3.0), -np.log(3.0)]])
    ids = oracle.top_k(L, 2)
    assert list(ids[0]) == [1, 0]
    np.testing.assert_allclose(oracle.sigmoid_selected(L, ids), [[0.6, 0.4]], rtol=0, atol=1e-15)


def test_sigmoid_gating_closed_forms():
    rng = np.random.default_rng(6)
    L = rng.standard_normal((12, 7)) * 4
    # one expert: weight 1
    assert np.all(oracle.sigmoid_selected(L, oracle.top_k(L, 1)) == 1.0)
    # a pair of logits a, -a: sigmoid(a) + sigmoid(-a) = 1, so the weights are
    # the sigmoids themselves (scipy's expit as the independent reference)
    from scipy.special import expit
    a = rng.standard_normal(9) * 3
    P = np.stack([a, -a], axis=1)
    ids = oracle.top_k(P, 2)
    w = oracle.sigmoid_selected(P, ids)
    np.testing.assert_allclose(w, expit(np.take_along_axis(P, ids.astype(np.int64), axis=1)),
                               rtol=1e-14, atol=0)
    # in general: positive, summing to 1, descending with the logits, and
    # different from softmax whenever the selected logits differ
    ids = oracle.top_k(L, 3)
    w = oracle.sigmoid_selected(L, ids)
    assert np.all(w > 0)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(np.diff(w, axis=1) <= 0)
    assert not np.allclose(w, oracle.softmax_selected(L, ids))


def test_route_gating_switch():
    inp = make_random(T=6, H=64, E=8, k=2, I=32, seed=7, router_std=0.3)
    ids_s, w_s, L = oracle.route(inp["x"], inp["w_router"], None, 2, gating="sigmoid")
    ids_m, w_m, _ = oracle.route(inp["x"], inp["w_router"], None, 2)
    assert np.array_equal(ids_s, ids_m)
    np.testing.assert_array_equal(w_s, oracle.sigmoid_selected(L, ids_s))
    np.testing.assert_array_equal(w_m, oracle.softmax_selected(L, ids_m))
    with pytest.raises(ValueError):
        oracle.route(inp["x"], inp["w_router"], None, 2, gating="relu")


def test_route_on_workloads_has_clear_gaps():
    # routing is unique when the float64 gaps between the k-th and (k+1)-th
    # logits (and between consecutive selected logits) are far above the
    # GPU's fp64 accumulation error
    for wid in sorted(WORKLOADS):
        inp = make_workload(wid, weights=False)
        ids, w, L = oracle.route(inp["x"], inp["w_router"], inp["bias"], inp["k"],
                                 inp["gating"])
        srt = -np.sort(-L, axis=1)
        gaps = -np.diff(srt[:, :inp["k"] + 1], axis=1)
        assert gaps.min() > 1e-9, (wid, gaps.min())
        assert len(set(map(tuple, ids))) >= 1
        for t in range(ids.shape[0]):
            assert len(set(ids[t])) == inp["k"]


# ---------------------------------------------------------------- tiles --

@pytest.mark.parametrize("T,k,E,BM", [(4, 2, 8, 16), (17, 3, 5, 4), (64, 4, 32, 16),
                                      (33, 1, 1, 8), (50, 4, 7, 32), (1, 4, 32, 16)])
def test_tiles_against_python_sort_and_invariants(T, k, E, BM):
    rng = np.random.default_rng(T * 100 + E)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    off, srt, tiles, nt = oracle.build_tiles(ids, E, BM)
    flat = ids.ravel()
    assert list(srt) == sorted(range(T * k), key=lambda p: flat[p])
    counts = np.array([(flat == e).sum() for e in range(E)])
    assert off[0] == 0 and off[-1] == T * k and np.all(np.diff(off) == counts)
    assert nt == sum(-(-int(c) // BM) for c in counts) == tiles.shape[0]
    # tiles: experts ascending, each segment covered exactly once in order
    covered = np.zeros(T * k, dtype=int)
    prev = (-1, -1)
    for e, r0, n in tiles:
        assert 1 <= n <= BM and (e, r0) > prev
        prev = (e, r0)
        assert off[e] <= r0 and r0 + n <= off[e + 1]
        covered[r0:r0 + n] += 1
        assert np.all(flat[srt[r0:r0 + n]] == e)
        if r0 + n < off[e + 1]:
            assert n == BM            # only an expert's last tile may be short
    assert np.all(covered == 1)
    # each token appears exactly k times across the tiles
    tok = np.bincount(srt // k, minlength=T)
    assert np.all(tok == k)


def test_tiles_empty_experts_and_k_equals_E():
    ids = np.tile(np.arange(4, dtype=np.int32), (3, 1))
    off, srt, tiles, nt = oracle.build_tiles(ids, 6, 2)
    assert list(off) == [0, 3, 6, 9, 12, 12, 12]
    assert nt == 8 and set(tiles[:, 0]) == {0, 1, 2, 3}
