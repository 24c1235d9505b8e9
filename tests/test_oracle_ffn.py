"""Pins for the oracle's expert FFN and combine (CPU only).

* a closed form: permutation-structured weights reduce the layer to indexing,
  so a transposed operand, a swapped gate/up half, a wrong nibble order or a
  dropped scale changes which inputs land where;
* a textbook dense SwiGLU MLP in torch (float64, CPU) for E = 1, k = 1, with
  weights decoded from the e2m1 bit fields in this file;
* brute force: every expert evaluated densely on every token, then selected;
* invariants: identical experts make the output independent of the routing
  weights; permuting tokens permutes outputs; relabelling experts changes
  nothing.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_inputs import make_random, identical_experts

from test_oracle_decode import _e2m1_from_bits


def _pack(codes: np.ndarray) -> np.ndarray:
    codes = codes.astype(np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def _decode_by_bits(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    table = np.array([_e2m1_from_bits(c) for c in range(16)])
    codes = np.empty(q.shape[:-1] + (q.shape[-1] * 2,), dtype=np.int64)
    codes[..., 0::2] = q & 15
    codes[..., 1::2] = q >> 4
    scale = 2.0 ** (np.repeat(s.astype(np.float64), 32, axis=-1) - 127)
    return table[codes] * scale


def test_permutation_weights_closed_form():
    H = I = 64
    T = 5
    rng = np.random.default_rng(11)
    pi, sigma, rho = rng.permutation(I), rng.permutation(I), rng.permutation(H)
    c13 = np.zeros((1, 2 * I, H), dtype=np.uint8)
    c13[0, np.arange(I), pi] = 2            # gate row n: +1.0 at column pi[n]
    c13[0, I + np.arange(I), sigma] = 2     # up row n: +1.0 at column sigma[n]
    s13 = np.full((1, 2 * I, H // 32), 127, dtype=np.uint8)
    s13[0, I:] = 128                        # up rows scaled by 2
    c2 = np.zeros((1, H, I), dtype=np.uint8)
    c2[0, np.arange(H), rho] = 10           # down row m: -1.0 at column rho[m]
    s2 = np.full((1, H, I // 32), 127, dtype=np.uint8)
    inp = make_random(T=T, H=H, E=1, k=1, I=I, seed=3)
    inp.update(w13_q=_pack(c13), w13_s=s13, w2_q=_pack(c2), w2_s=s2)
    res = oracle.moe_layer(inp)
    x = oracle.bf16_to_f64(inp["x"])
    g = x[:, pi]
    u = 2.0 * x[:, sigma]
    h = g / (1.0 + np.exp(-g)) * u
    want = -h[:, rho]
    np.testing.assert_allclose(res["out"], want, rtol=1e-15, atol=0)
    assert np.all(res["topk_weights"] == 1.0)


def test_single_expert_equals_textbook_swiglu_mlp():
    inp = make_random(T=7, H=96, E=1, k=1, I=64, seed=4)
    res = oracle.moe_layer(inp)
    x = torch.from_numpy(oracle.bf16_to_f64(inp["x"]))
    W13 = torch.from_numpy(_decode_by_bits(inp["w13_q"][0], inp["w13_s"][0]))
    W2 = torch.from_numpy(_decode_by_bits(inp["w2_q"][0], inp["w2_s"][0]))
    I = W13.shape[0] // 2
    gate = torch.nn.functional.linear(x, W13[:I])
    up = torch.nn.functional.linear(x, W13[I:])
    want = torch.nn.functional.linear(torch.nn.functional.silu(gate) * up, W2)
    np.testing.assert_allclose(res["out"], want.numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("T,H,E,k,I,bias", [(4, 64, 8, 2, 64, False), (9, 32, 5, 3, 96, True),
                                            (16, 64, 3, 3, 32, False)])
def test_routed_equals_dense_then_select(T, H, E, k, I, bias):
    inp = make_random(T=T, H=H, E=E, k=k, I=I, seed=T + E, router_bias=bias, router_std=0.3)
    res = oracle.moe_layer(inp, BM=4)
    x = oracle.bf16_to_f64(inp["x"])
    dense = np.stack([oracle.expert_ffn(x, inp["w13_q"][e], inp["w13_s"][e],
                                        inp["w2_q"][e], inp["w2_s"][e]) for e in range(E)])
    want = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            want[t] += res["topk_weights"][t, j] * dense[res["topk_ids"][t, j], t]
    np.testing.assert_allclose(res["out"], want, rtol=1e-12, atol=1e-9)


def test_identical_experts_ignore_routing_weights():
    inp = identical_experts(make_random(T=6, H=64, E=4, k=2, I=64, seed=8, router_std=0.5))
    res = oracle.moe_layer(inp)
    x = oracle.bf16_to_f64(inp["x"])
    one = oracle.expert_ffn(x, inp["w13_q"][0], inp["w13_s"][0], inp["w2_q"][0], inp["w2_s"][0])
    np.testing.assert_allclose(res["out"], one, rtol=1e-12, atol=1e-9)


def test_token_permutation_permutes_output():
    inp = make_random(T=8, H=64, E=6, k=2, I=32, seed=9, router_std=0.3)
    perm = np.random.default_rng(1).permutation(8)
    a = oracle.moe_layer(inp)["out"]
    inp2 = dict(inp, x=inp["x"][perm])
    b = oracle.moe_layer(inp2)["out"]
    np.testing.assert_allclose(b, a[perm], rtol=1e-13, atol=1e-12)


def test_expert_relabel_invariance():
    inp = make_random(T=8, H=64, E=6, k=2, I=32, seed=10, router_std=0.3)
    relabel = np.random.default_rng(2).permutation(6)
    a = oracle.moe_layer(inp)
    inp2 = dict(inp, w_router=inp["w_router"][relabel])
    for key in ("w13_q", "w13_s", "w2_q", "w2_s"):
        inp2[key] = inp[key][relabel]
    b = oracle.moe_layer(inp2)
    np.testing.assert_allclose(b["out"], a["out"], rtol=1e-13, atol=1e-12)
    inv = np.argsort(relabel)
    assert np.all(relabel[b["topk_ids"]] == a["topk_ids"])
    assert np.all(inv[a["topk_ids"]] == b["topk_ids"])


def test_token_subset_matches_full():
    inp = make_random(T=10, H=64, E=5, k=2, I=32, seed=12, router_std=0.3)
    full = oracle.moe_layer(inp)
    sub = oracle.moe_layer(inp, tokens=[7, 2, 9])
    # same arithmetic on fewer rows; BLAS blocking may move the last ulp
    np.testing.assert_allclose(sub["out"], full["out"][[7, 2, 9]], rtol=1e-13, atol=1e-13)
