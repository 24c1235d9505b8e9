"""Pins for the oracle's gpt-oss expert form (CPU only).

The form is not on the pages (they only say the official MXFP4 checkpoints
are loaded unchanged); the oracle takes the released model's definition as
given: w13 rows interleaved (2i: gate of output i, 2i + 1: its up), biases on
w13 and w2 rows, and h = min(g, L) * sigmoid(a * min(g, L)) *
(clip(u, -L, L) + 1) with a = 1.702, L = 7.  What pins it here:
* the row de-interleave against a plain index loop;
* a textbook torch float64 MLP of that form (weights decoded from the e2m1
  bit fields in test_oracle_ffn, not through the oracle);
* a worked example at exact dyadic values on both sides of each clamp;
* bias-only experts (zero codes): the output is the routing-weighted sum of
  the down biases exactly, and with a permutation down matrix the bias
  interleave is visible;
* an identity with the plain SwiGLU oracle: without the clamp, with a = 1
  and no biases, h = silu(g) * u + silu(g).
"""
import math

import numpy as np
import torch

import oracle
from moe_inputs import make_random, make_weights, with_gptoss_experts

from test_oracle_ffn import _decode_by_bits, _pack


def test_deinterleave_matches_index_loop_and_inverts():
    rng = np.random.default_rng(5)
    E, I, B = 3, 6, 5
    a = rng.integers(0, 256, size=(E, 2 * I, B), dtype=np.uint8)
    want = np.empty_like(a)
    for e in range(E):
        for i in range(I):
            want[e, i] = a[e, 2 * i]
            want[e, I + i] = a[e, 2 * i + 1]
    got = oracle.concatenated_from_interleaved(a, axis=1)
    np.testing.assert_array_equal(got, want)
    b = rng.normal(size=(E, 2 * I)).astype(np.float32)
    gb = oracle.concatenated_from_interleaved(b, axis=-1)
    for e in range(E):
        for i in range(I):
            assert gb[e, i] == b[e, 2 * i] and gb[e, I + i] == b[e, 2 * i + 1]
    back = np.empty_like(got)
    back[:, 0::2], back[:, 1::2] = got[:, :I], got[:, I:]
    np.testing.assert_array_equal(back, a)


def _textbook_torch(x, W13, b13, W2, b2, alpha, limit):
    """The model's MLP block written with torch ops (float64, CPU)."""
    z = torch.nn.functional.linear(x, W13, b13)
    x_glu, x_lin = z[..., ::2], z[..., 1::2]
    x_glu = x_glu.clamp(max=limit)
    x_lin = x_lin.clamp(min=-limit, max=limit)
    h = x_glu * torch.sigmoid(alpha * x_glu) * (x_lin + 1)
    return torch.nn.functional.linear(h, W2, b2)


def test_single_expert_equals_textbook_torch_mlp():
    T, H, I = 7, 96, 64
    inp = make_random(T=T, H=H, E=1, k=1, I=I, seed=21, router_std=0.3)
    inp.update(make_weights(1, H, I, 21, scale_lo=126, scale_hi=128))  # reach both clamps
    inp = with_gptoss_experts(inp, 9)
    res = oracle.moe_layer(inp)
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    W13 = t(_decode_by_bits(inp["w13_q"][0], inp["w13_s"][0]))
    W2 = t(_decode_by_bits(inp["w2_q"][0], inp["w2_s"][0]))
    want = _textbook_torch(t(oracle.bf16_to_f64(inp["x"])), W13, t(inp["b13"][0]), W2,
                           t(inp["b2"][0]), 1.702, 7.0).numpy()
    np.testing.assert_allclose(res["out"], want, rtol=1e-12, atol=1e-12)
    # the synthetic layer exercises both clamps
    z = oracle.bf16_to_f64(inp["x"]) @ W13.numpy().T + inp["b13"][0]
    assert (z[:, 0::2] > 7).any() and (z[:, 1::2] > 7).any() and (z[:, 1::2] < -7).any()


def _one_hot_expert(g_vals, u_vals, b_gate, b_up, H=32):
    """One expert whose w13 column 0 holds e2m1 * 2^(s-127) values: gate row
    i (row 2i) = g_vals[i], up row i (row 2i + 1) = u_vals[i]; the biases of
    those rows as given.  Values are (code, scale byte) pairs."""
    I = len(g_vals)
    codes = np.zeros((1, 2 * I, H), dtype=np.uint8)
    scales = np.full((1, 2 * I, H // 32), 127, dtype=np.uint8)
    b13 = np.zeros((1, 2 * I), dtype=np.float32)
    for i, ((cg, sg), (cu, su)) in enumerate(zip(g_vals, u_vals)):
        codes[0, 2 * i, 0], scales[0, 2 * i, 0] = cg, sg
        codes[0, 2 * i + 1, 0], scales[0, 2 * i + 1, 0] = cu, su
        b13[0, 2 * i], b13[0, 2 * i + 1] = b_gate[i], b_up[i]
    return _pack(codes), scales, b13


def test_clamp_boundaries_worked_example():
    # gate pre-activations -12, -6, 0, 3, 6, 7 (6 + bias 1), 8, 12 and up
    # pre-activations 12, -12, 7 (6 + 1), -8, 0.5, -0.5, 3, -3 at x = e_0
    # (e2m1 codes: 7 -> 6, 6 -> 4, 5 -> 3, 1 -> 0.5, +8 negates; scale byte
    # 128 doubles)
    g_vals = [(15, 128), (15, 127), (0, 127), (5, 127), (7, 127), (7, 127), (6, 128), (7, 128)]
    u_vals = [(7, 128), (15, 128), (7, 127), (14, 128), (1, 127), (9, 127), (5, 127), (13, 127)]
    b_gate = [0, 0, 0, 0, 0, 1, 0, 0]
    b_up = [0, 0, 1, 0, 0, 0, 0, 0]
    g = [-12.0, -6.0, 0.0, 3.0, 6.0, 7.0, 8.0, 12.0]
    u = [12.0, -12.0, 7.0, -8.0, 0.5, -0.5, 3.0, -3.0]
    n, I, H = 8, 32, 32  # outputs n..I-1 have zero rows: h = 0 there
    g_vals += [(0, 127)] * (I - n)
    u_vals += [(0, 127)] * (I - n)
    b_gate += [0] * (I - n)
    b_up += [0] * (I - n)
    q13, s13, b13 = _one_hot_expert(g_vals, u_vals, b_gate, b_up, H)
    # down: output m < n copies h[m] plus nothing; m >= n is its bias alone
    c2 = np.zeros((1, H, I), dtype=np.uint8)
    c2[0, np.arange(n), np.arange(n)] = 2
    s2 = np.full((1, H, I // 32), 127, dtype=np.uint8)
    b2 = np.zeros((1, H), dtype=np.float32)
    b2[0, n:] = np.arange(1, H - n + 1, dtype=np.float32) / 4
    x_bits = np.zeros((1, H), dtype=np.uint16)
    x_bits[0, 0] = 0x3F80  # bf16 1.0
    inp = dict(x=x_bits, w_router=np.zeros((1, H), np.float32), bias=None, k=1,
               w13_q=q13, w13_s=s13, w2_q=_pack(c2), w2_s=s2, activation="gptoss",
               b13=b13, b2=b2, alpha=1.702, limit=7.0)
    out = oracle.moe_layer(inp)["out"][0]
    for i in range(n):
        gc = min(g[i], 7.0)
        uc = max(min(u[i], 7.0), -7.0)
        h = gc / (1.0 + math.exp(-1.702 * gc)) * (uc + 1.0)
        assert math.isclose(out[i], h, rel_tol=1e-14, abs_tol=1e-300), (i, out[i], h)
    np.testing.assert_array_equal(out[n:], b2[0, n:].astype(np.float64))
    # spot values of the closed form: the gate clamp is from above only, the
    # up clamp two-sided, and u = -1 would zero the output
    assert math.isclose(out[0], -12.0 / (1.0 + math.exp(1.702 * 12.0)) * 8.0, rel_tol=1e-14)
    assert math.isclose(out[6], 7.0 / (1.0 + math.exp(-1.702 * 7.0)) * 4.0, rel_tol=1e-14)
    assert out[2] == 0.0


def test_bias_only_experts():
    T, H, E, k, I = 6, 64, 4, 2, 32
    inp = with_gptoss_experts(make_random(T=T, H=H, E=E, k=k, I=I, seed=33, router_std=0.5), 4)
    for key in ("w13_q", "w2_q"):
        inp[key] = np.zeros_like(inp[key])
    r = oracle.moe_layer(inp)
    ids, w = r["topk_ids"], r["topk_weights"]
    want = np.einsum("tj,tjh->th", w, inp["b2"][ids].astype(np.float64))
    np.testing.assert_allclose(r["out"], want, rtol=1e-15, atol=0)
    # a permutation down matrix shows h, made of the biases alone: gate bias
    # at even positions, up bias at odd ones
    rho = np.random.default_rng(2).permutation(I)
    c2 = np.zeros((E, H, I), dtype=np.uint8)
    c2[:, np.arange(I), rho] = 2
    inp["w2_q"] = _pack(c2)
    inp["w2_s"] = np.full_like(inp["w2_s"], 127)
    r = oracle.moe_layer(inp)
    bg = np.minimum(inp["b13"][:, 0::2].astype(np.float64), 7.0)
    bu = np.clip(inp["b13"][:, 1::2].astype(np.float64), -7.0, 7.0)
    hb = bg / (1.0 + np.exp(-1.702 * bg)) * (bu + 1.0)          # [E, I]
    y = inp["b2"].astype(np.float64).copy()
    y[:, :I] += hb[:, rho]
    want = np.einsum("tj,tjh->th", r["topk_weights"], y[r["topk_ids"]])
    np.testing.assert_allclose(r["out"], want, rtol=1e-14, atol=1e-14)


def test_reduces_to_plain_swiglu_plus_silu_term():
    T, H, I = 9, 64, 32
    inp = make_random(T=T, H=H, E=1, k=1, I=I, seed=44, router_std=0.3)
    x = oracle.bf16_to_f64(inp["x"])
    q13c = oracle.concatenated_from_interleaved(inp["w13_q"][0], axis=0)
    s13c = oracle.concatenated_from_interleaved(inp["w13_s"][0], axis=0)
    zeros13 = np.zeros(2 * I, np.float32)
    got = oracle.expert_ffn_gptoss(x, inp["w13_q"][0], inp["w13_s"][0], inp["w2_q"][0],
                                   inp["w2_s"][0], zeros13, np.zeros(H, np.float32),
                                   alpha=1.0, limit=np.inf)
    plain = oracle.expert_ffn(x, q13c, s13c, inp["w2_q"][0], inp["w2_s"][0])
    g = x @ oracle.dequant_mxfp4(q13c[:I], s13c[:I]).T
    extra = oracle.silu(g) @ oracle.dequant_mxfp4(inp["w2_q"][0], inp["w2_s"][0]).T
    np.testing.assert_allclose(got, plain + extra, rtol=1e-12, atol=1e-9)
