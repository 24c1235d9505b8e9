"""The oracle's pins must catch plausible mistakes (CPU only).

Each case plants one wrong convention in the oracle module (monkeypatched for
the duration of the case) and runs the pins that should notice it; the case
passes only if at least one of them fails.
"""
import numpy as np
import pytest

import oracle
from oracle import moe_oracle as mo

import test_oracle_decode as tdec
import test_oracle_ffn as tffn
import test_oracle_gptoss as tgpt
import test_oracle_routing as trout


def _unpack_high_first(q):
    q = np.asarray(q, dtype=np.uint8)
    out = np.empty(q.shape[:-1] + (q.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = q >> 4
    out[..., 1::2] = q & 0xF
    return out


def _e8m0_bias_126(s):
    s = np.asarray(s, dtype=np.int64)
    return np.where(s == 255, np.nan, np.ldexp(1.0, s - 126))


def _topk_ties_high(L, k):
    E = L.shape[1]
    order = np.argsort(-L[:, ::-1], axis=1, kind="stable")
    return (E - 1 - order[:, :k]).astype(np.int32)


def _softmax_all_experts(L, ids):
    z = np.exp(L - L.max(axis=1, keepdims=True))
    z = z / z.sum(axis=1, keepdims=True)
    return np.take_along_axis(z, ids.astype(np.int64), axis=1)


def _sigmoid_unnormalised(L, ids):
    sel = np.take_along_axis(L, ids.astype(np.int64), axis=1)
    return 1.0 / (1.0 + np.exp(-sel))


def _sigmoid_sign_flipped(L, ids):
    sel = np.take_along_axis(L, ids.astype(np.int64), axis=1)
    s = 1.0 / (1.0 + np.exp(sel))
    return s / s.sum(axis=1, keepdims=True)


def _ffn(swap=False, transpose_down=False, no_silu=False):
    def f(X, q13, s13, q2, s2):
        W13 = mo.dequant_mxfp4(q13, s13)
        I = W13.shape[0] // 2
        gate, up = (W13[I:], W13[:I]) if swap else (W13[:I], W13[I:])
        g, u = X @ gate.T, X @ up.T
        h = g * u if no_silu else mo.silu(g) * u
        W2 = mo.dequant_mxfp4(q2, s2)
        return h @ (W2 if transpose_down else W2.T)
    return f


def _combine_unweighted(y, w):
    T, k = w.shape
    return y.reshape(T, k, -1).sum(axis=1)


def _tiles_unstable(topk_ids, E, BM):
    off, srt, tiles, nt = _orig_build_tiles(topk_ids, E, BM)
    flat = np.asarray(topk_ids).ravel()
    srt = np.argsort(flat, kind="quicksort")[::-1].copy()
    srt = srt[np.argsort(flat[srt], kind="stable")].astype(np.int32)
    return off, srt, tiles, nt


def _blocked_unchanged(q):
    return np.ascontiguousarray(np.asarray(q, dtype=np.uint8))


def _blocked_whole_matrix(q):
    # block-major over all rows instead of within 16-row groups
    q = np.asarray(q, dtype=np.uint8)
    R, KH = q.shape[-2:]
    t = q.reshape(q.shape[:-2] + (R, KH // 16, 16))
    return np.ascontiguousarray(np.swapaxes(t, -3, -2)).reshape(q.shape)


def _gptoss(gate_first_half=False, no_plus_one=False, gate_clamp_both=False, up_unclamped=False,
            no_down_bias=False, alpha_one=False, bias_halves=False):
    """expert_ffn_gptoss with one plausible mistake."""
    def f(X, q13, s13, q2, s2, b13, b2, alpha=mo.GPTOSS_ALPHA, limit=mo.GPTOSS_LIMIT):
        W13 = mo.dequant_mxfp4(q13, s13)
        I = W13.shape[0] // 2
        b = np.asarray(b13, dtype=np.float64)
        if bias_halves:  # bias taken as [gate; up] while the rows interleave
            b = np.stack([b[:I], b[I:]], axis=1).reshape(-1)
        z = X @ W13.T + b[None, :]
        g, u = (z[:, :I], z[:, I:]) if gate_first_half else (z[:, 0::2], z[:, 1::2])
        g = np.clip(g, -limit, limit) if gate_clamp_both else np.minimum(g, limit)
        if not up_unclamped:
            u = np.clip(u, -limit, limit)
        a = 1.0 if alpha_one else alpha
        h = g / (1.0 + np.exp(-a * g)) * (u if no_plus_one else u + 1.0)
        y = h @ mo.dequant_mxfp4(q2, s2).T
        return y if no_down_bias else y + np.asarray(b2, dtype=np.float64)[None, :]
    return f


def _deinterleave_identity(a, axis):
    return np.ascontiguousarray(np.asarray(a))


_orig_build_tiles = mo.build_tiles

PINS = [
    tdec.test_nibble_order_low_first,
    tdec.test_e8m0_matches_torch_exhaustive,
    tdec.test_dequant_exhaustive_codes_times_scales,
    tdec.test_blocked_layout_matches_definition_and_inverts,
    trout.test_topk_tie_rule_and_order,
    trout.test_softmax_equals_renormalised_full_softmax,
    trout.test_sigmoid_gating_worked_example,
    trout.test_sigmoid_gating_closed_forms,
    lambda: trout.test_tiles_against_python_sort_and_invariants(17, 3, 5, 4),
    tffn.test_permutation_weights_closed_form,
    tffn.test_single_expert_equals_textbook_swiglu_mlp,
    lambda: tffn.test_routed_equals_dense_then_select(4, 64, 8, 2, 64, False),
    tgpt.test_deinterleave_matches_index_loop_and_inverts,
    tgpt.test_single_expert_equals_textbook_torch_mlp,
    tgpt.test_clamp_boundaries_worked_example,
    tgpt.test_bias_only_experts,
    tgpt.test_reduces_to_plain_swiglu_plus_silu_term,
]

MUTATIONS = {
    "nibble_high_first": ("unpack_codes", _unpack_high_first),
    "e8m0_bias_126": ("decode_e8m0", _e8m0_bias_126),
    "ties_to_higher_index": ("top_k", _topk_ties_high),
    "softmax_over_all_experts": ("softmax_selected", _softmax_all_experts),
    "sigmoid_unnormalised": ("sigmoid_selected", _sigmoid_unnormalised),
    "sigmoid_sign_flipped": ("sigmoid_selected", _sigmoid_sign_flipped),
    "gate_up_swapped": ("expert_ffn", _ffn(swap=True)),
    "down_transposed": ("expert_ffn", _ffn(transpose_down=True)),
    "no_silu": ("expert_ffn", _ffn(no_silu=True)),
    "combine_unweighted": ("combine", _combine_unweighted),
    "unstable_scatter": ("build_tiles", _tiles_unstable),
    "blocked_layout_unchanged": ("blocked_from_canonical", _blocked_unchanged),
    "blocked_over_whole_matrix": ("blocked_from_canonical", _blocked_whole_matrix),
    "gptoss_gate_first_half": ("expert_ffn_gptoss", _gptoss(gate_first_half=True)),
    "gptoss_no_plus_one": ("expert_ffn_gptoss", _gptoss(no_plus_one=True)),
    "gptoss_gate_clamped_both_sides": ("expert_ffn_gptoss", _gptoss(gate_clamp_both=True)),
    "gptoss_up_unclamped": ("expert_ffn_gptoss", _gptoss(up_unclamped=True)),
    "gptoss_no_down_bias": ("expert_ffn_gptoss", _gptoss(no_down_bias=True)),
    "gptoss_alpha_one": ("expert_ffn_gptoss", _gptoss(alpha_one=True)),
    "gptoss_bias_in_halves": ("expert_ffn_gptoss", _gptoss(bias_halves=True)),
    "deinterleave_identity": ("concatenated_from_interleaved", _deinterleave_identity),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(mo, attr, fn)
    monkeypatch.setattr(oracle, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError):
            caught.append(getattr(pin, "__name__", "lambda"))
    assert caught, f"mutation {name} passed every pin"
