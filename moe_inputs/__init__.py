"""Seeded synthetic inputs for the MXFP4 grouped-expert MoE layer.

This module only draws random numbers and packs them into the byte layouts
both sides consume; it holds none of the layer's arithmetic (no decoding, no
routing, no GEMM).  The float64 oracle and the HIP path both take the arrays
it returns, and neither imports the other.

Workloads are the gpt-oss-shaped MoE layers the SimpleLLM write-up measures
("A 297-line kernel file that decodes faster than vLLM", sections "Where the
time went" and "Optimizations": gpt-oss-20b and gpt-oss-120b, decode batch 1
and 64, 4k-token prefill), rebuilt synthetically because no checkpoint is
available:

  x        bf16 bits, uint16 [T, H], drawn N(0, 1) in float64, rounded to
           float32 then to bf16 (both round-to-nearest-even)
  w_router float32 [E, H], N(0, 0.02)  (0.02 is the standard deviation)
  bias     float32 [E] N(0, 1) for the skewed-load workload, else None
  w13_q    uint8 [E, 2I, H/2]   two e2m1 codes per byte, uniform over all 16
  w13_s    uint8 [E, 2I, H/32]  E8M0 scale bytes, uniform over 120..124
  w2_q     uint8 [E, H, I/2]
  w2_s     uint8 [E, H, I/32]

A uniformly random byte carries two independent uniform nibbles, so the
packed weight arrays are drawn as raw bytes.

Two more workloads take the shapes of the triton-kernels README's MoE
dispatch benchmark (section "Benchmarks": a Mixtral-8x7B-shaped layer, 8
experts, top-2, hidden 4096, FFN 14336; and a DeepSeek-V3-shaped layer, 256
experts with sigmoid gating as the report it cites describes; the top-8 and
the hidden 7168 / expert FFN 2048 widths are that model's published shape,
not stated on the pages) at 128 tokens, with the same distributions.

Seeds: weights come from ``default_rng([model_id, 1])`` (tiny = 0, 20b = 20,
120b = 120, Mixtral-shaped = 8, DeepSeek-V3-shaped = 671), so workloads that
share a model share its bytes; activations, router and bias come from
``default_rng([workload_id, 2])``.  Draw order: x, w_router, bias; then w13
codes, w13 scales, w2 codes, w2 scales.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

SCALE_BYTE_LO = 120  # exponent -7
SCALE_BYTE_HI = 124  # exponent -3


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    T: int
    H: int
    E: int
    k: int
    I: int
    model_id: int
    router_bias: bool
    gating: str = "softmax"


WORKLOADS = {
    0: Workload(0, "tiny_T4_H256_E8_k2_I512", 4, 256, 8, 2, 512, 0, False),
    1: Workload(1, "gptoss20b_decode_T1", 1, 2880, 32, 4, 2880, 20, False),
    2: Workload(2, "gptoss20b_decode_T64_biased_router", 64, 2880, 32, 4, 2880, 20, True),
    3: Workload(3, "gptoss120b_decode_T64", 64, 2880, 128, 4, 2880, 120, False),
    4: Workload(4, "gptoss120b_prefill_T4096", 4096, 2880, 128, 4, 2880, 120, False),
    5: Workload(5, "mixtral8x7b_shaped_T128", 128, 4096, 8, 2, 14336, 8, False),
    6: Workload(6, "deepseekv3_shaped_T128_sigmoid", 128, 7168, 256, 8, 2048, 671, False,
                "sigmoid"),
}


def f64_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (via float32, RNE at each step); uint16 bits."""
    b = np.ascontiguousarray(a, dtype=np.float64).astype(np.float32).view(np.uint32)
    b = b.astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def _bytes(rng: np.random.Generator, shape) -> np.ndarray:
    n = int(np.prod(shape))
    return np.frombuffer(rng.bytes(n), dtype=np.uint8).reshape(shape).copy()


def make_weights(E: int, H: int, I: int, model_id: int,
                 scale_lo: int = SCALE_BYTE_LO, scale_hi: int = SCALE_BYTE_HI) -> dict:
    """Packed MXFP4 expert weights for one layer (see module docstring)."""
    if H % 32 or I % 32:
        raise ValueError("H and I must be multiples of 32")
    rng = np.random.default_rng([model_id, 1])
    w13_q = _bytes(rng, (E, 2 * I, H // 2))
    w13_s = rng.integers(scale_lo, scale_hi + 1, size=(E, 2 * I, H // 32), dtype=np.uint8)
    w2_q = _bytes(rng, (E, H, I // 2))
    w2_s = rng.integers(scale_lo, scale_hi + 1, size=(E, H, I // 32), dtype=np.uint8)
    return dict(w13_q=w13_q, w13_s=w13_s, w2_q=w2_q, w2_s=w2_s)


def make_activations(T: int, H: int, E: int, seed, router_bias: bool,
                     router_std: float = 0.02) -> dict:
    """x (bf16 bits), router weight (fp32) and optional router bias (fp32)."""
    rng = np.random.default_rng(seed)
    x = f64_to_bf16_bits(rng.standard_normal((T, H)))
    w_router = rng.normal(0.0, router_std, size=(E, H)).astype(np.float32)
    bias = rng.standard_normal(E).astype(np.float32) if router_bias else None
    return dict(x=x, w_router=w_router, bias=bias)


def make_workload(wid: int, weights: bool = True) -> dict:
    """All inputs of one of the workloads above, with its shape and gating."""
    w = WORKLOADS[wid]
    out = dict(T=w.T, H=w.H, E=w.E, k=w.k, I=w.I, name=w.name, wid=wid, gating=w.gating)
    out.update(make_activations(w.T, w.H, w.E, [wid, 2], w.router_bias))
    if weights:
        out.update(make_weights(w.E, w.H, w.I, w.model_id))
    return out


def make_random(T: int, H: int, E: int, k: int, I: int, seed: int,
                router_bias: bool = False, router_std: float = 0.02,
                gating: str = "softmax") -> dict:
    """A small random layer of arbitrary shape, same distributions."""
    out = dict(T=T, H=H, E=E, k=k, I=I, name=f"rand_T{T}_H{H}_E{E}_k{k}_I{I}_s{seed}",
               gating=gating)
    out.update(make_activations(T, H, E, [1000 + seed, 2], router_bias, router_std))
    out.update(make_weights(E, H, I, 1000 + seed))
    return out


def with_gptoss_experts(inp: dict, seed: int, bias_std: float = 0.5) -> dict:
    """The same layer read in the gpt-oss expert form (w13 rows taken as
    interleaved gate/up pairs) with expert biases: b13 fp32 [E, 2I] (in the
    interleaved row order) and b2 fp32 [E, H], drawn N(0, bias_std) and
    rounded to bf16 values (the released checkpoints store bf16 biases),
    alpha 1.702 and limit 7.0.  Drawn from ``default_rng([seed, 3])``."""
    E, H, I = inp["w13_q"].shape[0], inp["H"], inp["I"]
    rng = np.random.default_rng([seed, 3])
    b13 = _bf16_values(rng.normal(0.0, bias_std, size=(E, 2 * I)))
    b2 = _bf16_values(rng.normal(0.0, bias_std, size=(E, H)))
    out = dict(inp)
    out.update(activation="gptoss", b13=b13, b2=b2, alpha=1.702, limit=7.0,
               name=inp.get("name", "?") + "_gptoss")
    return out


def _bf16_values(a: np.ndarray) -> np.ndarray:
    """float32 array of the bf16 values nearest to a (RNE)."""
    bits = f64_to_bf16_bits(a).astype(np.uint32) << 16
    return bits.view(np.float32).reshape(a.shape)


def identical_experts(inp: dict) -> dict:
    """Copy expert 0's packed weights into every expert (same bytes everywhere)."""
    out = dict(inp)
    for key in ("w13_q", "w13_s", "w2_q", "w2_s"):
        a = inp[key]
        out[key] = np.ascontiguousarray(np.broadcast_to(a[:1], a.shape))
    return out


__all__ = ["Workload", "WORKLOADS", "f64_to_bf16_bits", "make_weights",
           "make_activations", "make_workload", "make_random", "identical_experts",
           "with_gptoss_experts"]
