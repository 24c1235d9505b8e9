"""Plain float64 CPU oracle for the MXFP4 grouped-expert MoE layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call
this module; only the tests, the smoke check and the benchmark's CPU-baseline
leg do.  It shares no code with the HIP library and imports nothing from it.

The layer is the one the SimpleLLM write-up profiles as three rows of a
gpt-oss decode step ("A 297-line kernel file that decodes faster than vLLM",
section "Where the time went": "Router + top-k", "MoE gate/up + SwiGLU",
"MoE down + combine") and speeds up with MXFP4 expert weights and a
per-expert routing tile table (same page, section "Optimizations").  The
triton-kernels README (section "Quick Start", fused MoE dispatch) gives the
same pipeline as router -> permute -> expert FFN -> unpermute with softmax
gating and top-k.  Steps, each a function below:

  1. router logits  L[t, e] = sum_h x[t, h] * Wr[e, h] (+ b[e])
  2. top-k          the k largest logits per token, in descending order,
                    exact ties going to the lower expert index
  3. gating         softmax over the k selected logits only; or, with
                    sigmoid gating (the triton-kernels README's router,
                    section "Project Structure", moe/router.py: "softmax/
                    sigmoid gating + top-k"), s = sigmoid of each selected
                    logit, normalised to sum 1 over the k
  4. tile table     per-expert counts, exclusive offsets, a stable
                    counting sort of flat slot ids p = t*k + j, and tiles of
                    at most BM rows per expert
  5. gate/up        g = X W1^T, u = X W3^T with W1 = w13[e, :I] and
                    W3 = w13[e, I:]; h = silu(g) * u, silu(z) = z*sigmoid(z)
                    (the README's "Fused SwiGLU": silu(gate) * up)
  6. down           y[p] = W2_e h[p]
  7. combine        out[t] = sum_j w[t, j] * y[t*k + j]

Everything is computed in float64 over exactly decoded inputs: bf16 x and
fp32 router weights are exact in float64, each MXFP4 weight decodes exactly
(an e2m1 value times a power of two), so the only rounding is float64's own.

Readings where the pages are silent (the write-up says only that the
checkpoints' MXFP4 weights are loaded unchanged and reordered in memory;
section "Correctness"):
  * MXFP4 is the OCP Microscaling format: 4-bit e2m1 elements (1 sign bit,
    2 exponent bits with bias 1, 1 mantissa bit, no inf/nan) and one E8M0
    scale byte per 32 consecutive elements along K, value 2^(s - 127),
    s = 255 meaning NaN.
  * Two codes per byte, the even element in the low nibble.
  * w13 rows [0, I) are the gate projection, rows [I, 2I) the up projection.
  * The router bias, when present, is added before both top-k and softmax.
  * The gpt-oss expert form (an opt-in variant, not on the pages, which only
    say that the official MXFP4 checkpoints are loaded unchanged): w13 rows
    interleaved (row 2i the gate projection of output i, row 2i + 1 its up
    projection), a bias on each w13 row and on each w2 row, and a clamped
    SwiGLU, h = min(g, limit) * sigmoid(alpha * min(g, limit)) *
    (clip(u, -limit, limit) + 1), with alpha = 1.702 and limit = 7 for the
    released models.  This is the published model's own definition, taken
    as given; nothing on the pages confirms it, so parity against a real
    checkpoint is unpinned.
  * Sigmoid gating: the pages name it (the README's router; the DeepSeek-V3
    report cited there) but give no formula.  Read here as: experts chosen
    by the same top-k of the logits (sigmoid is increasing, so this is the
    top-k of the sigmoid scores, except where two large logits round to the
    same float64 sigmoid), weights sigmoid(L_j) / sum over the k selected of
    sigmoid(L_q), so the weights sum to 1 as softmax's do; the bias, when
    present, is part of the logit.
"""
from __future__ import annotations

import numpy as np

# e2m1 code -> value, codes 0..15 (sign in bit 3, exponent bits 2..1 with
# bias 1, mantissa bit 0; exponent field 0 is subnormal: 0 or 0.5).
E2M1_VALUES = np.array(
    [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
     -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0], dtype=np.float64)

MX_BLOCK = 32


# ---------------------------------------------------------------- decoding --

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 value of bf16 bit patterns (bf16 is fp32's top half)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):          # NaN payloads widen silently
        return b.view(np.float32).astype(np.float64)


def decode_e2m1(codes: np.ndarray) -> np.ndarray:
    """float64 value of 4-bit e2m1 codes (low 4 bits of each entry)."""
    return E2M1_VALUES[np.asarray(codes, dtype=np.uint8) & 0xF]


def decode_e8m0(s: np.ndarray) -> np.ndarray:
    """float64 value of E8M0 scale bytes: 2^(s - 127); 255 is NaN."""
    s = np.asarray(s, dtype=np.int64)
    v = np.ldexp(1.0, s - 127)
    return np.where(s == 255, np.nan, v)


def unpack_codes(q: np.ndarray) -> np.ndarray:
    """uint8 [..., K/2] packed codes -> uint8 [..., K] codes, even element low."""
    q = np.asarray(q, dtype=np.uint8)
    out = np.empty(q.shape[:-1] + (q.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = q & 0xF
    out[..., 1::2] = q >> 4
    return out


def dequant_mxfp4(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Decode one MXFP4 matrix: W[n, kk] = e2m1(code[n, kk]) * 2^(s[n, kk//32]-127).

    q: uint8 [..., N, K/2]; s: uint8 [..., N, K/32]; returns float64 [..., N, K].
    """
    vals = decode_e2m1(unpack_codes(q))
    scale = np.repeat(decode_e8m0(s), MX_BLOCK, axis=-1)
    if scale.shape != vals.shape:
        raise ValueError(f"scale shape {s.shape} does not match codes {q.shape}")
    return vals * scale


# ---------------------------------------------------------- weight layout --

def blocked_from_canonical(q: np.ndarray) -> np.ndarray:
    """The load-time repack of a packed code matrix uint8 [..., R, K/2]
    (R a multiple of 16): within each group of 16 consecutive rows the bytes
    go block-major, so byte i (0..15) of 32-element MX block b of row r
    moves to offset b*256 + (r % 16)*16 + i of the group's R/16-th share of
    the array (the group's 16 * K/2 bytes stay where they were as a whole).
    Returned in the same shape; the E8M0 scales are not repacked."""
    q = np.asarray(q, dtype=np.uint8)
    R, KH = q.shape[-2:]
    if R % 16 or KH % 16:
        raise ValueError("need rows % 16 == 0 and K % 32 == 0")
    lead = q.shape[:-2]
    groups = q.reshape(lead + (R // 16, 16, KH // 16, 16))  # group, row, block, byte
    return np.ascontiguousarray(np.swapaxes(groups, -3, -2)).reshape(q.shape)


def canonical_from_blocked(qb: np.ndarray) -> np.ndarray:
    """Inverse of blocked_from_canonical."""
    qb = np.asarray(qb, dtype=np.uint8)
    R, KH = qb.shape[-2:]
    if R % 16 or KH % 16:
        raise ValueError("need rows % 16 == 0 and K % 32 == 0")
    lead = qb.shape[:-2]
    groups = qb.reshape(lead + (R // 16, KH // 16, 16, 16))  # group, block, row, byte
    return np.ascontiguousarray(np.swapaxes(groups, -3, -2)).reshape(qb.shape)


# ----------------------------------------------------------------- routing --

def router_logits(x_bits: np.ndarray, w_router: np.ndarray, bias=None) -> np.ndarray:
    """Step 1: L = x Wr^T (+ b), float64 [T, E]."""
    x = bf16_to_f64(x_bits)
    L = x @ np.asarray(w_router, dtype=np.float64).T
    if bias is not None:
        L = L + np.asarray(bias, dtype=np.float64)[None, :]
    return L


def top_k(L: np.ndarray, k: int) -> np.ndarray:
    """Step 2: int32 [T, k] expert ids, descending logit, ties to lower index."""
    T, E = L.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    order = np.argsort(-L, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def softmax_selected(L: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Step 3: softmax over the k selected logits of each token, float64 [T, k]."""
    sel = np.take_along_axis(L, ids.astype(np.int64), axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def sigmoid_selected(L: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Step 3, sigmoid gating: s = 1 / (1 + exp(-L)) of the k selected logits
    of each token, divided by their sum, float64 [T, k]."""
    sel = np.take_along_axis(L, ids.astype(np.int64), axis=1)
    s = 1.0 / (1.0 + np.exp(-sel))
    return s / s.sum(axis=1, keepdims=True)


GATINGS = ("softmax", "sigmoid")


def route(x_bits, w_router, bias, k, gating="softmax"):
    """Steps 1-3. Returns (topk_ids int32 [T,k], topk_weights float64 [T,k], L)."""
    if gating not in GATINGS:
        raise ValueError(f"gating must be one of {GATINGS}")
    L = router_logits(x_bits, w_router, bias)
    ids = top_k(L, k)
    w = softmax_selected(L, ids) if gating == "softmax" else sigmoid_selected(L, ids)
    return ids, w, L


# -------------------------------------------------------------- tile table --

def build_tiles(topk_ids: np.ndarray, E: int, BM: int):
    """Step 4: per-expert tile table (the write-up's "Per-expert routing tile
    table": each expert lays out its own tiles; and "MoE token tile follows
    tokens per expert": BM is the token tile).

    Returns (expert_offsets int32 [E+1], sorted_ids int32 [T*k],
    tiles int32 [num_tiles, 3] of (expert, row_start, rows), num_tiles).
    sorted_ids holds flat slot ids p = t*k + j grouped by expert ascending and
    ascending p within an expert; tile rows index into sorted_ids.
    """
    flat = np.asarray(topk_ids, dtype=np.int64).ravel()
    counts = np.bincount(flat, minlength=E)
    if counts.shape[0] != E:
        raise ValueError("expert id out of range")
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    sorted_ids = np.argsort(flat, kind="stable")
    tiles = []
    for e in range(E):
        c = int(counts[e])
        for i in range(-(-c // BM)):
            tiles.append((e, int(offsets[e]) + i * BM, min(BM, c - i * BM)))
    tiles = np.array(tiles, dtype=np.int32).reshape(-1, 3)
    return (offsets.astype(np.int32), sorted_ids.astype(np.int32), tiles,
            int(tiles.shape[0]))


# ------------------------------------------------------------ expert FFN --

def silu(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(X: np.ndarray, w13_q_e, w13_s_e, w2_q_e, w2_s_e) -> np.ndarray:
    """Steps 5-6 for one expert: X float64 [M, H] -> y float64 [M, H]."""
    W13 = dequant_mxfp4(w13_q_e, w13_s_e)          # [2I, H]
    I = W13.shape[0] // 2
    g = X @ W13[:I].T                               # gate  [M, I]
    u = X @ W13[I:].T                               # up    [M, I]
    h = silu(g) * u
    W2 = dequant_mxfp4(w2_q_e, w2_s_e)             # [H, I]
    return h @ W2.T


# ---------------------------------------- gpt-oss expert form (opt-in) --

GPTOSS_ALPHA = 1.702
GPTOSS_LIMIT = 7.0


def concatenated_from_interleaved(a: np.ndarray, axis: int) -> np.ndarray:
    """Rows interleaved along `axis` (entry 2i: gate of output i, 2i + 1: its
    up) -> gate entries first, then up entries: out[i] = a[2i],
    out[I + i] = a[2i + 1] along that axis."""
    a = np.asarray(a)
    n = a.shape[axis]
    if n % 2:
        raise ValueError("need an even extent along axis")
    gate = np.take(a, np.arange(0, n, 2), axis=axis)
    up = np.take(a, np.arange(1, n, 2), axis=axis)
    return np.ascontiguousarray(np.concatenate([gate, up], axis=axis))


def swiglu_clamped(g: np.ndarray, u: np.ndarray, alpha: float, limit: float) -> np.ndarray:
    """gpt-oss SwiGLU: the gate clamped from above, the up projection on both
    sides, h = g * sigmoid(alpha * g) * (u + 1)."""
    g = np.minimum(g, limit)
    u = np.clip(u, -limit, limit)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-alpha * g)) * (u + 1.0)


def expert_ffn_gptoss(X: np.ndarray, w13_q_e, w13_s_e, w2_q_e, w2_s_e, b13_e, b2_e,
                      alpha: float = GPTOSS_ALPHA, limit: float = GPTOSS_LIMIT) -> np.ndarray:
    """Steps 5-6 for one expert in the gpt-oss form: w13 rows interleaved
    (gate = even rows, up = odd rows), b13_e [2I] in the same order, b2_e [H];
    X float64 [M, H] -> y float64 [M, H]."""
    W13 = dequant_mxfp4(w13_q_e, w13_s_e)            # [2I, H], interleaved rows
    z = X @ W13.T + np.asarray(b13_e, dtype=np.float64)[None, :]
    h = swiglu_clamped(z[:, 0::2], z[:, 1::2], alpha, limit)
    W2 = dequant_mxfp4(w2_q_e, w2_s_e)               # [H, I]
    return h @ W2.T + np.asarray(b2_e, dtype=np.float64)[None, :]


def combine(y: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Step 7: out[t] = sum_j w[t, j] * y[t*k + j] (float64, no rounding)."""
    T, k = w.shape
    return np.einsum("tj,tjh->th", w, y.reshape(T, k, -1))


def moe_layer(inp: dict, BM: int = 16, tokens=None, progress=None) -> dict:
    """The whole layer in float64.

    inp holds x, w_router, bias, w13_q, w13_s, w2_q, w2_s and k (and
    optionally gating, "softmax" when absent; and activation: "swiglu" when
    absent, or "gptoss" with b13, b2 and optionally alpha and limit, which
    runs expert_ffn_gptoss on the weights as given).  With
    ``tokens`` (an index array) only those tokens' outputs are evaluated
    (routing and the tile table still cover every token); experts are
    decoded one at a time so the largest layer stays within memory.
    ``progress``, if given, is called as progress(e, E) after expert e's
    rows are done (for logging only; it sees no values).
    """
    k = int(inp["k"])
    E = inp["w13_q"].shape[0]
    ids, w, L = route(inp["x"], inp["w_router"], inp.get("bias"), k,
                      inp.get("gating", "softmax"))
    offsets, sorted_ids, tiles, num_tiles = build_tiles(ids, E, BM)
    T = ids.shape[0]
    want = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    need_slot = np.zeros(T * k, dtype=bool)
    for t in want:
        need_slot[t * k:(t + 1) * k] = True
    x64 = bf16_to_f64(inp["x"])
    H = x64.shape[1]
    y = np.zeros((T * k, H), dtype=np.float64)
    for e in range(E):
        slots = sorted_ids[offsets[e]:offsets[e + 1]].astype(np.int64)
        slots = slots[need_slot[slots]]
        if slots.size == 0:
            continue
        if inp.get("activation", "swiglu") == "gptoss":
            y[slots] = expert_ffn_gptoss(x64[slots // k], inp["w13_q"][e], inp["w13_s"][e],
                                         inp["w2_q"][e], inp["w2_s"][e], inp["b13"][e],
                                         inp["b2"][e], inp.get("alpha", GPTOSS_ALPHA),
                                         inp.get("limit", GPTOSS_LIMIT))
        else:
            y[slots] = expert_ffn(x64[slots // k], inp["w13_q"][e], inp["w13_s"][e],
                                  inp["w2_q"][e], inp["w2_s"][e])
        if progress is not None:
            progress(e, E)
    out = combine(y, w)
    return dict(topk_ids=ids, topk_weights=w, logits=L, expert_offsets=offsets,
                sorted_ids=sorted_ids, tiles=tiles, num_tiles=num_tiles,
                y=y, out=out[want], tokens=want)
