"""MoeLayer: one MXFP4 MoE layer with every buffer allocated up front.

A call enqueues the library's entry points (moe_route, moe_build_tiles,
moe_forward; for small batches moe_route_tiles + moe_forward; for one token
the single-launch moe_layer_one_token, and on request for 2..4 tokens the
single-launch moe_layer_small_batch) on the current stream with
preallocated outputs and workspaces, so it allocates nothing per call and
can be captured in a HIP graph.  Weights are given as device tensors in the
library's canonical layout (see include/moe_mxfp4.h).  By default
(layout="blocked") the layer repacks the packed codes once, at construction,
into a copy its kernels read in the blocked layout (one contiguous kilobyte
per wave load); layout="canonical" reads the given codes as they are.

activation="gptoss" selects the released gpt-oss expert form
(moe_forward_gptoss: biases b13 [E, 2I] and b2 [E, H], clamped SwiGLU with
alpha and limit).  Its w13 rows (and b13 entries) are taken as a checkpoint
stores them, gate and up of each output adjacent, and are de-interleaved
once at construction (w13_interleaved=False when they already come as the
two halves).  That form runs as separate launches at every batch size.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import binding as B


def _expect(t, name: str, dtypes, shape, device=None):
    """Raises ValueError unless t is a contiguous tensor of one of `dtypes`
    and exactly `shape`, on `device` (when given) and on a GPU.  Shape, dtype
    and layout are checked before the device, so a malformed argument is
    named whatever device it is on; nothing is enqueued either way."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


class MoeLayer:
    def __init__(self, w_router: torch.Tensor, bias: Optional[torch.Tensor],
                 w13_q: torch.Tensor, w13_s: torch.Tensor, w2_q: torch.Tensor,
                 w2_s: torch.Tensor, k: int, gating: str = "softmax",
                 layout: str = "blocked", activation: str = "swiglu",
                 b13: Optional[torch.Tensor] = None, b2: Optional[torch.Tensor] = None,
                 alpha: float = B.GPTOSS_ALPHA, limit: float = B.GPTOSS_LIMIT,
                 w13_interleaved: bool = True):
        if activation not in ("swiglu", "gptoss"):
            raise ValueError("activation must be 'swiglu' or 'gptoss'")
        self.gptoss = activation == "gptoss"
        if not self.gptoss and (b13 is not None or b2 is not None):
            raise ValueError("expert biases need activation='gptoss'")
        self.alpha, self.limit = float(alpha), float(limit)
        self.gating = B.gating_code(gating)
        self.layout = B.layout_code(layout)
        if not isinstance(w13_q, torch.Tensor) or w13_q.dim() != 3:
            raise ValueError("w13_q must be a uint8 tensor [E, 2I, H/2]")
        self.E, I2, Hh = w13_q.shape
        self.H, self.I, self.k = Hh * 2, I2 // 2, int(k)
        if self.H % 32 or self.I % 32 or self.H == 0 or self.I == 0:
            raise ValueError("H and I must be positive multiples of 32")
        if not 1 <= self.k <= min(self.E, 8):
            raise ValueError("k must lie in [1, min(E, 8)]")
        _expect(w_router, "w_router", (torch.float32,), (self.E, self.H))
        self.device = w_router.device
        if bias is not None:
            _expect(bias, "bias", (torch.float32,), (self.E,), self.device)
        self.w_router, self.bias = w_router, bias
        if b13 is not None:
            _expect(b13, "b13", (torch.float32,), (self.E, 2 * self.I), self.device)
        if b2 is not None:
            _expect(b2, "b2", (torch.float32,), (self.E, self.H), self.device)
        if self.gptoss and w13_interleaved:
            _expect(w13_q, "w13_q", (torch.uint8,), (self.E, 2 * self.I, self.H // 2), self.device)
            _expect(w13_s, "w13_s", (torch.uint8,), (self.E, 2 * self.I, self.H // 32),
                    self.device)
            w13_q, w13_s = B.moe_deinterleave_rows(w13_q), B.moe_deinterleave_rows(w13_s)
            if b13 is not None:
                b13 = B.moe_deinterleave_rows(b13)
        self.b13, self.b2 = b13, b2
        self.set_weights(w13_q, w13_s, w2_q, w2_s, repack=True)
        self.T = None

    def set_weights(self, w13_q, w13_s, w2_q, w2_s, repack: bool = False):
        """Point the layer at another copy of the expert weights (same shapes).
        The codes are taken as they are (already in the layer's layout) unless
        repack is set, in which case canonical codes are repacked to it."""
        E, H, I = self.E, self.H, self.I
        _expect(w13_q, "w13_q", (torch.uint8,), (E, 2 * I, H // 2), self.device)
        _expect(w13_s, "w13_s", (torch.uint8,), (E, 2 * I, H // 32), self.device)
        _expect(w2_q, "w2_q", (torch.uint8,), (E, H, I // 2), self.device)
        _expect(w2_s, "w2_s", (torch.uint8,), (E, H, I // 32), self.device)
        if repack and self.layout == B.LAYOUTS["blocked"]:
            w13_q, w2_q = B.moe_repack_weights(w13_q), B.moe_repack_weights(w2_q)
        self.w13_q, self.w13_s, self.w2_q, self.w2_s = w13_q, w13_s, w2_q, w2_s

    def plan(self, T: int, BM: Optional[int] = None, one_launch: bool = True,
             small_batch: bool = False):
        """Allocate every buffer for batches of T tokens.  With one token the
        layer runs as one launch (moe_layer_one_token) unless one_launch is
        False or the shape is outside that entry point's range; with 2..4
        tokens and small_batch set it runs as one launch too
        (moe_layer_small_batch, blocked codes)."""
        dev, E, H, I, k = self.device, self.E, self.H, self.I, self.k
        self.T = T
        self.BM = B.pick_bm(T, k, E) if BM is None else BM
        self.topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.topk_weights = torch.empty((T, k), dtype=torch.float32, device=dev)
        # up to 16 tokens route and tile in one launch (moe_route_tiles: one
        # workgroup); from 17 to 64 tokens that entry point relays between
        # workgroups through tickets, which measured slower than the two
        # separate launches (13.5 vs 11.5 us at 64 tokens), so the layer
        # launches those.  The fused workspace must start zeroed, and every
        # call leaves it that way.
        self.fused = B.route_tiles_ok(T, E, k) and T <= B.ROUTE_TILES_ONE_WG_MAX_T
        ws = B.route_tiles_workspace_bytes(T, H, E) if self.fused else B.route_workspace_bytes(T, H, E)
        self.route_ws = torch.zeros(max(ws, 256), dtype=torch.uint8, device=dev)
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
        self.sorted_ids = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev)
        self.tiles_max = B.tiles_max(T, k, E, self.BM)
        self.tiles = torch.empty((max(self.tiles_max, 1), 3), dtype=torch.int32, device=dev)
        self.num_tiles = torch.zeros(1, dtype=torch.int32, device=dev)
        self.fwd_ws = torch.empty(max(B.forward_workspace_bytes(T, H, I, k), 16),
                                  dtype=torch.uint8, device=dev)
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        one_ws = B.layer_one_token_workspace_bytes(H, I, E, k) if T == 1 else 0
        self.one_launch = bool(one_launch and one_ws > 0 and not self.gptoss)
        # its counters must start zeroed; every call leaves them that way
        self.one_ws = (torch.zeros(one_ws, dtype=torch.uint8, device=dev)
                       if self.one_launch else None)
        # 2..4 tokens (T * k <= 16, blocked codes): the small-batch one launch,
        # only on request: on MI355X it does not beat the separate launches
        # (20b shape: 35.4 against 35.3 us at 2 tokens, 59.4 against 52.7 at
        # 4), so it serves callers bound by the host's enqueue rate
        small_ws = (B.layer_small_batch_workspace_bytes(T, H, I, E, k)
                    if 2 <= T and self.layout == B.LAYOUTS["blocked"] else 0)
        self.small_launch = bool(one_launch and small_batch and small_ws > 0 and not self.gptoss)
        self._launch_opts = dict(one_launch=one_launch, small_batch=small_batch)
        self.small_ws = (torch.zeros(small_ws, dtype=torch.uint8, device=dev)
                         if self.small_launch else None)
        return self

    def _args(self):
        lib = B.load()
        s = ctypes.c_void_p(torch.cuda.current_stream(self.device).cuda_stream)
        return lib, s

    @staticmethod
    def _p(t):
        return None if t is None else ctypes.c_void_p(t.data_ptr())

    def route_only(self, x: torch.Tensor):
        """moe_route (or, for small batches, moe_route_tiles) into the layer's buffers."""
        self.check_input(x)
        if x.shape[0] != self.T:
            raise ValueError(f"x has {x.shape[0]} tokens; the layer is planned for {self.T}")
        lib, s = self._args()
        p = self._p
        T, E, H, k = x.shape[0], self.E, self.H, self.k
        if self.fused:
            B._check(lib.moe_route_tiles(p(x), p(self.w_router), p(self.bias), T, H, E, k,
                                         self.gating, self.BM,
                                         p(self.topk_ids), p(self.topk_weights), None,
                                         p(self.offsets), p(self.sorted_ids), p(self.tiles),
                                         p(self.num_tiles), p(self.route_ws),
                                         self.route_ws.numel(), s), "moe_route_tiles")
            return
        B._check(lib.moe_route(p(x), p(self.w_router), p(self.bias), T, H, E, k, self.gating,
                               p(self.topk_ids), p(self.topk_weights), None, p(self.route_ws),
                               self.route_ws.numel(), s), "moe_route")

    def tiles_only(self):
        """moe_build_tiles from the layer's topk_ids (already done when fused)."""
        if self.fused:
            return
        lib, s = self._args()
        p = self._p
        B._check(lib.moe_build_tiles(p(self.topk_ids), self.T, self.k, self.E, self.BM,
                                     p(self.offsets), p(self.sorted_ids), p(self.tiles),
                                     p(self.num_tiles), s), "moe_build_tiles")

    def _h_y(self):
        n = self.T * self.k
        h_bytes = (n * self.I * 2 + 255) // 256 * 256
        return (self.fwd_ws[:h_bytes], self.fwd_ws[h_bytes:])

    def gateup_only(self, x: torch.Tensor):
        """moe_gateup_swiglu into the layer's h workspace."""
        self.check_input(x)
        if x.shape[0] != self.T:
            raise ValueError(f"x has {x.shape[0]} tokens; the layer is planned for {self.T}")
        lib, s = self._args()
        p = self._p
        h, _ = self._h_y()
        B._check(lib.moe_gateup_swiglu(p(x), p(self.w13_q), p(self.w13_s), p(self.sorted_ids),
                                       p(self.tiles), p(self.num_tiles), self.T, self.H, self.I,
                                       self.E, self.k, self.BM, self.layout, p(h), s),
                 "moe_gateup_swiglu")

    def down_only(self):
        """moe_down from the h workspace into the y workspace."""
        lib, s = self._args()
        p = self._p
        h, y = self._h_y()
        B._check(lib.moe_down(p(h), p(self.w2_q), p(self.w2_s), p(self.sorted_ids), p(self.tiles),
                              p(self.num_tiles), self.T, self.H, self.I, self.E, self.k, self.BM,
                              self.layout, p(y), s), "moe_down")

    def combine_only(self):
        """moe_combine from the y workspace into the layer's output."""
        lib, s = self._args()
        p = self._p
        _, y = self._h_y()
        B._check(lib.moe_combine(p(y), p(self.topk_weights), self.T, self.H, self.k, p(self.out),
                                 s), "moe_combine")

    def check_input(self, x: torch.Tensor):
        """Raises ValueError unless x is a contiguous bf16 [T, H] tensor (or its
        bits as int16 or uint16) on the
        layer's device (the kernels read T*H elements of it)."""
        if not isinstance(x, torch.Tensor) or x.dim() != 2:
            raise ValueError("x must be a bf16 tensor [T, H]")
        _expect(x, "x", B._BF16, (x.shape[0], self.H), self.device)

    def __call__(self, x: torch.Tensor) -> torch.Tensor:
        """One layer call: routing and tiles, then moe_forward (one launch for
        one token).  x: contiguous bf16 [T, H] on the layer's device."""
        self.check_input(x)
        T = x.shape[0]
        if self.T != T:
            self.plan(T, **getattr(self, "_launch_opts", {}))
        lib, s = self._args()
        p = self._p
        E, H, I, k, BM = self.E, self.H, self.I, self.k, self.BM
        if self.one_launch:
            B._check(lib.moe_layer_one_token(p(x), p(self.w_router), p(self.bias), p(self.w13_q),
                                             p(self.w13_s), p(self.w2_q), p(self.w2_s), H, I, E,
                                             k, self.gating, self.layout, p(self.topk_ids),
                                             p(self.topk_weights), None,
                                             p(self.offsets), p(self.sorted_ids), p(self.tiles),
                                             p(self.num_tiles), p(self.one_ws),
                                             self.one_ws.numel(), p(self.out), s),
                     "moe_layer_one_token")
            return self.out
        if self.small_launch:
            B._check(lib.moe_layer_small_batch(p(x), p(self.w_router), p(self.bias),
                                               p(self.w13_q), p(self.w13_s), p(self.w2_q),
                                               p(self.w2_s), T, H, I, E, k, self.gating,
                                               self.layout, p(self.topk_ids),
                                               p(self.topk_weights), None, p(self.offsets),
                                               p(self.sorted_ids), p(self.tiles),
                                               p(self.num_tiles), p(self.small_ws),
                                               self.small_ws.numel(), p(self.out), s),
                     "moe_layer_small_batch")
            return self.out
        self.route_only(x)
        self.tiles_only()
        if self.gptoss:
            B._check(lib.moe_forward_gptoss(p(x), p(self.w13_q), p(self.w13_s), p(self.w2_q),
                                            p(self.w2_s), p(self.b13), p(self.b2), self.alpha,
                                            self.limit, p(self.topk_weights), p(self.sorted_ids),
                                            p(self.tiles), p(self.num_tiles), T, H, I, E, k, BM,
                                            self.layout, p(self.fwd_ws), self.fwd_ws.numel(),
                                            p(self.out), s), "moe_forward_gptoss")
            return self.out
        B._check(lib.moe_forward(p(x), p(self.w13_q), p(self.w13_s), p(self.w2_q), p(self.w2_s),
                                 p(self.topk_weights), p(self.sorted_ids), p(self.tiles),
                                 p(self.num_tiles), T, H, I, E, k, BM, self.layout, p(self.fwd_ws),
                                 self.fwd_ws.numel(), p(self.out), s), "moe_forward")
        return self.out
