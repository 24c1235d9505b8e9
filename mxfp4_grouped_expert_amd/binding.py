"""Thin ctypes binding of libmoe_mxfp4.so (argument marshalling only).

Every step of the layer runs in the HIP library; this module only allocates
outputs and workspaces with torch on the tensors' device, passes their device
pointers and the current stream, and turns a non-OK status into an exception.
There is no fallback: if the library is missing, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mxfp4.so")

MOE_OK = 0
_lib = None

_p = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t


class MoeError(RuntimeError):
    """A library call returned a non-OK moe_status."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


def load() -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m mxfp4_grouped_expert_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.moe_status_string.argtypes = [_i]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_version.argtypes = []
    lib.moe_version.restype = ctypes.c_char_p
    lib.moe_pick_bm.argtypes = [_i, _i, _i]
    lib.moe_pick_bm.restype = _i
    lib.moe_tiles_max.argtypes = [_i, _i, _i, _i]
    lib.moe_tiles_max.restype = ctypes.c_int64
    lib.moe_route_workspace_bytes.argtypes = [_i, _i, _i]
    lib.moe_route_workspace_bytes.restype = _sz
    lib.moe_forward_workspace_bytes.argtypes = [_i, _i, _i, _i]
    lib.moe_forward_workspace_bytes.restype = _sz
    lib.moe_route.argtypes = [_p, _p, _p, _i, _i, _i, _i, _i, _p, _p, _p, _p, _sz, _p]
    lib.moe_route.restype = _i
    lib.moe_build_tiles.argtypes = [_p, _i, _i, _i, _i, _p, _p, _p, _p, _p]
    lib.moe_build_tiles.restype = _i
    lib.moe_forward.argtypes = [_p, _p, _p, _p, _p, _p, _p, _p, _p,
                                _i, _i, _i, _i, _i, _i, _i, _p, _sz, _p, _p]
    lib.moe_forward.restype = _i
    lib.moe_route_tiles_workspace_bytes.argtypes = [_i, _i, _i]
    lib.moe_route_tiles_workspace_bytes.restype = _sz
    lib.moe_route_tiles.argtypes = [_p, _p, _p, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p,
                                    _p, _sz, _p]
    lib.moe_route_tiles.restype = _i
    lib.moe_gateup_swiglu.argtypes = [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _p, _p]
    lib.moe_gateup_swiglu.restype = _i
    lib.moe_down.argtypes = [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _p, _p]
    lib.moe_down.restype = _i
    lib.moe_combine.argtypes = [_p, _p, _i, _i, _i, _p, _p]
    lib.moe_combine.restype = _i
    lib.moe_layer_one_token_workspace_bytes.argtypes = [_i, _i, _i, _i]
    lib.moe_layer_one_token_workspace_bytes.restype = _sz
    lib.moe_layer_one_token_sync_bytes.argtypes = [_i]
    lib.moe_layer_one_token_sync_bytes.restype = _sz
    lib.moe_layer_one_token.argtypes = [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i,
                                        _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p, _p]
    lib.moe_layer_one_token.restype = _i
    lib.moe_layer_small_batch_workspace_bytes.argtypes = [_i, _i, _i, _i, _i]
    lib.moe_layer_small_batch_workspace_bytes.restype = _sz
    lib.moe_layer_small_batch_sync_bytes.argtypes = []
    lib.moe_layer_small_batch_sync_bytes.restype = _sz
    lib.moe_layer_small_batch.argtypes = [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i,
                                          _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p, _p]
    lib.moe_layer_small_batch.restype = _i
    lib.moe_forward_static_workspace.argtypes = [_p, _p, _p, _p, _p, _p, _p, _p, _p,
                                                 _i, _i, _i, _i, _i, _i, _i, _p, _p]
    lib.moe_forward_static_workspace.restype = _i
    lib.moe_forward_gptoss.argtypes = [_p, _p, _p, _p, _p, _p, _p, ctypes.c_float,
                                       ctypes.c_float, _p, _p, _p, _p,
                                       _i, _i, _i, _i, _i, _i, _i, _p, _sz, _p, _p]
    lib.moe_forward_gptoss.restype = _i
    lib.moe_deinterleave_rows.argtypes = [_p, _i, _i, _i, _p, _p]
    lib.moe_deinterleave_rows.restype = _i
    lib.moe_repack_weights.argtypes = [_p, ctypes.c_int64, _i, _p, _p]
    lib.moe_repack_weights.restype = _i
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().moe_status_string(int(status)).decode()


def version() -> str:
    return load().moe_version().decode()


def pick_bm(T: int, k: int, E: int) -> int:
    return int(load().moe_pick_bm(T, k, E))


def tiles_max(T: int, k: int, E: int, BM: int) -> int:
    return int(load().moe_tiles_max(T, k, E, BM))


def route_workspace_bytes(T: int, H: int, E: int) -> int:
    return int(load().moe_route_workspace_bytes(T, H, E))


def forward_workspace_bytes(T: int, H: int, I: int, k: int) -> int:
    return int(load().moe_forward_workspace_bytes(T, H, I, k))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoeError(status, where)


def _need(t: torch.Tensor, name: str, dtypes, device=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtypes and t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_U8 = (torch.uint8,)


def _workspace(nbytes: int, device) -> torch.Tensor:
    # 16-byte aligned device buffer (torch's allocator aligns to >= 256 bytes)
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


GATINGS = {"softmax": 0, "sigmoid": 1}  # MOE_GATING_SOFTMAX, MOE_GATING_SIGMOID


def gating_code(gating: str) -> int:
    if gating not in GATINGS:
        raise ValueError(f"gating must be one of {sorted(GATINGS)}")
    return GATINGS[gating]


LAYOUTS = {"canonical": 0, "blocked": 1}  # MOE_LAYOUT_CANONICAL, MOE_LAYOUT_BLOCKED


def layout_code(layout: str) -> int:
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(LAYOUTS)}")
    return LAYOUTS[layout]


def moe_repack_weights(q: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Packed codes (w13_q [E, 2I, H/2] or w2_q [E, H, I/2], canonical) ->
    the same bytes in the blocked layout, as a new tensor of the same shape."""
    _need(q, "q", _U8)
    K = q.shape[-1] * 2
    rows = q.numel() // q.shape[-1]
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", _U8, q.device)
    if out.shape != q.shape:
        raise ValueError("out must have the shape of q")
    _check(load().moe_repack_weights(_ptr(q), rows, K, _ptr(out), _stream(q.device)),
           "moe_repack_weights")
    return out


def moe_route(x: torch.Tensor, w_router: torch.Tensor, bias: Optional[torch.Tensor], k: int,
              want_logits: bool = False, workspace: Optional[torch.Tensor] = None,
              gating: str = "softmax"):
    """Router logits (fp64) -> top-k -> gating (softmax, or sigmoid normalised
    over the k) of the k selected logits.

    x: bf16 [T, H] (or its bits as int16/uint16); w_router: fp32 [E, H];
    bias: fp32 [E] or None.  Returns (topk_ids int32 [T, k],
    topk_weights fp32 [T, k], logits fp64 [T, E] or None).
    """
    _need(x, "x", _BF16)
    dev = x.device
    _need(w_router, "w_router", (torch.float32,), dev)
    if bias is not None:
        _need(bias, "bias", (torch.float32,), dev)
    T, H = x.shape
    E = w_router.shape[0]
    if w_router.shape[1] != H or (bias is not None and bias.shape[0] != E):
        raise ValueError("router shapes do not match x")
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    wts = torch.empty((T, k), dtype=torch.float32, device=dev)
    logits = torch.empty((T, E), dtype=torch.float64, device=dev) if want_logits else None
    nbytes = route_workspace_bytes(T, H, E)
    if workspace is None:
        workspace = _workspace(nbytes, dev)
    _check(load().moe_route(_ptr(x), _ptr(w_router), _ptr(bias), T, H, E, k, gating_code(gating),
                            _ptr(ids),
                            _ptr(wts), _ptr(logits), _ptr(workspace), workspace.numel(),
                            _stream(dev)), "moe_route")
    return ids, wts, logits


def route_tiles_workspace_bytes(T: int, H: int, E: int) -> int:
    return int(load().moe_route_tiles_workspace_bytes(T, H, E))


# largest batch that moe_route_tiles routes and tiles in one workgroup
ROUTE_TILES_ONE_WG_MAX_T = 16


def route_tiles_ok(T: int, E: int, k: int) -> bool:
    """Whether the fused decode routing entry point accepts this batch."""
    return T <= 64


def zeroed_route_tiles_workspace(T: int, H: int, E: int, device) -> torch.Tensor:
    """A zeroed workspace for moe_route_tiles (it must start zero; every call
    leaves its sync block and hand-off words zero)."""
    return torch.zeros(max(route_tiles_workspace_bytes(T, H, E), 256), dtype=torch.uint8,
                       device=device)


def moe_route_tiles(x: torch.Tensor, w_router: torch.Tensor, bias: Optional[torch.Tensor],
                    k: int, BM: int, want_logits: bool = False,
                    workspace: Optional[torch.Tensor] = None, gating: str = "softmax"):
    """Fused decode routing + tile table.  Returns (topk_ids, topk_weights,
    logits or None, expert_offsets, sorted_ids, tiles, num_tiles)."""
    _need(x, "x", _BF16)
    dev = x.device
    _need(w_router, "w_router", (torch.float32,), dev)
    if bias is not None:
        _need(bias, "bias", (torch.float32,), dev)
    T, H = x.shape
    E = w_router.shape[0]
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    wts = torch.empty((T, k), dtype=torch.float32, device=dev)
    logits = torch.empty((T, E), dtype=torch.float64, device=dev) if want_logits else None
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sorted_ids = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev)[:T * k]
    tiles = torch.empty((max(tiles_max(T, k, E, BM), 1), 3), dtype=torch.int32, device=dev)
    num_tiles = torch.zeros(1, dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = zeroed_route_tiles_workspace(T, H, E, dev)
    _check(load().moe_route_tiles(_ptr(x), _ptr(w_router), _ptr(bias), T, H, E, k,
                                  gating_code(gating), BM, _ptr(ids),
                                  _ptr(wts), _ptr(logits), _ptr(offsets), _ptr(sorted_ids),
                                  _ptr(tiles), _ptr(num_tiles), _ptr(workspace),
                                  workspace.numel(), _stream(dev)), "moe_route_tiles")
    return ids, wts, logits, offsets, sorted_ids, tiles, num_tiles


def layer_one_token_workspace_bytes(H: int, I: int, E: int, k: int) -> int:
    """Workspace bytes of moe_layer_one_token; 0 if the shape is not accepted."""
    return int(load().moe_layer_one_token_workspace_bytes(H, I, E, k))


def layer_one_token_sync_bytes(H: int) -> int:
    """Bytes at the start of that workspace that must be zero before first use."""
    return int(load().moe_layer_one_token_sync_bytes(H))


def zeroed_layer_one_token_workspace(H: int, I: int, E: int, k: int, device) -> torch.Tensor:
    """A workspace for moe_layer_one_token whose sync block starts at zero."""
    return torch.zeros(max(layer_one_token_workspace_bytes(H, I, E, k), 256), dtype=torch.uint8,
                       device=device)


def moe_layer_one_token(x: torch.Tensor, w_router: torch.Tensor, bias: Optional[torch.Tensor],
                        w13_q: torch.Tensor, w13_s: torch.Tensor, w2_q: torch.Tensor,
                        w2_s: torch.Tensor, k: int, BM: int, want_logits: bool = False,
                        workspace: Optional[torch.Tensor] = None,
                        out: Optional[torch.Tensor] = None, gating: str = "softmax",
                        layout: str = "canonical"):
    """The whole layer for one token in one launch.  Returns (out bf16 [1, H],
    topk_ids, topk_weights, logits or None, expert_offsets, sorted_ids, tiles,
    num_tiles), each equal to what moe_route_tiles + moe_forward produce."""
    _need(x, "x", _BF16)
    dev = x.device
    _need(w_router, "w_router", (torch.float32,), dev)
    if bias is not None:
        _need(bias, "bias", (torch.float32,), dev)
    for name, t in (("w13_q", w13_q), ("w13_s", w13_s), ("w2_q", w2_q), ("w2_s", w2_s)):
        _need(t, name, _U8, dev)
    T, H = x.shape
    if T != 1:
        raise ValueError("moe_layer_one_token takes exactly one token")
    E, I2, _ = w13_q.shape
    I = I2 // 2
    ids = torch.empty((1, k), dtype=torch.int32, device=dev)
    wts = torch.empty((1, k), dtype=torch.float32, device=dev)
    logits = torch.empty((1, E), dtype=torch.float64, device=dev) if want_logits else None
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sorted_ids = torch.empty(k, dtype=torch.int32, device=dev)
    tiles = torch.empty((max(tiles_max(1, k, E, BM), 1), 3), dtype=torch.int32, device=dev)
    num_tiles = torch.zeros(1, dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty((1, H), dtype=torch.bfloat16, device=dev)
    _need(out, "out", _BF16, dev)
    if workspace is None:
        workspace = zeroed_layer_one_token_workspace(H, I, E, k, dev)
    _check(load().moe_layer_one_token(_ptr(x), _ptr(w_router), _ptr(bias), _ptr(w13_q),
                                      _ptr(w13_s), _ptr(w2_q), _ptr(w2_s), H, I, E, k,
                                      gating_code(gating), layout_code(layout), _ptr(ids),
                                      _ptr(wts), _ptr(logits), _ptr(offsets), _ptr(sorted_ids),
                                      _ptr(tiles), _ptr(num_tiles), _ptr(workspace),
                                      workspace.numel(), _ptr(out), _stream(dev)),
           "moe_layer_one_token")
    return out, ids, wts, logits, offsets, sorted_ids, tiles, num_tiles


def layer_small_batch_workspace_bytes(T: int, H: int, I: int, E: int, k: int) -> int:
    """Workspace bytes of moe_layer_small_batch; 0 if the shape is not accepted."""
    return int(load().moe_layer_small_batch_workspace_bytes(T, H, I, E, k))


def layer_small_batch_sync_bytes() -> int:
    """Bytes at the start of that workspace that must be zero before first use."""
    return int(load().moe_layer_small_batch_sync_bytes())


def zeroed_layer_small_batch_workspace(T: int, H: int, I: int, E: int, k: int,
                                       device) -> torch.Tensor:
    """A workspace for moe_layer_small_batch whose sync block starts at zero."""
    return torch.zeros(max(layer_small_batch_workspace_bytes(T, H, I, E, k), 256),
                       dtype=torch.uint8, device=device)


def moe_layer_small_batch(x: torch.Tensor, w_router: torch.Tensor, bias: Optional[torch.Tensor],
                          w13_q: torch.Tensor, w13_s: torch.Tensor, w2_q: torch.Tensor,
                          w2_s: torch.Tensor, k: int, BM: int, want_logits: bool = False,
                          workspace: Optional[torch.Tensor] = None,
                          out: Optional[torch.Tensor] = None, gating: str = "softmax"):
    """The whole layer for 2..4 tokens in one launch (codes in the blocked
    layout).  Returns (out bf16 [T, H], topk_ids, topk_weights, logits or
    None, expert_offsets, sorted_ids, tiles, num_tiles), each equal to what
    moe_route_tiles + moe_forward produce."""
    _need(x, "x", _BF16)
    dev = x.device
    _need(w_router, "w_router", (torch.float32,), dev)
    if bias is not None:
        _need(bias, "bias", (torch.float32,), dev)
    for name, t in (("w13_q", w13_q), ("w13_s", w13_s), ("w2_q", w2_q), ("w2_s", w2_s)):
        _need(t, name, _U8, dev)
    T, H = x.shape
    E, I2, _ = w13_q.shape
    I = I2 // 2
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    wts = torch.empty((T, k), dtype=torch.float32, device=dev)
    logits = torch.empty((T, E), dtype=torch.float64, device=dev) if want_logits else None
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sorted_ids = torch.empty(T * k, dtype=torch.int32, device=dev)
    tiles = torch.empty((max(tiles_max(T, k, E, BM), 1), 3), dtype=torch.int32, device=dev)
    num_tiles = torch.zeros(1, dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _need(out, "out", _BF16, dev)
    if workspace is None:
        workspace = zeroed_layer_small_batch_workspace(T, H, I, E, k, dev)
    _check(load().moe_layer_small_batch(_ptr(x), _ptr(w_router), _ptr(bias), _ptr(w13_q),
                                        _ptr(w13_s), _ptr(w2_q), _ptr(w2_s), T, H, I, E, k,
                                        gating_code(gating), LAYOUTS["blocked"], _ptr(ids),
                                        _ptr(wts), _ptr(logits), _ptr(offsets), _ptr(sorted_ids),
                                        _ptr(tiles), _ptr(num_tiles), _ptr(workspace),
                                        workspace.numel(), _ptr(out), _stream(dev)),
           "moe_layer_small_batch")
    return out, ids, wts, logits, offsets, sorted_ids, tiles, num_tiles


def moe_build_tiles(topk_ids: torch.Tensor, E: int, BM: int):
    """Per-expert tile table.  Returns (expert_offsets int32 [E+1],
    sorted_ids int32 [T*k], tiles int32 [tiles_max, 3], num_tiles int32 [1])."""
    _need(topk_ids, "topk_ids", (torch.int32,))
    dev = topk_ids.device
    T, k = topk_ids.shape
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sorted_ids = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev)[:T * k]
    tiles = torch.empty((max(tiles_max(T, k, E, BM), 1), 3), dtype=torch.int32, device=dev)
    num_tiles = torch.zeros(1, dtype=torch.int32, device=dev)
    _check(load().moe_build_tiles(_ptr(topk_ids), T, k, E, BM, _ptr(offsets), _ptr(sorted_ids),
                                  _ptr(tiles), _ptr(num_tiles), _stream(dev)), "moe_build_tiles")
    return offsets, sorted_ids, tiles, num_tiles


def moe_forward(x: torch.Tensor, w13_q: torch.Tensor, w13_s: torch.Tensor, w2_q: torch.Tensor,
                w2_s: torch.Tensor, topk_weights: torch.Tensor, sorted_ids: torch.Tensor,
                tiles: torch.Tensor, num_tiles: torch.Tensor, BM: int,
                out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None,
                layout: str = "canonical") -> torch.Tensor:
    """Grouped gate/up + SwiGLU, grouped down, weighted combine.  Returns
    out bf16 [T, H]."""
    _need(x, "x", _BF16)
    dev = x.device
    for name, t in (("w13_q", w13_q), ("w13_s", w13_s), ("w2_q", w2_q), ("w2_s", w2_s)):
        _need(t, name, _U8, dev)
    _need(topk_weights, "topk_weights", (torch.float32,), dev)
    _need(sorted_ids, "sorted_ids", (torch.int32,), dev)
    _need(tiles, "tiles", (torch.int32,), dev)
    _need(num_tiles, "num_tiles", (torch.int32,), dev)
    T, H = x.shape
    E, I2, Hh = w13_q.shape
    I = I2 // 2
    k = topk_weights.shape[1]
    if (Hh * 2 != H or tuple(w13_s.shape) != (E, 2 * I, H // 32)
            or tuple(w2_q.shape) != (E, H, I // 2) or tuple(w2_s.shape) != (E, H, I // 32)):
        raise ValueError("weight shapes do not match x")
    if topk_weights.shape[0] != T or sorted_ids.numel() != T * k:
        raise ValueError("routing tensors do not match x")
    if tiles.shape[0] < tiles_max(T, k, E, BM):
        raise ValueError("tiles has fewer rows than moe_tiles_max")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _need(out, "out", _BF16, dev)
    nbytes = forward_workspace_bytes(T, H, I, k)
    if workspace is None:
        workspace = _workspace(nbytes, dev)
    _check(load().moe_forward(_ptr(x), _ptr(w13_q), _ptr(w13_s), _ptr(w2_q), _ptr(w2_s),
                              _ptr(topk_weights), _ptr(sorted_ids), _ptr(tiles), _ptr(num_tiles),
                              T, H, I, E, k, BM, layout_code(layout), _ptr(workspace),
                              workspace.numel(), _ptr(out),
                              _stream(dev)), "moe_forward")
    return out


def moe_deinterleave_rows(src: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Rows interleaved in gate/up pairs -> gate rows first, then up rows, per
    expert: src [E, 2I, ...] (w13_q, w13_s, or b13 as fp32 [E, 2I]).  Returns
    a new tensor of the same shape (bytes moved, nothing converted)."""
    _need(src, "src", None)
    if src.dim() < 2 or src.shape[1] % 2:
        raise ValueError("src must be [E, 2I, ...]")
    E, I2 = src.shape[0], src.shape[1]
    row_bytes = src[0, 0].numel() * src.element_size()
    if out is None:
        out = torch.empty_like(src)
    _need(out, "out", (src.dtype,), src.device)
    if out.shape != src.shape:
        raise ValueError("out must have the shape of src")
    _check(load().moe_deinterleave_rows(_ptr(src), E, I2 // 2, row_bytes, _ptr(out),
                                        _stream(src.device)), "moe_deinterleave_rows")
    return out


GPTOSS_ALPHA, GPTOSS_LIMIT = 1.702, 7.0


def moe_forward_gptoss(x: torch.Tensor, w13_q: torch.Tensor, w13_s: torch.Tensor,
                       w2_q: torch.Tensor, w2_s: torch.Tensor, b13: Optional[torch.Tensor],
                       b2: Optional[torch.Tensor], topk_weights: torch.Tensor,
                       sorted_ids: torch.Tensor, tiles: torch.Tensor, num_tiles: torch.Tensor,
                       BM: int, alpha: float = GPTOSS_ALPHA, limit: float = GPTOSS_LIMIT,
                       out: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None,
                       layout: str = "canonical") -> torch.Tensor:
    """moe_forward with the gpt-oss expert form.  w13_q/w13_s and b13 are in
    the kernels' row order (gate rows, then up rows: moe_deinterleave_rows of
    a checkpoint's interleaved rows).  Returns out bf16 [T, H]."""
    _need(x, "x", _BF16)
    dev = x.device
    for name, t in (("w13_q", w13_q), ("w13_s", w13_s), ("w2_q", w2_q), ("w2_s", w2_s)):
        _need(t, name, _U8, dev)
    _need(topk_weights, "topk_weights", (torch.float32,), dev)
    _need(sorted_ids, "sorted_ids", (torch.int32,), dev)
    _need(tiles, "tiles", (torch.int32,), dev)
    _need(num_tiles, "num_tiles", (torch.int32,), dev)
    T, H = x.shape
    E, I2, Hh = w13_q.shape
    I = I2 // 2
    k = topk_weights.shape[1]
    if (Hh * 2 != H or tuple(w13_s.shape) != (E, 2 * I, H // 32)
            or tuple(w2_q.shape) != (E, H, I // 2) or tuple(w2_s.shape) != (E, H, I // 32)):
        raise ValueError("weight shapes do not match x")
    if b13 is not None:
        _need(b13, "b13", (torch.float32,), dev)
        if tuple(b13.shape) != (E, 2 * I):
            raise ValueError("b13 must be fp32 [E, 2I]")
    if b2 is not None:
        _need(b2, "b2", (torch.float32,), dev)
        if tuple(b2.shape) != (E, H):
            raise ValueError("b2 must be fp32 [E, H]")
    if topk_weights.shape[0] != T or sorted_ids.numel() != T * k:
        raise ValueError("routing tensors do not match x")
    if tiles.shape[0] < tiles_max(T, k, E, BM):
        raise ValueError("tiles has fewer rows than moe_tiles_max")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _need(out, "out", _BF16, dev)
    if workspace is None:
        workspace = _workspace(forward_workspace_bytes(T, H, I, k), dev)
    _check(load().moe_forward_gptoss(_ptr(x), _ptr(w13_q), _ptr(w13_s), _ptr(w2_q), _ptr(w2_s),
                                     _ptr(b13), _ptr(b2), float(alpha), float(limit),
                                     _ptr(topk_weights), _ptr(sorted_ids), _ptr(tiles),
                                     _ptr(num_tiles), T, H, I, E, k, BM, layout_code(layout),
                                     _ptr(workspace), workspace.numel(), _ptr(out),
                                     _stream(dev)), "moe_forward_gptoss")
    return out


STATIC_WORKSPACE_BYTES = 16 << 20  # MOE_STATIC_WORKSPACE_BYTES


def moe_forward_static_workspace(x: torch.Tensor, w13_q: torch.Tensor, w13_s: torch.Tensor,
                                 w2_q: torch.Tensor, w2_s: torch.Tensor,
                                 topk_weights: torch.Tensor, sorted_ids: torch.Tensor,
                                 tiles: torch.Tensor, num_tiles: torch.Tensor, BM: int,
                                 out: torch.Tensor, layout: str = "canonical") -> torch.Tensor:
    """moe_forward with the library's own per-device workspace: allocates
    nothing (out must be given).  Returns out."""
    _need(x, "x", _BF16)
    dev = x.device
    for name, t in (("w13_q", w13_q), ("w13_s", w13_s), ("w2_q", w2_q), ("w2_s", w2_s)):
        _need(t, name, _U8, dev)
    _need(topk_weights, "topk_weights", (torch.float32,), dev)
    _need(sorted_ids, "sorted_ids", (torch.int32,), dev)
    _need(tiles, "tiles", (torch.int32,), dev)
    _need(num_tiles, "num_tiles", (torch.int32,), dev)
    _need(out, "out", _BF16, dev)
    T, H = x.shape
    E, I2, Hh = w13_q.shape
    I = I2 // 2
    k = topk_weights.shape[1]
    if (Hh * 2 != H or tuple(w13_s.shape) != (E, 2 * I, H // 32)
            or tuple(w2_q.shape) != (E, H, I // 2) or tuple(w2_s.shape) != (E, H, I // 32)):
        raise ValueError("weight shapes do not match x")
    if topk_weights.shape[0] != T or sorted_ids.numel() != T * k or tuple(out.shape) != (T, H):
        raise ValueError("routing tensors or out do not match x")
    if tiles.shape[0] < tiles_max(T, k, E, BM):
        raise ValueError("tiles has fewer rows than moe_tiles_max")
    _check(load().moe_forward_static_workspace(_ptr(x), _ptr(w13_q), _ptr(w13_s), _ptr(w2_q),
                                               _ptr(w2_s), _ptr(topk_weights), _ptr(sorted_ids),
                                               _ptr(tiles), _ptr(num_tiles), T, H, I, E, k, BM,
                                               layout_code(layout), _ptr(out), _stream(dev)),
           "moe_forward_static_workspace")
    return out


def moe_gateup_swiglu(x, w13_q, w13_s, sorted_ids, tiles, num_tiles, k: int, BM: int,
                      h: Optional[torch.Tensor] = None, layout: str = "canonical") -> torch.Tensor:
    """Grouped gate/up GEMM + SwiGLU.  Returns h bf16 [T*k, I] in tile order."""
    _need(x, "x", _BF16)
    dev = x.device
    T, H = x.shape
    E, I2, _ = w13_q.shape
    I = I2 // 2
    if h is None:
        h = torch.empty((T * k, I), dtype=torch.bfloat16, device=dev)
    _need(h, "h", _BF16, dev)
    _check(load().moe_gateup_swiglu(_ptr(x), _ptr(w13_q), _ptr(w13_s), _ptr(sorted_ids),
                                    _ptr(tiles), _ptr(num_tiles), T, H, I, E, k, BM,
                                    layout_code(layout), _ptr(h),
                                    _stream(dev)), "moe_gateup_swiglu")
    return h


def moe_down(h, w2_q, w2_s, sorted_ids, tiles, num_tiles, T: int, k: int, BM: int,
             y: Optional[torch.Tensor] = None, layout: str = "canonical") -> torch.Tensor:
    """Grouped down GEMM.  Returns y fp32 [T*k, H] indexed by flat slot id."""
    _need(h, "h", _BF16)
    dev = h.device
    E, H, Ih = w2_q.shape
    I = Ih * 2
    if y is None:
        y = torch.empty((T * k, H), dtype=torch.float32, device=dev)
    _need(y, "y", (torch.float32,), dev)
    _check(load().moe_down(_ptr(h), _ptr(w2_q), _ptr(w2_s), _ptr(sorted_ids), _ptr(tiles),
                           _ptr(num_tiles), T, H, I, E, k, BM, layout_code(layout), _ptr(y),
                           _stream(dev)),
           "moe_down")
    return y


def moe_combine(y: torch.Tensor, topk_weights: torch.Tensor,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Weighted combine back to token order.  Returns out bf16 [T, H]."""
    _need(y, "y", (torch.float32,))
    dev = y.device
    T, k = topk_weights.shape
    H = y.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _need(out, "out", _BF16, dev)
    _check(load().moe_combine(_ptr(y), _ptr(topk_weights), T, H, k, _ptr(out), _stream(dev)),
           "moe_combine")
    return out
