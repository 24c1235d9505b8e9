"""MI355X (gfx950) MXFP4 grouped-expert MoE layer.

The layer runs as three calls of the HIP library libmoe_mxfp4.so (see
include/moe_mxfp4.h): moe_route, moe_build_tiles and moe_forward.  This
package is the thin Python binding over them; torch provides device memory
and streams only.
"""
from .binding import (MoeError, LIB_PATH, load, version, status_string, pick_bm, tiles_max,
                      route_workspace_bytes, forward_workspace_bytes, moe_route,
                      moe_build_tiles, moe_forward, moe_gateup_swiglu, moe_down, moe_combine,
                      moe_route_tiles, route_tiles_ok, route_tiles_workspace_bytes,
                      zeroed_route_tiles_workspace, moe_layer_one_token,
                      layer_one_token_workspace_bytes, layer_one_token_sync_bytes,
                      zeroed_layer_one_token_workspace, moe_layer_small_batch,
                      layer_small_batch_workspace_bytes, layer_small_batch_sync_bytes,
                      zeroed_layer_small_batch_workspace, moe_repack_weights, LAYOUTS,
                      GATINGS, moe_forward_static_workspace, STATIC_WORKSPACE_BYTES,
                      moe_forward_gptoss, moe_deinterleave_rows, GPTOSS_ALPHA, GPTOSS_LIMIT)
from .layer import MoeLayer

__all__ = ["MoeError", "LIB_PATH", "load", "version", "status_string", "pick_bm", "tiles_max",
           "route_workspace_bytes", "forward_workspace_bytes", "moe_route", "moe_build_tiles",
           "moe_forward", "moe_gateup_swiglu", "moe_down", "moe_combine", "moe_route_tiles",
           "route_tiles_ok", "route_tiles_workspace_bytes", "zeroed_route_tiles_workspace",
           "moe_layer_one_token", "layer_one_token_workspace_bytes", "layer_one_token_sync_bytes",
           "zeroed_layer_one_token_workspace", "moe_layer_small_batch",
           "layer_small_batch_workspace_bytes", "layer_small_batch_sync_bytes",
           "zeroed_layer_small_batch_workspace", "moe_repack_weights", "LAYOUTS", "GATINGS",
           "moe_forward_static_workspace", "STATIC_WORKSPACE_BYTES", "moe_forward_gptoss",
           "moe_deinterleave_rows", "GPTOSS_ALPHA", "GPTOSS_LIMIT", "MoeLayer"]
