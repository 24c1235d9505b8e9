// Internal launchers, one per kernel.  Callers (moe_api.hip) validate every
// argument first; these only size grids and enqueue on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// The expert activation of the gate/up epilogue, and the expert biases.
// kind 0: the SwiGLU of the pages, h = silu(g) * u, no biases (b13 and b2
// ignored).  kind 1: the gpt-oss form: g and u get their w13 row's bias
// (b13 [E][2I] in the kernels' row order: gate n at [e][n], up n at
// [e][I + n]), then h = min(g, limit) * sigmoid(alpha * min(g, limit)) *
// (clip(u, -limit, limit) + 1); the down output gets its w2 row's bias (b2
// [E][H]).  Null bias pointers mean zero biases.
struct ExpertAct {
  const float* b13;
  const float* b2;
  float alpha;
  float limit;
  int kind;
};
inline ExpertAct plain_swiglu() { return ExpertAct{nullptr, nullptr, 1.0f, 0.0f, 0}; }

// Router: fp64 partial logits over `splits` K-ranges, then top-k + softmax.
struct RouterPlan {
  int splits;      // number of K-ranges
  int split_len;   // elements per K-range (multiple of 4)
};
RouterPlan router_plan(int T, int H, int E);
size_t router_partial_bytes(int T, int H, int E);
void launch_router_logits(const uint16_t* x, const float* w_router, int T, int H, int E,
                          const RouterPlan& plan, double* partial, hipStream_t stream);
// gating: 0 softmax, 1 sigmoid (normalised over the k selected)
void launch_router_topk(const double* partial, const float* bias, int T, int E, int k,
                        int gating, int splits, int32_t* topk_ids, float* topk_weights,
                        double* logits, hipStream_t stream);

// Fused decode path: partial logits, then in the last workgroup the sum,
// top-k, softmax and tile table (T*E <= 8192, T*k <= 1024).  The workspace
// starts with a 256-byte counter block that must be zero before first use.
bool router_fused_ok(int T, int E, int k);
size_t router_fused_bytes(int T, int H, int E);
void launch_router_fused(const uint16_t* x, const float* w_router, const float* bias, int T,
                         int H, int E, int k, int gating, int BM, void* workspace,
                         int32_t* topk_ids,
                         float* topk_weights, double* logits, int32_t* expert_offsets,
                         int32_t* sorted_ids, int32_t* tiles, int32_t* num_tiles,
                         hipStream_t stream);

// Tile table: one workgroup counts, scans and scatters.
void launch_build_tiles(const int32_t* topk_ids, int N, int E, int BM, int32_t* expert_offsets,
                        int32_t* sorted_ids, int32_t* tiles, int32_t* num_tiles,
                        hipStream_t stream);

// Grouped expert GEMMs over the tile table.
void launch_gateup_swiglu(const uint16_t* x, const uint8_t* w13_q, const uint8_t* w13_s,
                          const int32_t* sorted_ids, const int32_t* tiles,
                          const int32_t* num_tiles, int tiles_max, int T, int H, int I, int E,
                          int k, int BM, bool blocked, uint16_t* h, const ExpertAct& act,
                          hipStream_t stream);
void launch_down(const uint16_t* h, const uint8_t* w2_q, const uint8_t* w2_s,
                 const int32_t* sorted_ids, const int32_t* tiles, const int32_t* num_tiles,
                 int tiles_max, int T, int H, int I, int E, int k, int BM, bool blocked,
                 float* y, const ExpertAct& act, hipStream_t stream);

// Down GEMM and combine of a single token in one launch (no y buffer).
bool down_combine_one_token_ok(int T, int H, int I, int k);
void launch_down_combine_one_token(const uint16_t* h, const uint8_t* w2_q, const uint8_t* w2_s,
                                   const int32_t* sorted_ids, const int32_t* tiles,
                                   const int32_t* num_tiles, const float* topk_weights, int H,
                                   int I, int E, int k, bool blocked, uint16_t* out,
                                   const ExpertAct& act, hipStream_t stream);

// Large-tile (prefill) form of the grouped GEMMs: 128-row tiles, LDS-staged
// operands.  expert_mma_ok says when the launchers above use it for the
// gate/up GEMM (gateup, K = H) or the down GEMM (K = I).
bool expert_mma_ok(bool gateup, int T, int H, int I, int E, int k, int BM);
void launch_expert_mma(bool gateup, const uint16_t* act, const uint8_t* wq, const uint8_t* ws,
                       const int32_t* sorted_ids, const int32_t* tiles, const int32_t* num_tiles,
                       int tiles_max, int T, int H, int I, int E, int k, bool blocked,
                       void* out, const ExpertAct& fn, hipStream_t stream);

// Rows interleaved in pairs within each of E blocks of 2I rows -> the two
// halves: dst row [e][i] = src row [e][2i], dst row [e][I + i] =
// src row [e][2i + 1]; rows of row_bytes bytes.
void launch_deinterleave_rows(const uint8_t* src, int E, int I, int row_bytes, uint8_t* dst,
                              hipStream_t stream);

// The whole layer for one token in one launch (routing, gate/up, down and
// combine; bit-identical to the separate launches).  The workspace starts
// with a sync block of layer_one_token_sync_bytes(H) bytes that must be zero
// before first use and is left zero by every call.
bool layer_one_token_ok(int H, int I, int E, int k);
size_t layer_one_token_sync_bytes(int H);
size_t layer_one_token_bytes(int H, int I, int E, int k);
void launch_layer_one_token(const uint16_t* x, const float* w_router, const float* bias,
                            const uint8_t* w13_q, const uint8_t* w13_s, const uint8_t* w2_q,
                            const uint8_t* w2_s, int H, int I, int E, int k, int gating,
                            bool blocked, int32_t* topk_ids,
                            float* topk_weights, double* logits, int32_t* expert_offsets,
                            int32_t* sorted_ids, int32_t* tiles, int32_t* num_tiles,
                            void* workspace, uint16_t* out, hipStream_t stream);

// The whole layer for 2..4 tokens in one launch (blocked codes; T * k <=
// 16), the same scheme with tiles of several rows.  The workspace starts
// with a sync block of layer_small_batch_sync_bytes() bytes that must be zero
// before first use and is left consistent by every call.
bool layer_small_batch_ok(int T, int H, int I, int E, int k);
size_t layer_small_batch_sync_bytes();
size_t layer_small_batch_bytes(int H, int I);
void launch_layer_small_batch(const uint16_t* x, const float* w_router, const float* bias,
                              const uint8_t* w13_q, const uint8_t* w13_s, const uint8_t* w2_q,
                              const uint8_t* w2_s, int T, int H, int I, int E, int k,
                              int gating, int32_t* topk_ids, float* topk_weights, double* logits,
                              int32_t* expert_offsets, int32_t* sorted_ids, int32_t* tiles,
                              int32_t* num_tiles, void* workspace, uint16_t* out,
                              hipStream_t stream);

// Code matrix [rows][K/2] (canonical) -> blocked layout, out of place.
void launch_repack_blocked(const uint8_t* q, long long rows, int K, uint8_t* qb,
                           hipStream_t stream);

// Weighted combine back to token order.
void launch_combine(const float* y, const float* topk_weights, int T, int H, int k,
                    uint16_t* out, hipStream_t stream);

}  // namespace moe
