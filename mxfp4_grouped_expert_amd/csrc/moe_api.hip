// C ABI of the MXFP4 grouped-expert MoE library (declared in moe_mxfp4.h).
//
// Every entry point validates its arguments on the host before anything is
// enqueued, checks once per device that the device is gfx950, then enqueues
// its kernels on the caller's stream and returns without synchronising.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>

#include "../../include/moe_mxfp4.h"
#include "moe_launch.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

moe_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return MOE_ERR_DEVICE;
  }
  int st = g_device_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return MOE_ERR_DEVICE;
    }
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_device_state[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? MOE_OK : MOE_ERR_DEVICE;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round256(size_t n) { return (n + 255) & ~size_t(255); }

bool valid_bm(int BM) { return BM == 16 || BM == 32 || BM == 64 || BM == 128; }
bool gating_ok(int gating) { return gating == MOE_GATING_SOFTMAX || gating == MOE_GATING_SIGMOID; }
bool layout_ok(int layout) { return layout == MOE_LAYOUT_CANONICAL || layout == MOE_LAYOUT_BLOCKED; }

moe_status finish_launches() {
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

hipStream_t as_stream(struct ihipStream_t* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK: success";
    case MOE_ERR_NULL: return "MOE_ERR_NULL: a required pointer is NULL";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE: a size is outside the supported range";
    case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN: a pointer is not 16-byte aligned";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace is too small";
    case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE: current device is not gfx950 or not usable";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a kernel launch failed";
    case MOE_ERR_OVERLAP: return "MOE_ERR_OVERLAP: an output overlaps an input";
    default: return "unknown moe_status";
  }
}

const char* moe_version(void) { return "0.1.0"; }

int moe_pick_bm(int T, int k, int E) {
  (void)k;
  (void)E;
  int bm = 16;
  while (bm < 128 && bm < T) bm <<= 1;
  return bm;
}

int64_t moe_tiles_max(int T, int k, int E, int BM) {
  if (T <= 0 || k <= 0 || E <= 0 || BM <= 0) return 0;
  const int64_t n = (int64_t)T * k;
  const int64_t a = (n + BM - 1) / BM + (E < n ? E : n);
  return a < n ? a : n;
}

size_t moe_route_workspace_bytes(int T, int H, int E) {
  if (T <= 0 || H <= 0 || E <= 0) return 0;
  return round256(moe::router_partial_bytes(T, H, E));
}

size_t moe_forward_workspace_bytes(int T, int H, int I, int k) {
  if (T <= 0 || H <= 0 || I <= 0 || k <= 0) return 0;
  const size_t n = (size_t)T * (size_t)k;
  return round256(n * (size_t)I * 2) + round256(n * (size_t)H * 4);
}

moe_status moe_route(const uint16_t* x, const float* w_router, const float* bias, int T, int H,
                     int E, int k, int gating, int32_t* topk_ids, float* topk_weights,
                     double* logits, void* workspace, size_t workspace_bytes,
                     struct ihipStream_t* stream) {
  if (!gating_ok(gating)) return MOE_ERR_SHAPE;
  if (T < 0 || H <= 0 || H % 32 != 0 || H > MOE_MAX_DIM || E < 1 || E > MOE_MAX_EXPERTS || k < 1 ||
      k > MOE_MAX_TOPK || k > E || (int64_t)T * E >= (int64_t(1) << 31) ||
      (int64_t)T * H >= (int64_t(1) << 40))
    return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !topk_ids || !topk_weights || !workspace) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(workspace)) return MOE_ERR_ALIGN;
  if (workspace_bytes < moe_route_workspace_bytes(T, H, E)) return MOE_ERR_WORKSPACE;
  moe_status st = check_device();
  if (st != MOE_OK) return st;
  (void)hipGetLastError();
  const moe::RouterPlan plan = moe::router_plan(T, H, E);
  double* partial = static_cast<double*>(workspace);
  moe::launch_router_logits(x, w_router, T, H, E, plan, partial, as_stream(stream));
  moe::launch_router_topk(partial, bias, T, E, k, gating, plan.splits, topk_ids, topk_weights,
                          logits, as_stream(stream));
  return finish_launches();
}

size_t moe_route_tiles_workspace_bytes(int T, int H, int E) {
  if (T <= 0 || H <= 0 || E <= 0) return 0;
  return round256(moe::router_fused_bytes(T, H, E));
}

moe_status moe_route_tiles(const uint16_t* x, const float* w_router, const float* bias, int T,
                           int H, int E, int k, int gating, int BM, int32_t* topk_ids,
                           float* topk_weights,
                           double* logits, int32_t* expert_offsets, int32_t* sorted_ids,
                           int32_t* tiles, int32_t* num_tiles, void* workspace,
                           size_t workspace_bytes, struct ihipStream_t* stream) {
  if (T < 0 || H <= 0 || H % 32 != 0 || H > MOE_MAX_DIM || E < 1 || E > MOE_MAX_EXPERTS ||
      k < 1 || k > MOE_MAX_TOPK || k > E || !valid_bm(BM) || !moe::router_fused_ok(T, E, k) ||
      !gating_ok(gating))
    return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !topk_ids || !topk_weights || !expert_offsets || !sorted_ids || !tiles ||
      !num_tiles || !workspace)
    return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(workspace)) return MOE_ERR_ALIGN;
  if (workspace_bytes < moe_route_tiles_workspace_bytes(T, H, E)) return MOE_ERR_WORKSPACE;
  moe_status st = check_device();
  if (st != MOE_OK) return st;
  (void)hipGetLastError();
  moe::launch_router_fused(x, w_router, bias, T, H, E, k, gating, BM, workspace, topk_ids,
                           topk_weights,
                           logits, expert_offsets, sorted_ids, tiles, num_tiles,
                           as_stream(stream));
  return finish_launches();
}

moe_status moe_build_tiles(const int32_t* topk_ids, int T, int k, int E, int BM,
                           int32_t* expert_offsets, int32_t* sorted_ids, int32_t* tiles,
                           int32_t* num_tiles, struct ihipStream_t* stream) {
  if (T < 0 || k < 1 || k > MOE_MAX_TOPK || E < 1 || E > MOE_MAX_EXPERTS || !valid_bm(BM) ||
      (int64_t)T * k >= (int64_t(1) << 31))
    return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (!topk_ids || !expert_offsets || !sorted_ids || !tiles || !num_tiles) return MOE_ERR_NULL;
  moe_status st = check_device();
  if (st != MOE_OK) return st;
  (void)hipGetLastError();
  moe::launch_build_tiles(topk_ids, T * k, E, BM, expert_offsets, sorted_ids, tiles, num_tiles,
                          as_stream(stream));
  return finish_launches();
}

namespace {

bool forward_shape_ok(int T, int H, int I, int E, int k, int BM) {
  return T >= 0 && H > 0 && I > 0 && H % 32 == 0 && I % 32 == 0 && H <= MOE_MAX_DIM &&
         I <= MOE_MAX_DIM && E >= 1 && E <= MOE_MAX_EXPERTS && k >= 1 && k <= MOE_MAX_TOPK &&
         k <= E && valid_bm(BM) && (int64_t)T * k < (int64_t(1) << 31) &&
         (int64_t)E * 2 * I < (int64_t(1) << 31) && (int64_t)E * H < (int64_t(1) << 31);
}

}  // namespace

moe_status moe_repack_weights(const uint8_t* q, int64_t rows, int K, uint8_t* q_blocked,
                              struct ihipStream_t* stream) {
  if (rows <= 0 || rows % 16 != 0 || K <= 0 || K % 32 != 0 || K > MOE_MAX_DIM ||
      rows > (int64_t(1) << 40) / K)
    return MOE_ERR_SHAPE;
  if (!q || !q_blocked) return MOE_ERR_NULL;
  if (!aligned16(q) || !aligned16(q_blocked)) return MOE_ERR_ALIGN;
  {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(q), b0 = reinterpret_cast<uintptr_t>(q_blocked);
    const uintptr_t n = (uintptr_t)rows * (uintptr_t)(K / 2);
    if (a0 < b0 + n && b0 < a0 + n) return MOE_ERR_OVERLAP;
  }
  moe_status st = check_device();
  if (st != MOE_OK) return st;
  (void)hipGetLastError();
  moe::launch_repack_blocked(q, rows, K, q_blocked, as_stream(stream));
  return finish_launches();
}

moe_status moe_gateup_swiglu(const uint16_t* x, const uint8_t* w13_q, const uint8_t* w13_s,
                             const int32_t* sorted_ids, const int32_t* tiles,
                             const int32_t* num_tiles, int T, int H, int I, int E, int k, int BM,
                             int layout, uint16_t* h, struct ihipStream_t* stream) {
  if (!forward_shape_ok(T, H, I, E, k, BM) || !layout_ok(layout)) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (!x || !w13_q || !w13_s || !sorted_ids || !tiles || !num_tiles || !h) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(w13_q) || !aligned16(w13_s)) return MOE_ERR_ALIGN;
  moe_status st = check_device();
  if (st != MOE_OK) return st;
  (void)hipGetLastError();
  moe::launch_gateup_swiglu(x, w13_q, w13_s, sorted_ids, tiles, num_tiles,
                            (int)moe_tiles_max(T, k, E, BM), T, H, I, E, k, BM,
                            layout == MOE_LAYOUT_BLOCKED, h, moe::plain_swiglu(),
                            as_stream(stream));
  return finish_launches();
}

moe_status moe_down(const uint16_t* h, const uint8_t* w2_q, const uint8_t* w2_s,
                    const int32_t* sorted_ids, const int32_t* tiles, const int32_t* num_tiles,
                    int T, int H, int I, int E, int k, int BM, int layout, float* y,
                    struct ihipStream_t* stream) {
  if (!forward_shape_ok(T, H, I, E, k, BM) || !layout_ok(layout)) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (!h || !w2_q || !w2_s || !sorted_ids || !tiles || !num_tiles || !y) return MOE_ERR_NULL;
  if (!aligned16(h) || !aligned16(w2_q) || !aligned16(w2_s)) return MOE_ERR_ALIGN;
  moe_status st = check_device();
  if (st != MOE_OK) return st;
  (void)hipGetLastError();
  moe::launch_down(h, w2_q, w2_s, sorted_ids, tiles, num_tiles, (int)moe_tiles_max(T, k, E, BM),
                   T, H, I, E, k, BM, layout == MOE_LAYOUT_BLOCKED, y, moe::plain_swiglu(),
                   as_stream(stream));
  return finish_launches();
}

moe_status moe_combine(const float* y, const float* topk_weights, int T, int H, int k,
                       uint16_t* out, struct ihipStream_t* stream) {
  if (T < 0 || H <= 0 || H % 32 != 0 || H > MOE_MAX_DIM || k < 1 || k > MOE_MAX_TOPK ||
      (int64_t)T * k >= (int64_t(1) << 31))
    return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (!y || !topk_weights || !out) return MOE_ERR_NULL;
  if (!aligned16(y)) return MOE_ERR_ALIGN;
  moe_status st = check_device();
  if (st != MOE_OK) return st;
  (void)hipGetLastError();
  moe::launch_combine(y, topk_weights, T, H, k, out, as_stream(stream));
  return finish_launches();
}

}  // extern "C"

namespace {

// Host validation shared by moe_forward and moe_forward_static_workspace
// (everything but the workspace).
moe_status forward_validate(const uint16_t* x, const uint8_t* w13_q, const uint8_t* w13_s,
                            const uint8_t* w2_q, const uint8_t* w2_s, const float* topk_weights,
                            const int32_t* sorted_ids, const int32_t* tiles,
                            const int32_t* num_tiles, int T, int H, int I, int E, int k, int BM,
                            int layout, const uint16_t* out) {
  if (!forward_shape_ok(T, H, I, E, k, BM) || !layout_ok(layout)) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (!x || !w13_q || !w13_s || !w2_q || !w2_s || !topk_weights || !sorted_ids || !tiles ||
      !num_tiles || !out)
    return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(w13_q) || !aligned16(w13_s) || !aligned16(w2_q) ||
      !aligned16(w2_s))
    return MOE_ERR_ALIGN;
  return MOE_OK;
}

// moe_forward's launches once every argument is valid; h and y are carved
// from `workspace` (moe_forward_workspace_bytes of it).
moe_status forward_launch(const uint16_t* x, const uint8_t* w13_q, const uint8_t* w13_s,
                          const uint8_t* w2_q, const uint8_t* w2_s, const float* topk_weights,
                          const int32_t* sorted_ids, const int32_t* tiles,
                          const int32_t* num_tiles, int T, int H, int I, int E, int k, int BM,
                          int layout, void* workspace, uint16_t* out, const moe::ExpertAct& fn,
                          hipStream_t s) {
  const int64_t tmax = moe_tiles_max(T, k, E, BM);
  const size_t nslots = (size_t)T * (size_t)k;
  uint16_t* h = static_cast<uint16_t*>(workspace);
  float* y = reinterpret_cast<float*>(static_cast<char*>(workspace) + round256(nslots * I * 2));
  const bool blocked = layout == MOE_LAYOUT_BLOCKED;
  moe::launch_gateup_swiglu(x, w13_q, w13_s, sorted_ids, tiles, num_tiles, (int)tmax, T, H, I, E,
                            k, BM, blocked, h, fn, s);
  if (moe::down_combine_one_token_ok(T, H, I, k)) {
    // one token: down GEMM and combine in one launch, bit-identical to the two
    moe::launch_down_combine_one_token(h, w2_q, w2_s, sorted_ids, tiles, num_tiles, topk_weights,
                                       H, I, E, k, blocked, out, fn, s);
    return finish_launches();
  }
  moe::launch_down(h, w2_q, w2_s, sorted_ids, tiles, num_tiles, (int)tmax, T, H, I, E, k, BM,
                   blocked, y, fn, s);
  moe::launch_combine(y, topk_weights, T, H, k, out, s);
  return finish_launches();
}

// The workspace of moe_forward_static_workspace: one copy per device, held
// until the process ends.  Host code never names `scratch` where it needs
// the memory (the name is a host-side stand-in there): it uses the device
// address hipGetSymbolAddress returns, looked up once per device with that
// device current.
__device__ __align__(256) unsigned char scratch[MOE_STATIC_WORKSPACE_BYTES];
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mutex;

moe_status scratch_address(void** addr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return MOE_ERR_DEVICE;
  }
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
        (void)hipGetLastError();
        return MOE_ERR_DEVICE;
      }
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *addr = p;
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_forward(const uint16_t* x, const uint8_t* w13_q, const uint8_t* w13_s,
                       const uint8_t* w2_q, const uint8_t* w2_s, const float* topk_weights,
                       const int32_t* sorted_ids, const int32_t* tiles, const int32_t* num_tiles,
                       int T, int H, int I, int E, int k, int BM, int layout, void* workspace,
                       size_t workspace_bytes, uint16_t* out, struct ihipStream_t* stream) {
  moe_status st = forward_validate(x, w13_q, w13_s, w2_q, w2_s, topk_weights, sorted_ids, tiles,
                                   num_tiles, T, H, I, E, k, BM, layout, out);
  if (st != MOE_OK || T == 0) return st;
  if (!workspace) return MOE_ERR_NULL;
  if (!aligned16(workspace)) return MOE_ERR_ALIGN;
  if (workspace_bytes < moe_forward_workspace_bytes(T, H, I, k)) return MOE_ERR_WORKSPACE;
  st = check_device();
  if (st != MOE_OK) return st;
  (void)hipGetLastError();
  return forward_launch(x, w13_q, w13_s, w2_q, w2_s, topk_weights, sorted_ids, tiles, num_tiles,
                        T, H, I, E, k, BM, layout, workspace, out, moe::plain_swiglu(),
                        as_stream(stream));
}

moe_status moe_forward_gptoss(const uint16_t* x, const uint8_t* w13_q, const uint8_t* w13_s,
                              const uint8_t* w2_q, const uint8_t* w2_s, const float* b13,
                              const float* b2, float alpha, float limit,
                              const float* topk_weights, const int32_t* sorted_ids,
                              const int32_t* tiles, const int32_t* num_tiles, int T, int H, int I,
                              int E, int k, int BM, int layout, void* workspace,
                              size_t workspace_bytes, uint16_t* out,
                              struct ihipStream_t* stream) {
  // alpha finite; limit > 0 (+inf: no clamp); NaN fails both
  if (!(alpha == alpha && alpha - alpha == 0.0f) || !(limit > 0.0f)) return MOE_ERR_SHAPE;
  moe_status st = forward_validate(x, w13_q, w13_s, w2_q, w2_s, topk_weights, sorted_ids, tiles,
                                   num_tiles, T, H, I, E, k, BM, layout, out);
  if (st != MOE_OK || T == 0) return st;
  if (!workspace) return MOE_ERR_NULL;
  if (!aligned16(workspace)) return MOE_ERR_ALIGN;
  if (workspace_bytes < moe_forward_workspace_bytes(T, H, I, k)) return MOE_ERR_WORKSPACE;
  st = check_device();
  if (st != MOE_OK) return st;
  (void)hipGetLastError();
  const moe::ExpertAct fn{b13, b2, alpha, limit, 1};
  return forward_launch(x, w13_q, w13_s, w2_q, w2_s, topk_weights, sorted_ids, tiles, num_tiles,
                        T, H, I, E, k, BM, layout, workspace, out, fn, as_stream(stream));
}

moe_status moe_deinterleave_rows(const void* src, int E, int I, int row_bytes, void* dst,
                                 struct ihipStream_t* stream) {
  if (E < 1 || I < 1 || row_bytes < 1 || (int64_t)E * 2 * I * row_bytes >= (int64_t(1) << 40))
    return MOE_ERR_SHAPE;
  if (!src || !dst) return MOE_ERR_NULL;
  {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(src), b0 = reinterpret_cast<uintptr_t>(dst);
    const uintptr_t n = (uintptr_t)E * 2 * I * (uintptr_t)row_bytes;
    if (a0 < b0 + n && b0 < a0 + n) return MOE_ERR_OVERLAP;
  }
  moe_status st = check_device();
  if (st != MOE_OK) return st;
  (void)hipGetLastError();
  moe::launch_deinterleave_rows(static_cast<const uint8_t*>(src), E, I, row_bytes,
                                static_cast<uint8_t*>(dst), as_stream(stream));
  return finish_launches();
}

moe_status moe_forward_static_workspace(const uint16_t* x, const uint8_t* w13_q,
                                        const uint8_t* w13_s, const uint8_t* w2_q,
                                        const uint8_t* w2_s, const float* topk_weights,
                                        const int32_t* sorted_ids, const int32_t* tiles,
                                        const int32_t* num_tiles, int T, int H, int I, int E,
                                        int k, int BM, int layout, uint16_t* out,
                                        struct ihipStream_t* stream) {
  moe_status st = forward_validate(x, w13_q, w13_s, w2_q, w2_s, topk_weights, sorted_ids, tiles,
                                   num_tiles, T, H, I, E, k, BM, layout, out);
  if (st != MOE_OK || T == 0) return st;
  if (moe_forward_workspace_bytes(T, H, I, k) > (size_t)MOE_STATIC_WORKSPACE_BYTES)
    return MOE_ERR_WORKSPACE;
  st = check_device();
  if (st != MOE_OK) return st;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != MOE_OK) return st;
  (void)hipGetLastError();
  return forward_launch(x, w13_q, w13_s, w2_q, w2_s, topk_weights, sorted_ids, tiles, num_tiles,
                        T, H, I, E, k, BM, layout, ws, out, moe::plain_swiglu(),
                        as_stream(stream));
}

size_t moe_layer_small_batch_workspace_bytes(int T, int H, int I, int E, int k) {
  if (H > MOE_MAX_DIM || I > MOE_MAX_DIM || !moe::layer_small_batch_ok(T, H, I, E, k)) return 0;
  return moe::layer_small_batch_bytes(H, I);
}

size_t moe_layer_small_batch_sync_bytes(void) { return moe::layer_small_batch_sync_bytes(); }

moe_status moe_layer_small_batch(const uint16_t* x, const float* w_router, const float* bias,
                                 const uint8_t* w13_q, const uint8_t* w13_s, const uint8_t* w2_q,
                                 const uint8_t* w2_s, int T, int H, int I, int E, int k,
                                 int gating, int layout, int32_t* topk_ids, float* topk_weights,
                                 double* logits, int32_t* expert_offsets, int32_t* sorted_ids,
                                 int32_t* tiles, int32_t* num_tiles, void* workspace,
                                 size_t workspace_bytes, uint16_t* out,
                                 struct ihipStream_t* stream) {
  if (H <= 0 || I <= 0 || H > MOE_MAX_DIM || I > MOE_MAX_DIM || E < 1 ||
      E > MOE_MAX_EXPERTS || k < 1 || k > MOE_MAX_TOPK || k > E ||
      (int64_t)E * 2 * I >= (int64_t(1) << 31) || !moe::layer_small_batch_ok(T, H, I, E, k) ||
      !gating_ok(gating) || layout != MOE_LAYOUT_BLOCKED)
    return MOE_ERR_SHAPE;
  if (!x || !w_router || !w13_q || !w13_s || !w2_q || !w2_s || !topk_ids || !topk_weights ||
      !expert_offsets || !sorted_ids || !tiles || !num_tiles || !workspace || !out)
    return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(w13_q) || !aligned16(w13_s) ||
      !aligned16(w2_q) || !aligned16(w2_s) || !aligned16(workspace))
    return MOE_ERR_ALIGN;
  if (workspace_bytes < moe::layer_small_batch_bytes(H, I)) return MOE_ERR_WORKSPACE;
  moe_status st = check_device();
  if (st != MOE_OK) return st;
  (void)hipGetLastError();
  moe::launch_layer_small_batch(x, w_router, bias, w13_q, w13_s, w2_q, w2_s, T, H, I, E, k,
                                gating, topk_ids, topk_weights, logits, expert_offsets,
                                sorted_ids, tiles, num_tiles, workspace, out, as_stream(stream));
  return finish_launches();
}

size_t moe_layer_one_token_workspace_bytes(int H, int I, int E, int k) {
  if (!moe::layer_one_token_ok(H, I, E, k) || H > MOE_MAX_DIM) return 0;
  return moe::layer_one_token_bytes(H, I, E, k);
}

size_t moe_layer_one_token_sync_bytes(int H) {
  if (H <= 0 || H % 32 != 0 || H > MOE_MAX_DIM) return 0;
  return moe::layer_one_token_sync_bytes(H);
}

moe_status moe_layer_one_token(const uint16_t* x, const float* w_router, const float* bias,
                               const uint8_t* w13_q, const uint8_t* w13_s, const uint8_t* w2_q,
                               const uint8_t* w2_s, int H, int I, int E, int k, int gating,
                               int layout, int32_t* topk_ids, float* topk_weights, double* logits,
                               int32_t* expert_offsets, int32_t* sorted_ids, int32_t* tiles,
                               int32_t* num_tiles, void* workspace, size_t workspace_bytes,
                               uint16_t* out, struct ihipStream_t* stream) {
  if (H <= 0 || I <= 0 || H > MOE_MAX_DIM || I > MOE_MAX_DIM || E < 1 ||
      E > MOE_MAX_EXPERTS || k < 1 || k > MOE_MAX_TOPK || k > E ||
      (int64_t)E * 2 * I >= (int64_t(1) << 31) || !moe::layer_one_token_ok(H, I, E, k) ||
      !gating_ok(gating) || !layout_ok(layout))
    return MOE_ERR_SHAPE;
  if (!x || !w_router || !w13_q || !w13_s || !w2_q || !w2_s || !topk_ids || !topk_weights ||
      !expert_offsets || !sorted_ids || !tiles || !num_tiles || !workspace || !out)
    return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(w13_q) || !aligned16(w13_s) ||
      !aligned16(w2_q) || !aligned16(w2_s) || !aligned16(workspace))
    return MOE_ERR_ALIGN;
  if (workspace_bytes < moe::layer_one_token_bytes(H, I, E, k)) return MOE_ERR_WORKSPACE;
  moe_status st = check_device();
  if (st != MOE_OK) return st;
  (void)hipGetLastError();
  moe::launch_layer_one_token(x, w_router, bias, w13_q, w13_s, w2_q, w2_s, H, I, E, k, gating,
                              layout == MOE_LAYOUT_BLOCKED, topk_ids,
                              topk_weights, logits, expert_offsets, sorted_ids, tiles, num_tiles,
                              workspace, out, as_stream(stream));
  return finish_launches();
}

}  // extern "C"
