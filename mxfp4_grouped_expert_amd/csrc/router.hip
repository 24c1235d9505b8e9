// Router: logits -> top-k -> softmax over the k selected logits.
//
// The SimpleLLM write-up ("A 297-line kernel file that decodes faster than
// vLLM", section "Where the time went") measures "Router + top-k" as its own
// row of a gpt-oss decode step; the triton-kernels README ("Project
// Structure", moe/router.py) pairs softmax gating with top-k.
//
// Logits are accumulated in fp64: a bf16 x fp32 product is exact in fp64, so
// the only error is fp64 summation (~1e-16 relative), far below the gaps
// between neighbouring logits, and the expert choice equals an exact
// evaluation's.  Two launches:
//   1. router_logits_partial: grid (token blocks of 4) x (expert blocks of
//      16) x (K-ranges).  Each wave owns 4 experts x 4 tokens, its lanes
//      stride the K-range four elements at a time (8-byte x loads, 16-byte
//      router loads, coalesced across lanes), and a butterfly reduction
//      leaves one partial sum per (K-range, token, expert).  Splitting K
//      spreads the router matrix over many CUs when T is small (decode), so
//      it streams at HBM speed instead of one CU's.  With many tokens
//      (prefill) router_logits_mfma computes whole logits on the fp64 matrix
//      cores instead.
//   2. router_topk_softmax: one wave per token sums the K-range partials in
//      a fixed order (deterministic), adds the bias, and runs k rounds of a
//      wave-wide argmax on a total order (higher logit first, then lower
//      expert index); the softmax of the k winners is taken in fp64.
// The device code of both steps lives in router_body.h.
#include "moe_device.h"
#include "moe_launch.h"
#include "router_body.h"
#include "tiles_block.h"

namespace moe {

namespace {

template <int TPW>
__global__ __launch_bounds__(256) void router_logits_partial(
    const uint16_t* __restrict__ x, const float* __restrict__ w_router, int T, int H, int E,
    int split_len, double* __restrict__ partial) {
  logits_partial_body<false, TPW>(x, w_router, T, H, E, split_len, partial, blockIdx.x,
                                  blockIdx.y, blockIdx.z);
}

// Logits of many tokens on the fp64 matrix cores (v_mfma_f64_16x16x4_f64).
// A workgroup of 8 waves (two per SIMD) takes 16 tokens and up to
// kMfmaExperts experts (8 tiles of 16), and its waves split K: wave w takes
// the 16-element groups g = w, w+8, ... .  Within a group, lane (r = l % 16, q = l / 16)
// loads elements 16g + 4q .. +3 of token row r (8 bytes of bf16) and of
// expert row r of each tile (16 bytes of fp32), and MFMA step s (0..3) takes
// element s of each: step s sums over q, so the four steps together cover
// the group.  Operands are converted to fp64 exactly (bf16 and fp32 both
// embed in fp64) and accumulated in fp64.  The eight waves' sums meet in LDS
// and are added in wave order, so the result does not depend on timing.
constexpr int kMfmaExperts = 128;
constexpr int kMfmaTiles = kMfmaExperts / 16;
constexpr int kMfmaWaves = 8;
typedef double doublex4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(64 * kMfmaWaves) void router_logits_mfma(
    const uint16_t* __restrict__ x, const float* __restrict__ w_router, int T, int H, int E,
    double* __restrict__ logits) {
  __shared__ double red[kMfmaWaves][16][kMfmaExperts + 1];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int q = lane >> 4;
  const int t0 = blockIdx.x * 16;
  const int nt = (E + 15) >> 4;  // expert tiles holding real experts

  const uint16_t* xr = x + (size_t)min(t0 + r, T - 1) * H + 4 * q;
  const float* wr[kMfmaTiles];
#pragma unroll
  for (int n = 0; n < kMfmaTiles; ++n)
    wr[n] = w_router + (size_t)min(16 * n + r, E - 1) * H + 4 * q;

  doublex4 acc[kMfmaTiles];
#pragma unroll
  for (int n = 0; n < kMfmaTiles; ++n) acc[n] = doublex4{0.0, 0.0, 0.0, 0.0};

  // group g+8's loads are in flight while group g is multiplied (the index
  // is clamped, so the load past the last group reads a valid one)
  const int ng = H / 16;
  auto load = [&](int g, uint2& xv, float4 (&w)[kMfmaTiles]) {
    g = min(g, ng - 1);
    xv = *reinterpret_cast<const uint2*>(xr + 16 * g);
    // all tiles, branch-free (tiles past E read clamped rows; their sums
    // are not stored)
#pragma unroll
    for (int n = 0; n < kMfmaTiles; ++n) w[n] = *reinterpret_cast<const float4*>(wr[n] + 16 * g);
  };
  uint2 xv;
  float4 w[kMfmaTiles];
  load(wave, xv, w);
  for (int g = wave; g < ng; g += kMfmaWaves) {
    uint2 xn;
    float4 wn[kMfmaTiles];
    load(g + kMfmaWaves, xn, wn);
    double a[4];
    a[0] = (double)bf16_to_float(xv.x & 0xffffu);
    a[1] = (double)bf16_to_float(xv.x >> 16);
    a[2] = (double)bf16_to_float(xv.y & 0xffffu);
    a[3] = (double)bf16_to_float(xv.y >> 16);
    // step-major order: consecutive MFMAs go to different accumulators, so
    // none waits for the previous one's result
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int n = 0; n < kMfmaTiles; ++n) {
        const float wv = st == 0 ? w[n].x : st == 1 ? w[n].y : st == 2 ? w[n].z : w[n].w;
        acc[n] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[st], (double)wv, acc[n], 0, 0, 0);
      }
    xv = xn;
#pragma unroll
    for (int n = 0; n < kMfmaTiles; ++n) w[n] = wn[n];
  }

  // The fp64 MFMA leaves D[q + 4i][r] of tile n in register i of lane
  // (r, q): token t0 + q + 4i, expert 16n + r.
#pragma unroll
  for (int n = 0; n < kMfmaTiles; ++n)
    if (n < nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][q + 4 * i][16 * n + r] = acc[n][i];
  __syncthreads();
  for (int o = threadIdx.x; o < 16 * E; o += 64 * kMfmaWaves) {
    const int tt = o / E, e = o - tt * E;
    if (t0 + tt < T) {
      double v = red[0][tt][e];
#pragma unroll
      for (int ww = 1; ww < kMfmaWaves; ++ww) v += red[ww][tt][e];
      logits[(size_t)(t0 + tt) * E + e] = v;
    }
  }
}

__global__ __launch_bounds__(256) void router_topk_softmax(
    const double* __restrict__ partial, const float* __restrict__ bias, int T, int E, int k,
    int gating, int splits, int32_t* __restrict__ topk_ids, float* __restrict__ topk_weights,
    double* __restrict__ logits) {
  __shared__ __align__(16) long long s_rank[kWavesPerBlock][kRankScratch];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kWavesPerBlock + wave;
  if (t >= T) return;  // wave-uniform; no barrier below

  double val[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + kWave * i;
    double v = 0.0;
    if (e < E) {
      // eight K-range partials in flight at a time, summed in ascending order
      for (int s0 = 0; s0 < splits; s0 += 8) {
        double p[8];
#pragma unroll
        for (int c = 0; c < 8; ++c)
          p[c] = (s0 + c < splits) ? partial[((size_t)(s0 + c) * T + t) * E + e] : 0.0;
#pragma unroll
        for (int c = 0; c < 8; ++c) v += p[c];
      }
      if (bias) v += (double)bias[e];
      if (logits) logits[(size_t)t * E + e] = v;
    }
    val[i] = v;
  }
  topk_softmax_wave(val, E, k, gating, t, topk_ids, topk_weights, nullptr, nullptr, s_rank[wave]);
}

// ------------------------------------------------------------ fused decode
// Logits partials, then (in the last workgroup to finish) the fixed-order
// sum, top-k, softmax and the tile table, all in one launch.  The workgroups
// take tickets from a counter at the start of the workspace; the last one
// resets it to zero, so the counter must be zero before the first call.
constexpr int kFusedThreads = 1024;  // 16 waves: one token per wave in the tail
constexpr int kFusedMaxT = 16;
constexpr int kFusedMaxSlots = kFusedMaxT * kMaxTopk;

__global__ __launch_bounds__(kFusedThreads) void router_decode_fused(
    const uint16_t* __restrict__ x, const float* __restrict__ w_router,
    const float* __restrict__ bias, int T, int H, int E, int k, int gating, int BM,
    int split_len, int splits, int* __restrict__ counter, double* __restrict__ partial,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_weights,
    double* __restrict__ logits, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ tiles,
    int32_t* __restrict__ num_tiles) {
  __shared__ __align__(16) long long s_rank[kFusedThreads / kWave][kRankScratch];
  __shared__ int s_ids[kFusedMaxSlots];
  __shared__ int s_tab[kWaveTablesScratch];
  __shared__ int s_last;

  // Partials are written with agent-scope atomic stores, which are coherent
  // across the XCDs' L2 caches; waiting for their completion before taking a
  // ticket orders them before it.  (A full __threadfence would also write
  // back every dirty line of the L2, in every workgroup.)  The 16 waves
  // cover 4 expert blocks of the partial grid.
  // (one token: one token per wave, so no wave computes copies of it)
  if (T == 1)
    logits_partial_body<true, 1>(x, w_router, T, H, E, split_len, partial, blockIdx.x,
                                 blockIdx.y * 4 + (threadIdx.x >> 8), blockIdx.z);
  else
    logits_partial_body<true>(x, w_router, T, H, E, split_len, partial, blockIdx.x,
                              blockIdx.y * 4 + (threadIdx.x >> 8), blockIdx.z);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int nwg = gridDim.x * gridDim.y * gridDim.z;
  if (threadIdx.x == 0) s_last = (atomicAdd(counter, 1) == nwg - 1);
  __syncthreads();
  if (!s_last) return;  // uniform over the workgroup
  // The tail: wave t sums token t's partials and runs its top-k and gating
  // with the unfused path's wave code (router_topk_softmax), so ids and
  // weights are identical to moe_route's; then one wave builds the table.
  const int wave = threadIdx.x >> 6;
  if (T == 1) {  // uniform: one wave finishes a single token, no barriers
    if (wave == 0) {
      double val[4];
      token_logits<true>(partial, bias, 1, 0, E, splits, val);
      tail_one_token(val, E, k, gating, topk_ids, topk_weights, logits, s_ids, expert_offsets,
                     sorted_ids, tiles, num_tiles, nullptr, s_rank[0]);
      if (threadIdx.x == 0)
        __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }
  if (wave < T) {  // wave-uniform
    double val[4];
    token_logits<false>(partial, bias, T, wave, E, splits, val);
    if (logits)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = (threadIdx.x & (kWave - 1)) + kWave * i;
        if (e < E) logits[(size_t)wave * E + e] = val[i];
      }
    topk_softmax_wave(val, E, k, gating, wave, topk_ids, topk_weights, s_ids, nullptr,
                      s_rank[wave]);
  }
  lds_barrier();
  if (wave != 0) return;
  build_tiles_wave(s_ids, T * k, E, BM, s_tab, expert_offsets, sorted_ids, tiles, num_tiles);
  if (threadIdx.x == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// --------------------------------------------- fused routing, 17..64 tokens
// moe_route_tiles for batches the single tail above serves slowly (one
// workgroup running every token's top-k and the table): the work after the
// partial logits is spread over the token blocks.
//   routing  tb x ceil(eb/2) x splits workgroups of 512 threads (two
//            16-expert blocks each) compute the partial logits of
//            router_logits_partial and take a ticket of their 4-token block;
//   top-k    the last routing workgroup of a token block sums that block's
//            partials in split order and adds the bias (as
//            router_topk_softmax does) and runs the same wave top-k and
//            gating, one wave per token; it publishes the selected ids and
//            takes a ticket of the call;
//   tiles    the last token block reads every selected id and builds the
//            table with the per-wave builder of tiles_block.h.
// Partials and ids are written with agent-scope atomic stores, which are
// coherent across the XCDs' L2 caches; each workgroup waits for their
// completion before it takes a ticket, so a ticket's last holder sees all of
// them (the single-tail kernel's ordering argument).  The tickets (ints 16..
// of the workspace) are reset by their last holders, so they must be zero
// before the first call and are zero after each.
constexpr int kRelayThreads = 512;
constexpr int kRelayMaxT = 64;
constexpr int kRelayTicket0 = 16;  // first ticket int of the sync block

__global__ __launch_bounds__(kRelayThreads) void route_tiles_relay(
    const uint16_t* __restrict__ x, const float* __restrict__ w_router,
    const float* __restrict__ bias, int T, int H, int E, int k, int gating, int BM,
    int split_len, int splits, int* __restrict__ tickets, double* __restrict__ partial,
    int* __restrict__ idw, int32_t* __restrict__ topk_ids, float* __restrict__ topk_weights,
    double* __restrict__ logits, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ tiles,
    int32_t* __restrict__ num_tiles) {
  __shared__ __align__(16) long long s_rank[kWavesPerBlock][kRankScratch];
  __shared__ int s_ids[kRelayMaxT * kMaxTopk];
  __shared__ TilesScratch<kRelayThreads> S;
  __shared__ int s_last;
  const int tb = (T + kTokPerWave - 1) / kTokPerWave;
  const int eb = (E + kExpPerBlock - 1) / kExpPerBlock;
  const int ebp = (eb + 1) / 2;
  const int wg = blockIdx.x;
  const int bz = wg / (tb * ebp), rem = wg - bz * tb * ebp;
  const int by = (rem / tb) * 2 + (threadIdx.x >> 8), bx = rem % tb;
  if (by < eb)  // uniform per 256-thread half
    logits_partial_body<true>(x, w_router, T, H, E, split_len, partial, bx, by, bz);
  __builtin_amdgcn_s_waitcnt(0);  // this workgroup's partials are stored
  __syncthreads();
  if (threadIdx.x == 0) s_last = atomicAdd(&tickets[bx], 1) == ebp * splits - 1;
  __syncthreads();
  if (!s_last) return;  // uniform
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = bx * kTokPerWave + wave;
  if (wave < kTokPerWave && t < T) {  // wave-uniform
    double val[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + kWave * i;
      double v = 0.0;
      if (e < E) {
        double p[kFusedMaxSplits];
#pragma unroll
        for (int c = 0; c < kFusedMaxSplits; ++c)
          p[c] = __hip_atomic_load(&partial[((size_t)min(c, splits - 1) * T + t) * E + e],
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int c = 0; c < kFusedMaxSplits; ++c)
          if (c < splits) v += p[c];
        if (bias) v += (double)bias[e];
        if (logits) logits[(size_t)t * E + e] = v;
      }
      val[i] = v;
    }
    topk_softmax_wave(val, E, k, gating, t, topk_ids, topk_weights, s_ids, nullptr,
                      s_rank[wave]);
    wave_lds_sync();
    if (lane < k)
      __hip_atomic_store(&idw[t * k + lane], s_ids[t * k + lane], __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0);  // this block's ids are stored
  __syncthreads();
  if (threadIdx.x == 0) {
    tickets[bx] = 0;  // the block's last holder resets its ticket
    s_last = atomicAdd(&tickets[tb], 1) == tb - 1;
  }
  __syncthreads();
  if (!s_last) return;  // uniform
  const int N = T * k;
  for (int p = threadIdx.x; p < N; p += kRelayThreads)
    s_ids[p] = __hip_atomic_load(&idw[p], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  lds_barrier();
  build_tiles_block<kRelayThreads>(static_cast<const int*>(s_ids), N, E, BM, S, expert_offsets,
                                   sorted_ids, tiles, num_tiles);
  if (threadIdx.x == 0) tickets[tb] = 0;
}

}  // namespace

// Many tokens (enough 16-token workgroups to fill the chip), at most
// kMfmaExperts experts, K a multiple of 16.
bool router_mfma_ok(int T, int H, int E) {
  return T >= 1024 && E <= kMfmaExperts && H % 16 == 0;
}

RouterPlan router_plan(int T, int H, int E) {
  const long long tb = (T + kTokPerWave - 1) / kTokPerWave;
  const long long eb = (E + kExpPerBlock - 1) / kExpPerBlock;
  // aim for >= 512 waves of 4x4 (token, expert) pairs; keep each K-range
  // >= 128 elements and at most 32 of them
  int splits = (int)(512 / (tb * eb));
  int max_splits = H / 128 > 0 ? H / 128 : 1;
  if (max_splits > kFusedMaxSplits) max_splits = kFusedMaxSplits;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  int split_len = (H + splits - 1) / splits;
  split_len = (split_len + 3) & ~3;
  splits = (H + split_len - 1) / split_len;
  return RouterPlan{splits, split_len};
}

size_t router_partial_bytes(int T, int H, int E) {
  if (T <= 0) return 0;
  const RouterPlan p = router_plan(T, H, E);
  return (size_t)p.splits * (size_t)T * (size_t)E * sizeof(double);
}

void launch_router_logits(const uint16_t* x, const float* w_router, int T, int H, int E,
                          const RouterPlan& plan, double* partial, hipStream_t stream) {
  if (router_mfma_ok(T, H, E) && plan.splits == 1) {
    hipLaunchKernelGGL(router_logits_mfma, dim3((T + 15) / 16), dim3(64 * kMfmaWaves), 0, stream,
                       x, w_router, T, H, E, partial);
    return;
  }
  dim3 grid((T + kTokPerWave - 1) / kTokPerWave, (E + kExpPerBlock - 1) / kExpPerBlock,
            plan.splits);
  hipLaunchKernelGGL(router_logits_partial<kTokPerWave>, grid, dim3(256), 0, stream, x,
                     w_router, T, H, E, plan.split_len, partial);
}

bool router_fused_ok(int T, int E, int k) {
  (void)E;
  (void)k;
  return T <= kRelayMaxT;
}

namespace {
size_t round256(size_t n) { return (n + 255) & ~size_t(255); }
}  // namespace

size_t router_fused_bytes(int T, int H, int E) {
  // 256-byte block of ticket counters (int 0: the single tail's; ints 16..:
  // the relay's), the K-range partials, the relay's selected ids
  return 256 + round256(router_partial_bytes(T, H, E)) + round256((size_t)T * kMaxTopk * 4);
}

void launch_router_fused(const uint16_t* x, const float* w_router, const float* bias, int T,
                         int H, int E, int k, int gating, int BM, void* workspace,
                         int32_t* topk_ids,
                         float* topk_weights, double* logits, int32_t* expert_offsets,
                         int32_t* sorted_ids, int32_t* tiles, int32_t* num_tiles,
                         hipStream_t stream) {
  const RouterPlan plan = router_plan(T, H, E);
  int* counter = static_cast<int*>(workspace);
  double* partial = reinterpret_cast<double*>(static_cast<char*>(workspace) + 256);
  const int eb = (E + kExpPerBlock - 1) / kExpPerBlock;
  if (T > kFusedMaxT) {
    const size_t pb = round256(router_partial_bytes(T, H, E));
    int* idw = reinterpret_cast<int*>(static_cast<char*>(workspace) + 256 + pb);
    const int tb = (T + kTokPerWave - 1) / kTokPerWave;
    const int n_route = tb * ((eb + 1) / 2) * plan.splits;
    hipLaunchKernelGGL(route_tiles_relay, dim3(n_route), dim3(kRelayThreads), 0, stream, x,
                       w_router, bias, T, H, E, k, gating, BM, plan.split_len, plan.splits,
                       counter + kRelayTicket0, partial, idw, topk_ids, topk_weights, logits,
                       expert_offsets, sorted_ids, tiles, num_tiles);
    return;
  }
  dim3 grid((T + kTokPerWave - 1) / kTokPerWave, (eb + 3) / 4, plan.splits);
  hipLaunchKernelGGL(router_decode_fused, grid, dim3(kFusedThreads), 0, stream, x, w_router, bias,
                     T, H, E, k, gating, BM, plan.split_len, plan.splits, counter, partial,
                     topk_ids,
                     topk_weights, logits, expert_offsets, sorted_ids, tiles, num_tiles);
}

void launch_router_topk(const double* partial, const float* bias, int T, int E, int k,
                        int gating, int splits, int32_t* topk_ids, float* topk_weights,
                        double* logits, hipStream_t stream) {
  dim3 grid((T + kWavesPerBlock - 1) / kWavesPerBlock);
  hipLaunchKernelGGL(router_topk_softmax, grid, dim3(256), 0, stream, partial, bias, T, E, k,
                     gating, splits, topk_ids, topk_weights, logits);
}

}  // namespace moe
