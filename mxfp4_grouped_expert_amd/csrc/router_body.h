// Router device code shared by the routing kernels and the one-token layer
// kernel: fp64 partial logits over K-ranges, the wave top-k + softmax, and
// the one-token tail (top-k, softmax and tile table of a single token).
// Included by one translation unit per kernel file; everything is internal.
#pragma once

#include "moe_device.h"

namespace moe {

namespace {

constexpr int kTokPerWave = 4;
constexpr int kExpPerWave = 4;
constexpr int kWavesPerBlock = 4;
constexpr int kExpPerBlock = kExpPerWave * kWavesPerBlock;

// v of the lane that DPP control CTRL selects (every lane has a source for
// the row rotations and quad permutations used here)
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(b & 0xffffffffLL), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// One workgroup's share of the partial logits: tokens [TPW*bx, +TPW), experts
// [16*by, +16) (4 per wave), K-range bz.  Each finished value is handed to
// store(split, token, expert, value), called by one lane per value.
template <int TPW, typename Store>
__device__ void logits_partial_compute(const uint16_t* __restrict__ x,
                                       const float* __restrict__ w_router, int T, int H, int E,
                                       int split_len, int bx, int by, int bz, Store store) {
  const int wave = (threadIdx.x >> 6) & 3;  // wave within this 256-thread expert block
  const int lane = threadIdx.x & 63;
  const int t0 = bx * TPW;
  const int e0 = by * kExpPerBlock + wave * kExpPerWave;
  const int s = bz;
  if (e0 >= E) return;  // wave-uniform; no barrier in this body
  const int kbeg = s * split_len;
  const int kend = min(H, kbeg + split_len);

  const uint16_t* xr[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) xr[t] = x + (size_t)min(t0 + t, T - 1) * H;
  const float* wr[kExpPerWave];
#pragma unroll
  for (int e = 0; e < kExpPerWave; ++e) wr[e] = w_router + (size_t)min(e0 + e, E - 1) * H;

  double acc[TPW][kExpPerWave];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int e = 0; e < kExpPerWave; ++e) acc[t][e] = 0.0;

  // The wave's 4x4 router weights of a K step stay in registers while each
  // token's 4 activations stream past (each accumulator sees the same FMA
  // sequence whatever TPW is).
  for (int kk = kbeg + 4 * lane; kk < kend; kk += 4 * kWave) {
    double wv[kExpPerWave][4];
#pragma unroll
    for (int e = 0; e < kExpPerWave; ++e) {
      const float4 w = *reinterpret_cast<const float4*>(wr[e] + kk);
      wv[e][0] = w.x; wv[e][1] = w.y; wv[e][2] = w.z; wv[e][3] = w.w;
    }
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const uint2 v = *reinterpret_cast<const uint2*>(xr[t] + kk);
      const double x0 = (double)bf16_to_float(v.x & 0xffffu);
      const double x1 = (double)bf16_to_float(v.x >> 16);
      const double x2 = (double)bf16_to_float(v.y & 0xffffu);
      const double x3 = (double)bf16_to_float(v.y >> 16);
#pragma unroll
      for (int e = 0; e < kExpPerWave; ++e) {
        double a = acc[t][e];
        a = fma(x0, wv[e][0], a);
        a = fma(x1, wv[e][1], a);
        a = fma(x2, wv[e][2], a);
        a = fma(x3, wv[e][3], a);
        acc[t][e] = a;
      }
    }
  }

  // Sum each of the N = TPW*4 values over the wave's 64 lanes, as a
  // reduce-scatter: at lane offsets 32, 16, ... a lane keeps one half of its
  // live values, receives its partner's copy of that half and adds it, so
  // after log2(N) steps it holds one value (index = its lane bits 5, 4, ...)
  // that the remaining offsets finish as a plain butterfly: N - 1 + 6 -
  // log2(N) exchanges instead of 6N.  Every lane of a group ends with the
  // same bits (a + b and b + a are the same double).
  constexpr int N = TPW * kExpPerWave;
  constexpr int LOGN = N == 16 ? 4 : N == 8 ? 3 : N == 4 ? 2 : N == 2 ? 1 : 0;
  static_assert((1 << LOGN) == N, "a power of two");
  double v[N];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int e = 0; e < kExpPerWave; ++e) v[t * kExpPerWave + e] = acc[t][e];
#pragma unroll
  for (int st = 0; st < LOGN; ++st) {
    const int off = 32 >> st;
    const int half = N >> (st + 1);
    const bool up = (lane & off) != 0;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const double send = up ? v[i] : v[i + half];
      const double keep = up ? v[i + half] : v[i];
      v[i] = keep + __shfl_xor(send, off);
    }
  }
  // the rest within 16-lane rows, on DPP (no LDS): rotations by 8 and 4,
  // then quad swaps 2 and 1; lane 0 of each row ends with the row's sum
  static_assert(LOGN >= 2, "the rest fits one 16-lane row");
  if constexpr (LOGN <= 2) v[0] += dpp_f64<0x128>(v[0]);  // row_ror:8
  if constexpr (LOGN <= 3) v[0] += dpp_f64<0x124>(v[0]);  // row_ror:4
  v[0] += dpp_f64<0x4E>(v[0]);                            // quad_perm [2,3,0,1]
  v[0] += dpp_f64<0xB1>(v[0]);                            // quad_perm [1,0,3,2]
  const int idx = lane >> (6 - LOGN);  // the value this lane holds
  const int t = idx / kExpPerWave, e = idx % kExpPerWave;
  if ((lane & ((64 >> LOGN) - 1)) == 0 && t0 + t < T && e0 + e < E)
    store(s, t0 + t, e0 + e, v[0]);
}

// logits_partial_compute into partial[split][token][expert].  ATOMIC_OUT
// stores with agent-scope atomics so another workgroup of the same launch
// may read them.
template <bool ATOMIC_OUT, int TPW = kTokPerWave>
__device__ void logits_partial_body(const uint16_t* __restrict__ x,
                                    const float* __restrict__ w_router, int T, int H, int E,
                                    int split_len, double* __restrict__ partial, int bx, int by,
                                    int bz) {
  logits_partial_compute<TPW>(x, w_router, T, H, E, split_len, bx, by, bz,
                              [&](int s, int t, int e, double v) {
                                double* dst = &partial[((size_t)s * T + t) * E + e];
                                if (ATOMIC_OUT)
                                  __hip_atomic_store(dst, v, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
                                else
                                  *dst = v;
                              });
}

// Total order on doubles as int64 (larger key = larger value); -0 is folded
// into +0 so the two compare equal, and NaN sorts below everything.
__device__ __forceinline__ long long order_key(double v) {
  v = v + 0.0;
  if (v != v) return LLONG_MIN + 1;
  long long b = __double_as_longlong(v);
  return b >= 0 ? b : (b ^ 0x7fffffffffffffffLL);
}

__device__ __forceinline__ double readlane_f64(double v, int l) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)(b & 0xffffffffLL), l);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), l);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

__device__ __forceinline__ long long readlane_i64(long long v, int l) {
  const int lo = __builtin_amdgcn_readlane((int)(v & 0xffffffffLL), l);
  const int hi = __builtin_amdgcn_readlane((int)(v >> 32), l);
  return ((long long)hi << 32) | (unsigned int)lo;
}

// max(v, v of the lane DPP control CTRL selects); lanes without a source
// keep v
template <int CTRL>
__device__ __forceinline__ long long dpp_max_i64(long long v) {
  const int lo = __builtin_amdgcn_update_dpp((int)(v & 0xffffffffLL), (int)(v & 0xffffffffLL),
                                             CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp((int)(v >> 32), (int)(v >> 32), CTRL, 0xF, 0xF,
                                             false);
  const long long o = ((long long)hi << 32) | (unsigned int)lo;
  return o > v ? o : v;
}

// Largest 64-bit key of the wave, the same value in every lane: the maximum
// within each quad, then within each row of 16 (DPP), then over the 4 rows.
__device__ __forceinline__ long long wave_max_i64(long long v) {
  v = dpp_max_i64<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_max_i64<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_max_i64<0x124>(v);  // row_ror:4
  v = dpp_max_i64<0x128>(v);  // row_ror:8
  long long m = readlane_i64(v, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    const long long o = readlane_i64(v, 16 * r);
    m = o > m ? o : m;
  }
  return m;
}

// Gating term of a selected logit v (m: the largest selected logit): exp(v - m)
// for softmax, sigmoid(v) = 1 / (1 + exp(-v)) for sigmoid gating.  Either
// way the weights are the terms divided by their sum (taken in ascending
// slot order).
constexpr int kGatingSoftmax = 0;
constexpr int kGatingSigmoid = 1;
__device__ __forceinline__ double gate_term(double v, double m, int gating) {
  return gating == kGatingSigmoid ? 1.0 / (1.0 + exp(-v)) : exp(v - m);
}

// Top-k and softmax of one token by one wave.  Lane l holds the logits of
// experts l, l+64, l+128, l+192 in val[] (entries >= E are ignored).  k
// rounds of a wave-wide argmax on (higher logit, then lower expert index):
// each round takes the largest order key, then the lowest expert holding it
// (one ballot per slot), and retires that expert.  The softmax over the
// winners is computed in fp64 as one formula: m = their maximum,
// z_j = exp(v_j - m) with lane j taking z_j, the sum of z_0..z_{k-1} in
// ascending j, w_j = z_j / sum, so the weights do not depend on which lane
// computed which term.  Writes ids and weights to topk_ids / topk_weights
// and ids_lds / w_lds, each where given (non-null).
//
// With at most 64 experts and `scratch` given (kRankScratch entries of
// wave-private LDS), the same picks in the same order come from a rank
// count instead: each lane's rank is the number of experts with a larger
// order key, or an equal key and a lower index, so ranks 0..k-1 are the
// argmax rounds' picks in selection order.  Every key is compared at once
// (the keys are read from LDS in 16-byte pairs, branch-free), where the
// rounds are k dependent chains of cross-lane steps: at E = 32, k = 4 the
// selection measured about 2,700 cycles as rounds.  With at most 32 experts
// lanes l and l + 32 both rank expert l, each against half of the keys, and
// add their counts (one cross-lane swap): the count is a serial chain of
// 64-bit compares whose vector and scalar steps wait on each other (0.8 us
// for 32 keys inside the one-token layer), and halving it halves that.
// The softmax below it is the same formula in the same order, so the
// weights are identical.
constexpr int kRankScratch = kWave + 2 * kMaxTopk;  // keys, then (expert, value) by slot

__device__ __forceinline__ void wave_lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <bool WEIGHTS = true>
__device__ void topk_softmax_rank(double v0, int E, int k, int gating, int t,
                                  int32_t* __restrict__ topk_ids,
                                  float* __restrict__ topk_weights, int* ids_lds, float* w_lds,
                                  long long* scratch) {
  const int lane = threadIdx.x & 63;
  const long long key = lane < E ? order_key(v0) : LLONG_MIN;  // below every expert's key
  long long* s_key = scratch;
  long long* s_e = scratch + kWave;
  double* s_v = reinterpret_cast<double*>(scratch + kWave + kMaxTopk);
  s_key[lane] = key;
  wave_lds_order();
  int rank = 0;
  if (E <= kWave / 2) {  // uniform: two lanes per expert, 16 keys each
    const int ex = lane & (kWave / 2 - 1);  // the expert this lane ranks
    const int j0 = lane & (kWave / 2);      // its half of the keys: 0..15 or 16..31
    const long long kx = s_key[ex];
    int r = 0;
#pragma unroll
    for (int b = 0; b < kWave / 4; b += 8) {
      long long o[8];
#pragma unroll
      for (int q = 0; q < 8; q += 2) {
        const longlong2 pr = *reinterpret_cast<const longlong2*>(s_key + j0 / 2 + b + q);
        o[q] = pr.x;
        o[q + 1] = pr.y;
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) r += (o[q] > kx) | ((o[q] == kx) & (j0 / 2 + b + q < ex));
    }
    rank = r + __shfl_xor(r, kWave / 2);
  } else {
#pragma unroll
    for (int b = 0; b < kWave; b += 8) {
      if (b >= E) break;  // uniform
      long long o[8];
#pragma unroll
      for (int q = 0; q < 8; q += 2) {
        const longlong2 pr = *reinterpret_cast<const longlong2*>(s_key + b + q);
        o[q] = pr.x;
        o[q + 1] = pr.y;
      }
#pragma unroll
      for (int q = 0; q < 8; ++q)
        rank += (o[q] > key) | ((o[q] == key) & (b + q < lane));
    }
  }
  wave_lds_order();  // every key read before the slot table overwrites nothing of it
  if (lane < E && rank < k) {
    s_e[rank] = lane;
    s_v[rank] = v0;
  }
  wave_lds_order();
  if constexpr (!WEIGHTS) {  // the selection only: ids in slot order
    if (lane < k) {
      const int el = (int)s_e[lane];
      if (topk_ids) topk_ids[(size_t)t * k + lane] = el;
      if (ids_lds) ids_lds[t * k + lane] = el;
    }
    return;
  }
  double m = s_v[0];
#pragma unroll
  for (int j = 1; j < kMaxTopk; ++j)
    if (j < k) m = fmax(m, s_v[j]);
  const int jl = lane < k ? lane : 0;
  const double vl = s_v[jl];
  const int el = (int)s_e[jl];
  const double z = gate_term(vl, m, gating);
  double sum = 0.0;
#pragma unroll
  for (int j = 0; j < kMaxTopk; ++j)
    if (j < k) sum += readlane_f64(z, j);
  if (lane < k) {
    const float w = (float)(z / sum);
    if (topk_ids) topk_ids[(size_t)t * k + lane] = el;
    if (topk_weights) topk_weights[(size_t)t * k + lane] = w;
    if (ids_lds) ids_lds[t * k + lane] = el;
    if (w_lds) w_lds[t * k + lane] = w;
  }
}

// With WEIGHTS false only the selection is made (ids_lds / topk_ids, the
// same ids in the same slot order); the gating is skipped.
template <bool WEIGHTS = true>
__device__ void topk_softmax_wave(const double (&val)[4], int E, int k, int gating, int t,
                                  int32_t* __restrict__ topk_ids,
                                  float* __restrict__ topk_weights, int* ids_lds,
                                  float* w_lds = nullptr, long long* scratch = nullptr) {
  if (scratch && E <= kWave) {  // uniform
    topk_softmax_rank<WEIGHTS>(val[0], E, k, gating, t, topk_ids, topk_weights, ids_lds, w_lds,
                               scratch);
    return;
  }
  const int lane = threadIdx.x & 63;
  const int nI = (E + kWave - 1) / kWave;  // slots that hold experts (uniform)
  long long key[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) key[i] = (lane + kWave * i < E) ? order_key(val[i]) : LLONG_MIN;

  int sel_e[kMaxTopk];
  double sel_v[kMaxTopk];
#pragma unroll
  for (int j = 0; j < kMaxTopk; ++j) {
    sel_e[j] = 0;
    sel_v[j] = 0.0;
    if (j >= k) continue;
    long long mine = key[0];
#pragma unroll
    for (int i = 1; i < 4; ++i)
      if (i < nI) mine = key[i] > mine ? key[i] : mine;
    const long long best = wave_max_i64(mine);
    // the lowest expert with the best key: slots in order, lanes in order
    int slot = 0, src = 0;
#pragma unroll
    for (int i = 3; i >= 0; --i) {
      if (i >= nI) continue;
      const uint64_t hit = __ballot(key[i] == best);
      if (hit) { slot = i; src = __builtin_ctzll(hit); }
    }
    double v = val[0];
#pragma unroll
    for (int i = 1; i < 4; ++i)
      if (slot == i) v = val[i];
    sel_e[j] = src + kWave * slot;
    sel_v[j] = readlane_f64(v, src);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i == slot && lane == src) key[i] = LLONG_MIN;
  }

  if constexpr (!WEIGHTS) {
    int el = sel_e[0];
#pragma unroll
    for (int j = 1; j < kMaxTopk; ++j)
      if (lane == j) el = sel_e[j];
    if (lane < k) {
      if (topk_ids) topk_ids[(size_t)t * k + lane] = el;
      if (ids_lds) ids_lds[t * k + lane] = el;
    }
    return;
  }
  double m = sel_v[0];
#pragma unroll
  for (int j = 1; j < kMaxTopk; ++j)
    if (j < k) m = fmax(m, sel_v[j]);
  double vl = sel_v[0];
  int el = sel_e[0];
#pragma unroll
  for (int j = 1; j < kMaxTopk; ++j)
    if (lane == j) { vl = sel_v[j]; el = sel_e[j]; }
  const double z = gate_term(vl, m, gating);
  double sum = 0.0;
#pragma unroll
  for (int j = 0; j < kMaxTopk; ++j)
    if (j < k) sum += readlane_f64(z, j);
  if (lane < k) {
    const float w = (float)(z / sum);
    if (topk_ids) topk_ids[(size_t)t * k + lane] = el;
    if (topk_weights) topk_weights[(size_t)t * k + lane] = w;
    if (ids_lds) ids_lds[t * k + lane] = el;
    if (w_lds) w_lds[t * k + lane] = w;
  }
}

// Most K-ranges a one-token logit is summed over.
constexpr int kFusedMaxSplits = 32;

// The logits of token t of T, lane l holding experts l, l+64, ...: the
// K-range partials ([split][token][expert], agent-scope atomic loads, all in
// flight at once) summed in order plus the bias, as router_topk_softmax sums
// them.  ALL_LOADS issues kFusedMaxSplits loads branch-free (the surplus ones
// at the last K-range's address, unused), which measured faster for a single
// token; otherwise only the K-ranges that exist are loaded, which halves a
// multi-token tail's load count.
template <bool ALL_LOADS>
__device__ void token_logits(const double* __restrict__ partial, const float* __restrict__ bias,
                             int T, int t, int E, int splits, double (&val)[4]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + kWave * i;
    double v = 0.0;
    if (e < E) {
      double p[kFusedMaxSplits];
#pragma unroll
      for (int c = 0; c < kFusedMaxSplits; ++c)
        if (ALL_LOADS || c < splits)  // uniform
          p[c] = __hip_atomic_load(&partial[((size_t)min(c, splits - 1) * T + t) * E + e],
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int c = 0; c < kFusedMaxSplits; ++c)
        if (c < splits) v += p[c];
      if (bias) v += (double)bias[e];
    }
    val[i] = v;
  }
}

// The tile table of one token's k slots from their experts in s_ids (LDS,
// written by this wave and synchronised): slot j's position in expert order
// is the number of selected experts below its own, and every selected
// expert gets one tile of one row.
__device__ void one_token_tables(int E, int k, const int* s_ids,
                                 int32_t* __restrict__ expert_offsets,
                                 int32_t* __restrict__ sorted_ids, int32_t* __restrict__ tiles,
                                 int32_t* __restrict__ num_tiles) {
  const int lane = threadIdx.x & 63;
  int ej = 0;
  if (lane < k) ej = s_ids[lane];
  int pos = 0;  // selected experts below ej
  for (int q = 0; q < k; ++q) pos += s_ids[q] < ej;
  if (lane < k) {
    sorted_ids[pos] = lane;
    tiles[3 * pos + 0] = ej;
    tiles[3 * pos + 1] = pos;
    tiles[3 * pos + 2] = 1;
  }
  for (int e = lane; e <= E; e += kWave) {
    int below = 0;
    for (int q = 0; q < k; ++q) below += s_ids[q] < e;
    expert_offsets[e] = below;
  }
  if (lane == 0) num_tiles[0] = k;
}


// The tail of the fused launch for a single token, run by one wave with the
// token's logits in val (lane l: experts l, l+64, ...): top-k and softmax by
// topk_softmax_wave (the unfused path's code, so ids and weights are
// identical), and the tile table of the k slots.  Their experts are
// distinct, so slot j's position in expert order is the number of selected
// experts below its own, every selected expert gets one tile of one row, and
// build_tiles_small would produce exactly this table.  The selected ids go
// to s_ids (LDS) and, if s_w is given, their weights to s_w.
[[maybe_unused]] __device__ void tail_one_token(const double (&val)[4], int E, int k, int gating,
                               int32_t* __restrict__ topk_ids,
                               float* __restrict__ topk_weights, double* __restrict__ logits,
                               int* s_ids, int32_t* __restrict__ expert_offsets,
                               int32_t* __restrict__ sorted_ids, int32_t* __restrict__ tiles,
                               int32_t* __restrict__ num_tiles, float* s_w = nullptr,
                               long long* scratch = nullptr) {
  const int lane = threadIdx.x & 63;
  if (logits)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (lane + kWave * i < E) logits[lane + kWave * i] = val[i];
  topk_softmax_wave(val, E, k, gating, 0, topk_ids, topk_weights, s_ids, s_w,
                    scratch);  // lanes < k fill s_ids
  wave_lds_sync();
  one_token_tables(E, k, s_ids, expert_offsets, sorted_ids, tiles, num_tiles);
}

}  // namespace

}  // namespace moe
