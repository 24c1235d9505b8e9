// Per-expert routing tile table.
//
// The SimpleLLM write-up ("A 297-line kernel file that decodes faster than
// vLLM", section "Optimizations", "Per-expert routing tile table") has each
// expert write its own tiles instead of the expert GEMM searching a
// tiles x experts grid, and sizes the token tile from tokens per expert
// ("MoE token tile follows tokens per expert").
//
// One workgroup of 1024 threads (16 waves) does it all in LDS, without any
// order-dependent atomics, so the result is bit-exact and deterministic:
//   1. count slots per expert (LDS integer adds: the totals do not depend on
//      their order); ids outside [0, E) go to a trash bucket E;
//   2. exclusive scans of the counts (row offsets) and of ceil(count/BM)
//      (tile offsets), one wave each;
//   3. stable scatter in chunks of 1024 slots: within a wave, lanes with the
//      same expert find each other with nine ballots (one per bit of the
//      bucket index) and rank themselves with mbcnt; per-wave counts in LDS
//      give each wave's base; a running count per expert carries across
//      chunks.  Slot order inside an expert is therefore ascending;
//   4. tiles: each tile index finds its expert by binary search over the
//      tile offsets and writes (expert, row_start, rows).
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kBuckets = kMaxExperts + 1;  // + trash bucket

// Exclusive scan of n <= 320 ints by one wave (5 per lane); writes out[0..n]
// with out[n] = total.
__device__ void wave_exclusive_scan(const int* in, int* out, int n, int lane) {
  const int base = lane * 5;
  int loc[5];
  int sum = 0;
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    loc[j] = (base + j < n) ? in[base + j] : 0;
    sum += loc[j];
  }
  int incl = sum;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  int run = incl - sum;
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    if (base + j < n) out[base + j] = run;
    run += loc[j];
  }
  if (lane == kWave - 1) out[n] = incl;
}

__global__ __launch_bounds__(kThreads) void build_tiles_kernel(
    const int32_t* __restrict__ topk_ids, int N, int E, int BM,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ tiles, int32_t* __restrict__ num_tiles) {
  __shared__ int cnt[kBuckets];
  __shared__ int ntile[kBuckets];
  __shared__ int off[kBuckets + 1];
  __shared__ int toff[kBuckets + 1];
  __shared__ int run[kBuckets];
  __shared__ int wcnt[kWaves][kBuckets];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int NB = E + 1;  // buckets in use

  for (int i = tid; i < NB; i += kThreads) { cnt[i] = 0; run[i] = 0; }
  __syncthreads();
  for (int p = tid; p < N; p += kThreads) {
    int e = topk_ids[p];
    e = (e < 0 || e >= E) ? E : e;
    atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  for (int i = tid; i < NB; i += kThreads) ntile[i] = (i < E) ? (cnt[i] + BM - 1) / BM : 0;
  __syncthreads();
  if (wave == 0) wave_exclusive_scan(cnt, off, NB, lane);
  if (wave == 1) wave_exclusive_scan(ntile, toff, NB, lane);
  __syncthreads();
  for (int i = tid; i <= E; i += kThreads) expert_offsets[i] = off[i];

  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int c0 = 0; c0 < N; c0 += kThreads) {
    for (int i = tid; i < kWaves * NB; i += kThreads) (&wcnt[0][0])[(i / NB) * kBuckets + i % NB] = 0;
    const int p = c0 + tid;
    const bool valid = p < N;
    int e = 0;
    if (valid) {
      e = topk_ids[p];
      e = (e < 0 || e >= E) ? E : e;
    }
    uint64_t same = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 9; ++bit) {
      const bool b = (e >> bit) & 1;
      const uint64_t bal = __ballot(b);
      same &= b ? bal : ~bal;
    }
    const int rank = lanes_below(same);
    __syncthreads();  // wcnt zeroed
    if (valid && (same & ~lt_mask & ~(1ull << lane)) == 0)  // last lane of its group
      wcnt[wave][e] = rank + 1;
    __syncthreads();
    if (valid) {
      int before = off[e] + run[e] + rank;
      for (int w = 0; w < wave; ++w) before += wcnt[w][e];
      sorted_ids[before] = p;
    }
    __syncthreads();
    for (int i = tid; i < NB; i += kThreads) {
      int add = 0;
      for (int w = 0; w < kWaves; ++w) add += wcnt[w][i];
      run[i] += add;
    }
    __syncthreads();
  }

  const int total = toff[E];
  for (int i = tid; i < total; i += kThreads) {
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (toff[mid] <= i) lo = mid; else hi = mid - 1;
    }
    const int j = i - toff[lo];
    tiles[3 * i + 0] = lo;
    tiles[3 * i + 1] = off[lo] + j * BM;
    tiles[3 * i + 2] = min(BM, cnt[lo] - j * BM);
  }
  if (tid == 0) num_tiles[0] = total;
}

}  // namespace

void launch_build_tiles(const int32_t* topk_ids, int N, int E, int BM, int32_t* expert_offsets,
                        int32_t* sorted_ids, int32_t* tiles, int32_t* num_tiles,
                        hipStream_t stream) {
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(kThreads), 0, stream, topk_ids, N, E, BM,
                     expert_offsets, sorted_ids, tiles, num_tiles);
}

}  // namespace moe
