// Per-expert routing tile table as its own launch (any T): workgroups of
// 1024 threads run a builder of tiles_block.h over topk_ids (the all-pairs
// one for a few slots, the per-wave one otherwise; above kSplitMinN slots
// several workgroups each scatter one range of the slots).
#include "moe_device.h"
#include "moe_launch.h"
#include "tiles_block.h"

namespace moe {

namespace {

constexpr int kThreads = 1024;
// The all-pairs builder costs O(N) dependent LDS reads per thread; above
// this many slots the per-wave builder is faster.
constexpr int kSmallN = 128;
// From this many slots the scatter is split over workgroups of about
// kSlotsPerGroup slots each (two 64-slot rounds per wave), at most
// kMaxGroups of them: every one also counts all N ids, so more would add
// reads, not speed.  At the 4k-token prefill (16,384 slots, 8 workgroups)
// the table took 18.8 us in one workgroup, whose waves each walk 1,024
// slots in 16 rounds.
constexpr int kSplitMinN = 4096;
constexpr int kSlotsPerGroup = 2048;
constexpr int kMaxGroups = 64;

int tile_groups(int N) {
  if (N < kSplitMinN) return 1;
  const int g = (N + kSlotsPerGroup - 1) / kSlotsPerGroup;
  return g < kMaxGroups ? g : kMaxGroups;
}

__global__ __launch_bounds__(kThreads) void build_tiles_kernel(
    const int32_t* __restrict__ topk_ids, int N, int E, int BM,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ tiles, int32_t* __restrict__ num_tiles) {
  __shared__ TilesScratch<kThreads> S;
  __shared__ int s_ids[kSmallN];
  __shared__ int s_outside[2][kBuckets];
  if (N <= kSmallN) {  // uniform: few slots, all-pairs form
    if (threadIdx.x < N) s_ids[threadIdx.x] = topk_ids[threadIdx.x];
    lds_barrier();
    build_tiles_small<kThreads>(static_cast<const int*>(s_ids), N, E, BM, S, expert_offsets,
                                sorted_ids, tiles, num_tiles);
  } else if (gridDim.x == 1) {
    build_tiles_block<kThreads>(topk_ids, N, E, BM, S, expert_offsets, sorted_ids, tiles,
                                num_tiles);
  } else {
    // range of this workgroup: a multiple of 64 slots (the last one may be
    // shorter, or empty: its workgroup then only counts)
    const long long G = gridDim.x;
    const long long per = ((N + G - 1) / G + kWave - 1) / kWave * kWave;
    const int q0 = (int)min((long long)N, (long long)blockIdx.x * per);
    const int q1 = (int)min((long long)N, q0 + per);
    build_tiles_block<kThreads>(topk_ids, N, E, BM, S, expert_offsets, sorted_ids, tiles,
                                num_tiles,
                                TilesRange{q0, q1, s_outside[0], s_outside[1], blockIdx.x == 0});
  }
}

}  // namespace

void launch_build_tiles(const int32_t* topk_ids, int N, int E, int BM, int32_t* expert_offsets,
                        int32_t* sorted_ids, int32_t* tiles, int32_t* num_tiles,
                        hipStream_t stream) {
  hipLaunchKernelGGL(build_tiles_kernel, dim3(tile_groups(N)), dim3(kThreads), 0, stream,
                     topk_ids, N, E, BM,
                     expert_offsets, sorted_ids, tiles, num_tiles);
}

}  // namespace moe
