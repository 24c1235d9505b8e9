// Per-expert routing tile table as its own launch (any T): one workgroup of
// 1024 threads runs a builder of tiles_block.h over topk_ids (the all-pairs
// one for a few slots, the per-wave one otherwise).
#include "moe_device.h"
#include "moe_launch.h"
#include "tiles_block.h"

namespace moe {

namespace {

constexpr int kThreads = 1024;
// The all-pairs builder costs O(N) dependent LDS reads per thread; above
// this many slots the per-wave builder is faster.
constexpr int kSmallN = 128;

__global__ __launch_bounds__(kThreads) void build_tiles_kernel(
    const int32_t* __restrict__ topk_ids, int N, int E, int BM,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ tiles, int32_t* __restrict__ num_tiles) {
  __shared__ TilesScratch<kThreads> S;
  __shared__ int s_ids[kSmallN];
  if (N <= kSmallN) {  // uniform: few slots, all-pairs form
    if (threadIdx.x < N) s_ids[threadIdx.x] = topk_ids[threadIdx.x];
    lds_barrier();
    build_tiles_small<kThreads>(static_cast<const int*>(s_ids), N, E, BM, S, expert_offsets,
                                sorted_ids, tiles, num_tiles);
  } else {
    build_tiles_block<kThreads>(topk_ids, N, E, BM, S, expert_offsets, sorted_ids, tiles,
                                num_tiles);
  }
}

}  // namespace

void launch_build_tiles(const int32_t* topk_ids, int N, int E, int BM, int32_t* expert_offsets,
                        int32_t* sorted_ids, int32_t* tiles, int32_t* num_tiles,
                        hipStream_t stream) {
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(kThreads), 0, stream, topk_ids, N, E, BM,
                     expert_offsets, sorted_ids, tiles, num_tiles);
}

}  // namespace moe
