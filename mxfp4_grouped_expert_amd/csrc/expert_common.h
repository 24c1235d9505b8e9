// Constants and small helpers of the row-tile expert GEMMs, shared by
// expert_gemm.hip and the one-token layer kernel.
#pragma once

#include "moe_device.h"

namespace moe {

namespace {

constexpr int kRowsPerBlock = 16;   // weight rows per 16-row block (MFMA N)
constexpr int kBlocksPerStep = 16;  // MX blocks per step (4 waves x 4 lane groups)
constexpr int kChunk = 6;           // steps whose weights a wave holds at once (K = 3072)
constexpr int kChunkK = kChunk * kBlocksPerStep * 32;  // K elements per chunk (3072)

// A tile row that does not describe slots of one valid expert is skipped, so
// a corrupted table cannot send loads or stores out of bounds.
constexpr int kMaxRows = 128;       // largest token tile (BM)

__device__ __forceinline__ bool tile_ok(int e, int r0, int rows, int E, long long nslots) {
  return e >= 0 && e < E && r0 >= 0 && rows > 0 && rows <= kMaxRows &&
         (long long)r0 + rows <= nslots;
}

__device__ __forceinline__ uint32_t word(const uint4& q, int j) {
  return j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w;
}

// Scale table: the E8M0 bytes of a workgroup's weight rows.  The 16 rows of
// one (16-row block, gate/up half) are consecutive rows of the matrix, so
// their scales are one contiguous run of 16*KB bytes: a multiple of 16
// bytes that starts 16-byte aligned (the run starts at row index
// (expert*rows_per_expert + half*I + block*16), and I*KB, H*KB and 16*KB are
// multiples of 16).  Each thread fetches one 16-byte piece of some run, so a
// wave instruction reads 1 KB of consecutive bytes, where per-lane loads of
// each row's byte touch a cache line per row.  ONECHUNK kernels only
// (K <= kChunk * 512, KB <= 96).
constexpr int kScaleRunMax = kRowsPerBlock * kChunk * kBlocksPerStep;  // 1536 bytes

// Wait until at most N of this wave's vector-memory operations are pending.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Row stride of the staged activations in LDS: K bf16 plus a 16-byte pad.
__host__ __device__ __forceinline__ int act_stride_bytes(int K) { return K * 2 + 16; }

}  // namespace

}  // namespace moe
