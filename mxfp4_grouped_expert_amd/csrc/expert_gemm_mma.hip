// Grouped MXFP4 expert GEMMs for large token tiles (prefill).
//
// The SimpleLLM write-up grows the MoE token tile with tokens per expert so
// that a weight tile is unpacked once for many tokens instead of once per
// small tile ("A 297-line kernel file that decodes faster than vLLM",
// section "Optimizations", "MoE token tile follows tokens per expert"; a
// 4k-token prefill is its example).  This kernel is the MI355X form of that
// regime: the work is a dense contraction per expert, so it is organised
// around the matrix cores and LDS.
//
// Tile: one workgroup (4 waves, 2 x 2) computes a tile of up to 128 token
// rows of one expert against 192 weight rows: for gate/up 96 gate rows and
// the 96 matching up rows (so SwiGLU is applied in registers: gate fragment
// f and up fragment f + 3 of a lane hold the same (token, column)), for down
// 192 rows of w2.  A wave owns 64 token rows (4 fragments of 16, interleaved
// between the two M-waves so small tiles stay balanced) x 96 weight rows
// (6 fragments), i.e. 24 MFMA 16x16x32 accumulators.
//
// K loop: 128 K per iteration (4 MX blocks; MX block g of the iteration goes
// to lane group g, the order-free K assignment of the decode kernel), three
// LDS stages in flight.  Every load in the loop is a direct global->LDS
// 128-bit load (global_load_lds_dwordx4), a fixed number per wave and
// iteration, so the wait for a stage is an exact vmcnt and no registers hold
// data in flight:
//   * activations: 128 rows x 256 B, gathered by a row table, each row's
//     sixteen 16-byte chunks stored at chunk ^ (row & 15) (conflict-free
//     128-bit reads for the MFMA A operand);
//   * weights: 192 rows x 64 B of e2m1 codes, the four 16-byte MX blocks of
//     a row stored at block ^ ((row >> 2) & 3) (conflict-free reads of a
//     lane's block).
// The E8M0 scales of the workgroup's 192 rows are loaded once into LDS.
// Weights are decoded to bf16 in registers (v_cvt_scalef32_pk_bf16_fp4) right
// before their MFMAs.
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

namespace {

constexpr int kMT = 128;          // token rows per tile (largest BM)
constexpr int kWRows = 192;       // weight rows per workgroup
constexpr int kNFW = 6;           // weight fragments (of 16 rows) per wave
constexpr int kMFW = 4;           // token fragments (of 16 rows) per wave
constexpr int kBK = 128;          // K per iteration
constexpr int kStages = 3;
constexpr int kXStage = kMT * kBK * 2;       // 32 KB of bf16 activations
constexpr int kWStage = kWRows * kBK / 2;    // 12 KB of e2m1 codes
constexpr int kStage = kXStage + kWStage;
constexpr int kXLoads = kXStage / 1024 / 4;  // direct loads per wave per stage (8)
constexpr int kWLoads = kWStage / 1024 / 4;  // (3)
constexpr int kLoadsPerStage = kXLoads + kWLoads;


__device__ __forceinline__ bool tile_ok(int e, int r0, int rows, int E, long long nslots) {
  return e >= 0 && e < E && r0 >= 0 && rows > 0 && rows <= kMT && (long long)r0 + rows <= nslots;
}

__device__ __forceinline__ uint32_t word(const uint4& q, int j) {
  return j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w;
}

// Direct global->LDS 16-byte load: lane l's data lands at lds + 16*l (lds is
// wave-uniform).  Issued as inline asm so the compiler does not add its own
// conservative vmcnt(0) before later LDS reads of other stages; this kernel
// waits for the stages explicitly (stage_wait) before its barrier.
__device__ __forceinline__ void lds_load16(const void* g, unsigned char* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)lds);
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(m0) : "memory");
}

// Wait until at most N of this wave's vector-memory loads are outstanding.
template <int N>
__device__ __forceinline__ void stage_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <bool GATEUP>
__global__ __launch_bounds__(256, 1) void expert_mma_kernel(
    const uint16_t* __restrict__ act, const uint8_t* __restrict__ wq,
    const uint8_t* __restrict__ ws, const int32_t* sorted_ids,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ num_tiles, int T, int H,
    int I, int E, int k, void* __restrict__ out) {
  extern __shared__ __align__(16) unsigned char smem[];

  const int tile = blockIdx.x;
  if (tile >= num_tiles[0]) return;  // uniform over the workgroup
  const int e = tiles[3 * tile + 0];
  const int r0 = tiles[3 * tile + 1];
  const int rows = tiles[3 * tile + 2];
  const long long nslots = (long long)T * k;
  if (!tile_ok(e, r0, rows, E, nslots)) return;  // uniform

  const int K = GATEUP ? H : I;
  const int N = GATEUP ? I : H;          // output columns
  const int KB = K / 32;
  const int niters = (KB + 3) / 4;
  const int ncol = GATEUP ? kWRows / 2 : kWRows;
  const int n0 = blockIdx.y * ncol;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int li = lane & 15;
  const int grp = lane >> 4;
  const int wm = wave & 1;
  const int wn = wave >> 1;

  unsigned char* s_scale = smem + kStages * kStage;                    // [192][KB]
  long long* s_rowoff = reinterpret_cast<long long*>(s_scale + ((kWRows * KB + 15) & ~15));
  int* s_slot = reinterpret_cast<int*>(s_rowoff + kMT);

  // global weight row of local weight row r (clamped to the matrix)
  auto wrow = [&](int r) -> size_t {
    if (GATEUP) {
      const int half = r >= kWRows / 2;
      const int n = min(n0 + r - half * (kWRows / 2), I - 1);
      return (size_t)e * 2 * I + (size_t)half * I + n;
    }
    return (size_t)e * H + min(n0 + r, H - 1);
  };

  // ---- row table and the scale slab (plain loads, once)
  if (tid < kMT) {
    const int rr = min(tid, rows - 1);
    const int slot = sorted_ids[r0 + rr];
    long long off;
    if (GATEUP) {
      off = (long long)min(max(slot / k, 0), T - 1) * H;
    } else {
      off = (long long)(r0 + rr) * I;
    }
    s_rowoff[tid] = off;
    s_slot[tid] = slot;
  }
  for (int i = tid; i < kWRows * KB; i += 256) {
    const int r = i / KB;
    s_scale[i] = ws[wrow(r) * KB + (i - r * KB)];
  }
  __syncthreads();

  // ---- per-lane constants of the staging loads
  // activations: load q (0..7) of this wave covers rows 4*(8*wave+q) .. +4
  const int x_slot = lane & 15;
  const uint16_t* x_row[kXLoads];
  int x_swz[kXLoads];
#pragma unroll
  for (int q = 0; q < kXLoads; ++q) {
    const int r = 4 * (kXLoads * wave + q) + (lane >> 4);
    x_row[q] = act + s_rowoff[min(r, rows - 1)];
    x_swz[q] = x_slot ^ (r & 15);
  }
  // weights: load q (0..2) covers weight rows 16*(3*wave+q) .. +16
  const int w_slot = lane & 3;
  size_t w_base[kWLoads];
  int w_swz[kWLoads];
#pragma unroll
  for (int q = 0; q < kWLoads; ++q) {
    const int r = 16 * (kWLoads * wave + q) + (lane >> 2);
    w_base[q] = wrow(r) * (size_t)(K / 2);
    w_swz[q] = w_slot ^ ((r >> 2) & 3);
  }

  auto issue = [&](int it, int st) {
    unsigned char* xs = smem + st * kStage;
    unsigned char* wsb = xs + kXStage;
#pragma unroll
    for (int q = 0; q < kXLoads; ++q) {
      const int ii = kXLoads * wave + q;
      const int kel = min(it * kBK + 8 * x_swz[q], K - 8);  // past K: finite values, scale 0
      lds_load16(x_row[q] + kel, xs + ii * 1024);
    }
#pragma unroll
    for (int q = 0; q < kWLoads; ++q) {
      const int ii = kWLoads * wave + q;
      const int blk = min(it * 4 + w_swz[q], KB - 1);
      lds_load16(wq + w_base[q] + (size_t)blk * 16, wsb + ii * 1024);
    }
  };

  // local weight rows of this lane's six fragments
  int frow[kNFW];
#pragma unroll
  for (int f = 0; f < kNFW; ++f) {
    if (GATEUP)
      frow[f] = (f < 3 ? 0 : kWRows / 2) + 48 * wn + 16 * (f % 3) + li;
    else
      frow[f] = 96 * wn + 16 * f + li;
  }
  bool mact[kMFW];
#pragma unroll
  for (int i = 0; i < kMFW; ++i) mact[i] = 16 * (2 * i + wm) < rows;  // uniform per wave

  floatx4 acc[kMFW][kNFW];
#pragma unroll
  for (int i = 0; i < kMFW; ++i)
#pragma unroll
    for (int f = 0; f < kNFW; ++f) acc[i][f] = floatx4{0.f, 0.f, 0.f, 0.f};

  issue(0, 0);
  if (niters > 1) issue(1, 1);

  for (int it = 0; it < niters; ++it) {
    // stage `it` landed: at most the next stage's loads are still in flight
    if (it + 1 < niters)
      stage_wait<kLoadsPerStage>();
    else
      stage_wait<0>();
    wg_barrier();  // every wave's share landed; every wave is done with stage it-1
    if (it + 2 < niters) issue(it + 2, (it + 2) % kStages);

    const unsigned char* xs = smem + (it % kStages) * kStage;
    const unsigned char* wsb = xs + kXStage;
    const int blk = it * 4 + grp;
    const bool bvalid = blk < KB;
    const int blkc = min(blk, KB - 1);

    uint4 wraw[kNFW];
    float scale[kNFW];
#pragma unroll
    for (int f = 0; f < kNFW; ++f) {
      const int r = frow[f];
      wraw[f] = *reinterpret_cast<const uint4*>(wsb + r * 64 + 16 * (grp ^ ((r >> 2) & 3)));
      scale[f] = bvalid ? e8m0_to_float(s_scale[r * KB + blkc]) : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x8 a[kMFW];
#pragma unroll
      for (int i = 0; i < kMFW; ++i) {
        const int r = 16 * (2 * i + wm) + li;
        a[i] = mact[i] ? as_bf16x8(*reinterpret_cast<const uint4*>(
                             xs + r * 256 + 16 * ((4 * grp + j) ^ (r & 15))))
                       : bf16x8{};
      }
#pragma unroll
      for (int f = 0; f < kNFW; ++f) {
        const bf16x8 b = dequant8_bf16(word(wraw[f], j), scale[f]);
#pragma unroll
        for (int i = 0; i < kMFW; ++i)
          if (mact[i]) acc[i][f] = mfma16x16x32(a[i], b, acc[i][f]);
      }
    }
  }

  // ---- epilogue straight from the accumulators: lane holds
  // D[4*grp + r][li] of each (token fragment, weight fragment)
#pragma unroll
  for (int i = 0; i < kMFW; ++i) {
    if (!mact[i]) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * (2 * i + wm) + 4 * grp + r;
      if (row >= rows) continue;
      if (GATEUP) {
#pragma unroll
        for (int f = 0; f < 3; ++f) {
          const int col = n0 + 48 * wn + 16 * f + li;
          if (col < N)
            reinterpret_cast<uint16_t*>(out)[(size_t)(r0 + row) * I + col] =
                float_to_bf16(silu(acc[i][f][r]) * acc[i][f + 3][r]);
        }
      } else {
        const long long p = s_slot[row];
        if (p < 0 || p >= nslots) continue;
#pragma unroll
        for (int f = 0; f < kNFW; ++f) {
          const int col = n0 + 96 * wn + 16 * f + li;
          if (col < N) reinterpret_cast<float*>(out)[(size_t)p * H + col] = acc[i][f][r];
        }
      }
    }
  }
}

size_t mma_lds_bytes(int K) {
  const int KB = K / 32;
  return (size_t)kStages * kStage + (((size_t)kWRows * KB + 15) & ~(size_t)15) + kMT * 8 +
         kMT * 4;
}

}  // namespace

bool expert_mma_ok(int T, int H, int I, int E, int k, int BM) {
  // large token tiles, K small enough for the scale slab, and the expected
  // rows per expert large enough that 128-row tiles are mostly full
  const int Kmax = H > I ? H : I;
  return BM == kMT && Kmax <= 3072 && (long long)T * k >= 32LL * E;
}

void launch_expert_mma(bool gateup, const uint16_t* act, const uint8_t* wq, const uint8_t* ws,
                       const int32_t* sorted_ids, const int32_t* tiles, const int32_t* num_tiles,
                       int tiles_max, int T, int H, int I, int E, int k, void* out,
                       hipStream_t stream) {
  const int K = gateup ? H : I;
  const int N = gateup ? I : H;
  const int ncol = gateup ? kWRows / 2 : kWRows;
  dim3 grid(tiles_max, (N + ncol - 1) / ncol);
  const size_t lds = mma_lds_bytes(K);
  if (gateup)
    hipLaunchKernelGGL(expert_mma_kernel<true>, grid, dim3(256), lds, stream, act, wq, ws,
                       sorted_ids, tiles, num_tiles, T, H, I, E, k, out);
  else
    hipLaunchKernelGGL(expert_mma_kernel<false>, grid, dim3(256), lds, stream, act, wq, ws,
                       sorted_ids, tiles, num_tiles, T, H, I, E, k, out);
}

}  // namespace moe
