// Grouped MXFP4 expert GEMMs over the per-expert tile table.
//
// The SimpleLLM write-up ("A 297-line kernel file that decodes faster than
// vLLM", section "Optimizations", "MXFP4 MoE on tensor cores") runs the
// expert FFN as one grouped matrix-core kernel for any token count, decoding
// MXFP4 to bf16 with a few bit operations and one multiply per two values;
// "Where the time went" splits it into "MoE gate/up + SwiGLU" and "MoE down
// + combine".  Here both GEMMs run on gfx950's bf16 MFMA (16x16x32, fp32
// accumulate); the weights are decoded in registers by
// v_cvt_scalef32_pk_bf16_fp4, which turns one byte (two e2m1 codes) into two
// bf16 already multiplied by the block's E8M0 scale.
//
// Work split.  A workgroup (4 waves) owns one tile (<= BM slots of one
// expert) and 16 output rows of the weight matrix (for gate/up: gate rows
// n..n+15 and the matching up rows I+n..I+n+15, so SwiGLU fuses into the
// epilogue).  The reduction dimension is cut into 32-element MX blocks; block
// b = 16*step + 4*wave + group goes to lane group `group` (lanes 16*group ..
// 16*group+15) of wave `wave`.  Each lane then issues one 16-byte load per
// weight row per step: exactly one MX block (32 codes) plus its scale byte,
// and the 16 lanes of a group read 16 rows while the 4 groups of a wave read
// 64 contiguous bytes of each row.  Since an MFMA sums over its whole K
// range, the order in which K elements are assigned to lanes is free as long
// as the activation operand uses the same assignment: for MFMA j (0..3) of a
// step, group g supplies elements 32*b + 8*j .. +8 of both operands.
// The four waves' partial sums meet in LDS in a fixed order, so results are
// bit-reproducible.
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

namespace {

constexpr int kRowsPerBlock = 16;  // weight rows per workgroup (MFMA N)
constexpr int kTokPerMfma = 16;    // tokens per MFMA (MFMA M)
constexpr int kBlocksPerStep = 16; // MX blocks per workgroup step (4 waves x 4 groups)

struct Operand16 {
  uint4 q;     // 32 e2m1 codes of one MX block
  float scale; // its E8M0 scale as fp32
};

__device__ __forceinline__ Operand16 load_block(const uint8_t* q_row, const uint8_t* s_row, int b,
                                                bool valid) {
  Operand16 o;
  if (valid) {
    o.q = *reinterpret_cast<const uint4*>(q_row + (size_t)b * 16);
    o.scale = e8m0_to_float(s_row[b]);
  } else {
    o.q = make_uint4(0u, 0u, 0u, 0u);
    o.scale = 1.0f;
  }
  return o;
}

// Four 8-element bf16 slices of a 32-element block of a bf16 row.
struct Act32 {
  uint4 v[4];
};

__device__ __forceinline__ Act32 load_act(const uint16_t* row, int b, bool valid) {
  Act32 a;
  if (valid) {
    const uint4* p = reinterpret_cast<const uint4*>(row + (size_t)b * 32);
#pragma unroll
    for (int j = 0; j < 4; ++j) a.v[j] = p[j];
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) a.v[j] = make_uint4(0u, 0u, 0u, 0u);
  }
  return a;
}

// A tile row that does not describe slots of one valid expert is skipped, so
// a corrupted table cannot send loads or stores out of bounds.
__device__ __forceinline__ bool tile_ok(int e, int r0, int rows, int E, long long nslots) {
  return e >= 0 && e < E && r0 >= 0 && rows > 0 && (long long)r0 + rows <= nslots;
}

__device__ __forceinline__ uint32_t word(const uint4& q, int j) {
  return j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w;
}

// ----------------------------------------------------------- gate/up + SwiGLU
__global__ __launch_bounds__(256) void gateup_swiglu_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ w13_q,
    const uint8_t* __restrict__ w13_s, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ num_tiles, int T, int H, int I,
    int E, int k, uint16_t* __restrict__ h_out) {
  __shared__ float red[4][2][kTokPerMfma * kRowsPerBlock];

  const int tile = blockIdx.x;
  if (tile >= num_tiles[0]) return;  // uniform over the workgroup
  const int e = tiles[3 * tile + 0];
  const int r0 = tiles[3 * tile + 1];
  const int rows = tiles[3 * tile + 2];
  if (!tile_ok(e, r0, rows, E, (long long)T * k)) return;  // uniform
  const int n_base = blockIdx.y * kRowsPerBlock;

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int li = lane & 15;
  const int grp = lane >> 4;
  const int KB = H / 32;

  const size_t q_stride = (size_t)H / 2;
  const size_t s_stride = (size_t)H / 32;
  const size_t gate_row = (size_t)e * 2 * I + n_base + li;
  const size_t up_row = gate_row + I;
  const uint8_t* qg = w13_q + gate_row * q_stride;
  const uint8_t* qu = w13_q + up_row * q_stride;
  const uint8_t* sg = w13_s + gate_row * s_stride;
  const uint8_t* su = w13_s + up_row * s_stride;

  for (int mb = 0; mb < rows; mb += kTokPerMfma) {
    const int m = min(mb + li, rows - 1);
    int t = sorted_ids[r0 + m] / k;
    t = min(max(t, 0), T - 1);
    const uint16_t* xr = x + (size_t)t * H;

    floatx4 acc_g = {0.f, 0.f, 0.f, 0.f};
    floatx4 acc_u = {0.f, 0.f, 0.f, 0.f};
    for (int step = 0; step * kBlocksPerStep < KB; ++step) {
      const int b = step * kBlocksPerStep + wave * 4 + grp;
      const bool valid = b < KB;
      const Operand16 g = load_block(qg, sg, b, valid);
      const Operand16 u = load_block(qu, su, b, valid);
      const Act32 a = load_act(xr, b, valid);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8 av = as_bf16x8(a.v[j]);
        acc_g = mfma16x16x32(av, dequant8_bf16(word(g.q, j), g.scale), acc_g);
        acc_u = mfma16x16x32(av, dequant8_bf16(word(u.q, j), u.scale), acc_u);
      }
    }

    // lane holds D[4*grp + r][li]: token row 4*grp + r, weight row li
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      red[wave][0][(4 * grp + r) * kRowsPerBlock + li] = acc_g[r];
      red[wave][1][(4 * grp + r) * kRowsPerBlock + li] = acc_u[r];
    }
    __syncthreads();
    {
      const int idx = threadIdx.x;  // 256 = 16 tokens x 16 rows
      const int tm = idx / kRowsPerBlock;
      const int tn = idx % kRowsPerBlock;
      float gs = red[0][0][idx], us = red[0][1][idx];
#pragma unroll
      for (int w = 1; w < 4; ++w) { gs += red[w][0][idx]; us += red[w][1][idx]; }
      if (mb + tm < rows)
        h_out[(size_t)(r0 + mb + tm) * I + n_base + tn] = float_to_bf16(silu(gs) * us);
    }
    __syncthreads();
  }
}

// --------------------------------------------------------------------- down
__global__ __launch_bounds__(256) void down_kernel(
    const uint16_t* __restrict__ h, const uint8_t* __restrict__ w2_q,
    const uint8_t* __restrict__ w2_s, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ num_tiles, int T, int H, int I,
    int E, int k, float* __restrict__ y) {
  __shared__ float red[4][kTokPerMfma * kRowsPerBlock];

  const int tile = blockIdx.x;
  if (tile >= num_tiles[0]) return;
  const int e = tiles[3 * tile + 0];
  const int r0 = tiles[3 * tile + 1];
  const int rows = tiles[3 * tile + 2];
  if (!tile_ok(e, r0, rows, E, (long long)T * k)) return;  // uniform
  const int n_base = blockIdx.y * kRowsPerBlock;

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int li = lane & 15;
  const int grp = lane >> 4;
  const int KB = I / 32;

  const size_t wrow = (size_t)e * H + n_base + li;
  const uint8_t* q = w2_q + wrow * ((size_t)I / 2);
  const uint8_t* s = w2_s + wrow * ((size_t)I / 32);
  const long long nslots = (long long)T * k;

  for (int mb = 0; mb < rows; mb += kTokPerMfma) {
    const int m = min(mb + li, rows - 1);
    const uint16_t* hr = h + (size_t)(r0 + m) * I;

    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int step = 0; step * kBlocksPerStep < KB; ++step) {
      const int b = step * kBlocksPerStep + wave * 4 + grp;
      const bool valid = b < KB;
      const Operand16 w = load_block(q, s, b, valid);
      const Act32 a = load_act(hr, b, valid);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc = mfma16x16x32(as_bf16x8(a.v[j]), dequant8_bf16(word(w.q, j), w.scale), acc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][(4 * grp + r) * kRowsPerBlock + li] = acc[r];
    __syncthreads();
    {
      const int idx = threadIdx.x;
      const int tm = idx / kRowsPerBlock;
      const int tn = idx % kRowsPerBlock;
      float v = red[0][idx];
#pragma unroll
      for (int w = 1; w < 4; ++w) v += red[w][idx];
      if (mb + tm < rows) {
        const long long p = sorted_ids[r0 + mb + tm];
        if (p >= 0 && p < nslots) y[(size_t)p * H + n_base + tn] = v;
      }
    }
    __syncthreads();
  }
}

}  // namespace

void launch_gateup_swiglu(const uint16_t* x, const uint8_t* w13_q, const uint8_t* w13_s,
                          const int32_t* sorted_ids, const int32_t* tiles,
                          const int32_t* num_tiles, int tiles_max, int T, int H, int I, int E,
                          int k, uint16_t* h, hipStream_t stream) {
  dim3 grid(tiles_max, I / kRowsPerBlock);
  hipLaunchKernelGGL(gateup_swiglu_kernel, grid, dim3(256), 0, stream, x, w13_q, w13_s,
                     sorted_ids, tiles, num_tiles, T, H, I, E, k, h);
}

void launch_down(const uint16_t* h, const uint8_t* w2_q, const uint8_t* w2_s,
                 const int32_t* sorted_ids, const int32_t* tiles, const int32_t* num_tiles,
                 int tiles_max, int T, int H, int I, int E, int k, float* y,
                 hipStream_t stream) {
  dim3 grid(tiles_max, H / kRowsPerBlock);
  hipLaunchKernelGGL(down_kernel, grid, dim3(256), 0, stream, h, w2_q, w2_s, sorted_ids, tiles,
                     num_tiles, T, H, I, E, k, y);
}

}  // namespace moe
