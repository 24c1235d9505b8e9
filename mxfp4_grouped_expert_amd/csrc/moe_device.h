// Device helpers shared by the MoE kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_launch.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxExperts = 256;
constexpr int kMaxTopk = 8;

// bf16 bit pattern -> float (exact: bf16 is the top half of fp32).
__device__ __forceinline__ float bf16_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// float -> bf16 bits, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t float_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// E8M0 scale byte -> fp32 2^(s-127).  s = 0 is the fp32 subnormal 2^-127,
// s = 255 is NaN (OCP MX).
__device__ __forceinline__ float e8m0_to_float(uint32_t s) {
  uint32_t bits = s << 23;
  bits = (s == 0u) ? 0x00400000u : bits;
  bits = (s == 255u) ? 0x7fc00000u : bits;
  return __uint_as_float(bits);
}

// Eight e2m1 codes (one dword, element 2i in the low nibble of byte i) times
// a power-of-two scale -> eight bf16, exact for scales 2^-125..2^125.
// v_cvt_scalef32_pk_bf16_fp4 decodes one byte (two codes) per instruction.
__device__ __forceinline__ bf16x8 dequant8_bf16(uint32_t q, float scale) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 0);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 1);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 2);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 3);
  bf16x4 lo = __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
  bf16x4 hi = __builtin_shufflevector(p2, p3, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

// D(16x16 fp32) += A(16x32 bf16) * B(32x16 bf16).  Lane l supplies
// A[l%16][8*(l/16) .. +8] and B[8*(l/16) .. +8][l%16]; it receives
// D[4*(l/16) + r][l%16], r = 0..3.
__device__ __forceinline__ floatx4 mfma16x16x32(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// silu with the hardware exp2 and reciprocal (about 1 ulp each, far below
// the bf16 rounding of the result): z * 1 / (1 + 2^(-z * log2 e)).  Large
// negative z gives 1 / inf = 0, large positive z gives z.
__device__ __forceinline__ float silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.4426950408889634f));
}

// The gpt-oss activation of a (gate, up) pair with their biases already
// added (ExpertAct kind 1, moe_launch.h).
__device__ __forceinline__ float act_gptoss(float g, float u, float alpha, float limit) {
  g = fminf(g, limit);
  u = fminf(fmaxf(u, -limit), limit);
  return g / (1.0f + expf(-alpha * g)) * (u + 1.0f);
}

// The same with the hardware exp2 and reciprocal (as silu_fast).
__device__ __forceinline__ float act_gptoss_fast(float g, float u, float alpha, float limit) {
  g = fminf(g, limit);
  u = fminf(fmaxf(u, -limit), limit);
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-alpha * g * 1.4426950408889634f)) *
         (u + 1.0f);
}

// Value of the other lane of an even/odd lane pair (quad permutation 1,0,3,2
// through DPP, no LDS traffic).
__device__ __forceinline__ float swap_pair(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
}

// Workgroup barrier for phases that exchange data through LDS only: waits
// for this wave's LDS operations, not for its global stores (__syncthreads
// also waits for every outstanding global access, i.e. for store
// acknowledgements from memory).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Waits until this wave's LDS writes have completed, so its later reads (of
// other lanes' entries) see them; the memory clobber keeps the compiler from
// moving LDS accesses across.
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Layouts of a packed MXFP4 code matrix (K/2 bytes per weight row, one
// 16-byte piece per 32-element MX block).  Canonical: row-major.  Blocked:
// within each group of 16 consecutive rows the pieces are stored block by
// block, piece (row, b) at group offset b*256 + (row % 16)*16, so the 16 rows
// of one MX block are 256 contiguous bytes and 4 consecutive blocks of a
// 16-row group are one contiguous kilobyte.  Byte offset of piece (row, 0)
// and the distance between consecutive pieces of one row:
__device__ __forceinline__ size_t wq_row_offset(size_t row, size_t row_bytes, bool blocked) {
  return blocked ? (row & ~size_t(15)) * row_bytes + (row & 15) * 16 : row * row_bytes;
}
__device__ __forceinline__ int wq_piece_stride(bool blocked) { return blocked ? 256 : 16; }

// Number of lanes below this one whose bit is set in `mask`.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

}  // namespace moe
