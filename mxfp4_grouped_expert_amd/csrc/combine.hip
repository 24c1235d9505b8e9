// Weighted combine back to token order (the "MoE down + combine" row of the
// SimpleLLM write-up's "Where the time went"; the triton-kernels README's
// "unpermute" step).
//
// out[t][n] = sum_{j<k} w[t][j] * y[t*k + j][n]: y rows are written at their
// flat slot id by the down GEMM, so token t's k expert outputs are adjacent.
// Each thread owns four consecutive columns of one token (16-byte loads of y,
// an 8-byte store of four bf16), accumulates in fp32 in ascending j and rounds
// once to bf16.  No atomics: every output is written by exactly one thread,
// so the result does not depend on scheduling.
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

namespace {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const float* __restrict__ w, int T, int H,
                                                      int k, uint16_t* __restrict__ out) {
  const int cols4 = H / 4;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)T * cols4) return;
  const int t = (int)(idx / cols4);
  const int c = (int)(idx % cols4);
  float wj[kMaxTopk];
  float4 v[kMaxTopk];
#pragma unroll
  for (int j = 0; j < kMaxTopk; ++j) {  // all k loads in flight together
    if (j < k) {
      wj[j] = w[(size_t)t * k + j];
      v[j] = reinterpret_cast<const float4*>(y + ((size_t)t * k + j) * H)[c];
    }
  }
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxTopk; ++j) {
    if (j < k) {
      a0 = fmaf(wj[j], v[j].x, a0);
      a1 = fmaf(wj[j], v[j].y, a1);
      a2 = fmaf(wj[j], v[j].z, a2);
      a3 = fmaf(wj[j], v[j].w, a3);
    }
  }
  uint2 o;
  o.x = (uint32_t)float_to_bf16(a0) | ((uint32_t)float_to_bf16(a1) << 16);
  o.y = (uint32_t)float_to_bf16(a2) | ((uint32_t)float_to_bf16(a3) << 16);
  reinterpret_cast<uint2*>(out + (size_t)t * H)[c] = o;
}

}  // namespace

void launch_combine(const float* y, const float* topk_weights, int T, int H, int k,
                    uint16_t* out, hipStream_t stream) {
  const long long n = (long long)T * (H / 4);
  const unsigned blocks = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(combine_kernel, dim3(blocks), dim3(256), 0, stream, y, topk_weights, T, H, k,
                     out);
}

}  // namespace moe
