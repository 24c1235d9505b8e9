// Load-time repack of a packed MXFP4 code matrix into the blocked layout.
//
// The SimpleLLM write-up ("A 297-line kernel file that decodes faster than
// vLLM") reorders the checkpoint's MXFP4 weights in memory once, at load,
// into the order its tensor-core kernel consumes (section "Optimizations",
// "MXFP4 MoE on tensor cores"), found that fixing the layout up inside the
// kernel was slower (section "Dead ends"), and re-quantizes nothing (section
// "Correctness").  The same holds here: bytes move, values do not.  The
// grouped GEMMs here read each 16-row
// block of a weight matrix one MX block (16 bytes per row) at a time, which
// in the row-major layout is 16 separate 16-byte pieces per block.  This
// kernel rewrites the codes once, at load time, so that those 16 pieces are
// adjacent (see wq_row_offset for the layout); the values, the scales and
// every kernel's arithmetic stay the same.
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

namespace {

// One thread per 16-byte piece of the output, in output order (each wave
// writes one contiguous kilobyte; its reads are 16 rows x 16 bytes of one MX
// block, four blocks per wave).  Grid-stride over the whole matrix.
__global__ __launch_bounds__(256) void repack_blocked_kernel(const uint4* __restrict__ q,
                                                             long long npieces, int KB,
                                                             uint4* __restrict__ qb) {
  const long long group = 16LL * KB;  // pieces per 16-row group
  for (long long d = (long long)blockIdx.x * 256 + threadIdx.x; d < npieces;
       d += (long long)gridDim.x * 256) {
    const long long g = d / group;
    const long long within = d - g * group;
    const long long b = within >> 4;
    const long long li = within & 15;
    qb[d] = q[(g * 16 + li) * KB + b];
  }
}

}  // namespace

void launch_repack_blocked(const uint8_t* q, long long rows, int K, uint8_t* qb,
                           hipStream_t stream) {
  const int KB = K / 32;
  const long long npieces = rows * KB;
  long long blocks = (npieces + 255) / 256;
  if (blocks > 8192) blocks = 8192;  // 32 waves per CU, then grid-stride
  hipLaunchKernelGGL(repack_blocked_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<const uint4*>(q), npieces, KB,
                     reinterpret_cast<uint4*>(qb));
}

}  // namespace moe
