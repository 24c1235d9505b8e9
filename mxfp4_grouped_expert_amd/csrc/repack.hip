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

// Row de-interleave of a [E][2I] stack of rows (the gpt-oss checkpoints
// keep each output's gate and up rows adjacent; the kernels read the two
// halves): destination row (e, i) <- source row (e, 2i), destination row
// (e, I + i) <- source row (e, 2i + 1).  One thread per CH-byte piece, in
// destination order (CH = 16 when rows are whole 16-byte pieces, else 1).
template <typename Piece>
__global__ __launch_bounds__(256) void deinterleave_rows_kernel(const Piece* __restrict__ src,
                                                                long long npieces,
                                                                long long per_row, int I,
                                                                Piece* __restrict__ dst) {
  for (long long d = (long long)blockIdx.x * 256 + threadIdx.x; d < npieces;
       d += (long long)gridDim.x * 256) {
    const long long row = d / per_row, off = d - row * per_row;
    const long long e = row / (2LL * I), r = row - e * 2LL * I;
    const long long sr = r < I ? 2 * r : 2 * (r - I) + 1;
    dst[d] = src[(e * 2LL * I + sr) * per_row + off];
  }
}

}  // namespace

void launch_deinterleave_rows(const uint8_t* src, int E, int I, int row_bytes, uint8_t* dst,
                              hipStream_t stream) {
  const long long rows = 2LL * E * I;
  const bool wide = row_bytes % 16 == 0 && (reinterpret_cast<uintptr_t>(src) & 15) == 0 &&
                    (reinterpret_cast<uintptr_t>(dst) & 15) == 0;
  const long long per_row = wide ? row_bytes / 16 : row_bytes;
  const long long npieces = rows * per_row;
  long long blocks = (npieces + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (wide)
    hipLaunchKernelGGL(deinterleave_rows_kernel<uint4>, dim3((unsigned)blocks), dim3(256), 0,
                       stream, reinterpret_cast<const uint4*>(src), npieces, per_row, I,
                       reinterpret_cast<uint4*>(dst));
  else
    hipLaunchKernelGGL(deinterleave_rows_kernel<uint8_t>, dim3((unsigned)blocks), dim3(256), 0,
                       stream, src, npieces, per_row, I, dst);
}

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
