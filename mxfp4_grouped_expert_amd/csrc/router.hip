// Router: logits -> top-k -> softmax over the k selected logits.
//
// The SimpleLLM write-up ("A 297-line kernel file that decodes faster than
// vLLM", section "Where the time went") measures "Router + top-k" as its own
// row of a gpt-oss decode step; the triton-kernels README ("Project
// Structure", moe/router.py) pairs softmax gating with top-k.
//
// Logits are accumulated in fp64: a bf16 x fp32 product is exact in fp64, so
// the only error is fp64 summation (~1e-16 relative), far below the gaps
// between neighbouring logits, and the expert choice equals an exact
// evaluation's.  Two launches:
//   1. router_logits_partial: grid (token blocks of 4) x (expert blocks of
//      16) x (K-ranges).  Each wave owns 4 experts x 4 tokens, its lanes
//      stride the K-range four elements at a time (8-byte x loads, 16-byte
//      router loads, coalesced across lanes), and a butterfly reduction
//      leaves one partial sum per (K-range, token, expert).  Splitting K
//      spreads the router matrix over many CUs when T is small (decode), so
//      it streams at HBM speed instead of one CU's.
//   2. router_topk_softmax: one wave per token sums the K-range partials in
//      a fixed order (deterministic), adds the bias, and runs k rounds of a
//      wave-wide argmax on a total order (higher logit first, then lower
//      expert index); lane 0 takes the softmax of the k winners in fp64.
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

namespace {

constexpr int kTokPerWave = 4;
constexpr int kExpPerWave = 4;
constexpr int kWavesPerBlock = 4;
constexpr int kExpPerBlock = kExpPerWave * kWavesPerBlock;

__global__ __launch_bounds__(256) void router_logits_partial(
    const uint16_t* __restrict__ x, const float* __restrict__ w_router, int T, int H, int E,
    int split_len, double* __restrict__ partial) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int t0 = blockIdx.x * kTokPerWave;
  const int e0 = blockIdx.y * kExpPerBlock + wave * kExpPerWave;
  const int s = blockIdx.z;
  if (e0 >= E) return;  // wave-uniform; this kernel has no barrier
  const int kbeg = s * split_len;
  const int kend = min(H, kbeg + split_len);

  const uint16_t* xr[kTokPerWave];
#pragma unroll
  for (int t = 0; t < kTokPerWave; ++t) xr[t] = x + (size_t)min(t0 + t, T - 1) * H;
  const float* wr[kExpPerWave];
#pragma unroll
  for (int e = 0; e < kExpPerWave; ++e) wr[e] = w_router + (size_t)min(e0 + e, E - 1) * H;

  double acc[kTokPerWave][kExpPerWave];
#pragma unroll
  for (int t = 0; t < kTokPerWave; ++t)
#pragma unroll
    for (int e = 0; e < kExpPerWave; ++e) acc[t][e] = 0.0;

  for (int kk = kbeg + 4 * lane; kk < kend; kk += 4 * kWave) {
    double xv[kTokPerWave][4];
#pragma unroll
    for (int t = 0; t < kTokPerWave; ++t) {
      const uint2 v = *reinterpret_cast<const uint2*>(xr[t] + kk);
      xv[t][0] = (double)bf16_to_float(v.x & 0xffffu);
      xv[t][1] = (double)bf16_to_float(v.x >> 16);
      xv[t][2] = (double)bf16_to_float(v.y & 0xffffu);
      xv[t][3] = (double)bf16_to_float(v.y >> 16);
    }
#pragma unroll
    for (int e = 0; e < kExpPerWave; ++e) {
      const float4 w = *reinterpret_cast<const float4*>(wr[e] + kk);
      const double w0 = w.x, w1 = w.y, w2 = w.z, w3 = w.w;
#pragma unroll
      for (int t = 0; t < kTokPerWave; ++t) {
        double a = acc[t][e];
        a = fma(xv[t][0], w0, a);
        a = fma(xv[t][1], w1, a);
        a = fma(xv[t][2], w2, a);
        a = fma(xv[t][3], w3, a);
        acc[t][e] = a;
      }
    }
  }

#pragma unroll
  for (int t = 0; t < kTokPerWave; ++t) {
#pragma unroll
    for (int e = 0; e < kExpPerWave; ++e) {
      double v = acc[t][e];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
      if (lane == 0 && t0 + t < T && e0 + e < E)
        partial[((size_t)s * T + (t0 + t)) * E + (e0 + e)] = v;
    }
  }
}

// Total order on doubles as int64 (larger key = larger value); -0 is folded
// into +0 so the two compare equal, and NaN sorts below everything.
__device__ __forceinline__ long long order_key(double v) {
  v = v + 0.0;
  if (v != v) return LLONG_MIN + 1;
  long long b = __double_as_longlong(v);
  return b >= 0 ? b : (b ^ 0x7fffffffffffffffLL);
}

__global__ __launch_bounds__(256) void router_topk_softmax(
    const double* __restrict__ partial, const float* __restrict__ bias, int T, int E, int k,
    int splits, int32_t* __restrict__ topk_ids, float* __restrict__ topk_weights,
    double* __restrict__ logits) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kWavesPerBlock + wave;
  if (t >= T) return;  // wave-uniform; no barrier below

  // lane owns experts lane, lane+64, lane+128, lane+192
  double val[4];
  long long key[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + kWave * i;
    double v = 0.0;
    if (e < E) {
      // eight K-range partials in flight at a time, summed in ascending order
      for (int s0 = 0; s0 < splits; s0 += 8) {
        double p[8];
#pragma unroll
        for (int c = 0; c < 8; ++c)
          p[c] = (s0 + c < splits) ? partial[((size_t)(s0 + c) * T + t) * E + e] : 0.0;
#pragma unroll
        for (int c = 0; c < 8; ++c) v += p[c];
      }
      if (bias) v += (double)bias[e];
      if (logits) logits[(size_t)t * E + e] = v;
      key[i] = order_key(v);
    } else {
      key[i] = LLONG_MIN;  // absent expert: never chosen
    }
    val[i] = v;
  }

  int sel_e[kMaxTopk];
  double sel_v[kMaxTopk];
#pragma unroll
  for (int j = 0; j < kMaxTopk; ++j) {
    if (j >= k) break;
    // best candidate of this lane: highest key, then lowest expert index
    long long bk = LLONG_MIN;
    int be = 0x7fffffff;
    double bv = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + kWave * i;
      if (key[i] > bk) { bk = key[i]; be = e; bv = val[i]; }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const long long ok = __shfl_xor(bk, off);
      const int oe = __shfl_xor(be, off);
      const double ov = __shfl_xor(bv, off);
      if (ok > bk || (ok == bk && oe < be)) { bk = ok; be = oe; bv = ov; }
    }
    sel_e[j] = be;
    sel_v[j] = bv;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (lane + kWave * i == be) key[i] = LLONG_MIN;
  }

  if (lane == 0) {
    double m = sel_v[0];
#pragma unroll
    for (int j = 1; j < kMaxTopk; ++j)
      if (j < k) m = fmax(m, sel_v[j]);
    double z[kMaxTopk];
    double sum = 0.0;
#pragma unroll
    for (int j = 0; j < kMaxTopk; ++j)
      if (j < k) { z[j] = exp(sel_v[j] - m); sum += z[j]; }
#pragma unroll
    for (int j = 0; j < kMaxTopk; ++j) {
      if (j < k) {
        topk_ids[(size_t)t * k + j] = sel_e[j];
        topk_weights[(size_t)t * k + j] = (float)(z[j] / sum);
      }
    }
  }
}

}  // namespace

RouterPlan router_plan(int T, int H, int E) {
  const long long tb = (T + kTokPerWave - 1) / kTokPerWave;
  const long long eb = (E + kExpPerBlock - 1) / kExpPerBlock;
  // aim for >= 512 workgroups; keep each K-range >= 128 elements
  int splits = (int)(512 / (tb * eb));
  const int max_splits = H / 128 > 0 ? H / 128 : 1;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  int split_len = (H + splits - 1) / splits;
  split_len = (split_len + 3) & ~3;
  splits = (H + split_len - 1) / split_len;
  return RouterPlan{splits, split_len};
}

size_t router_partial_bytes(int T, int H, int E) {
  if (T <= 0) return 0;
  const RouterPlan p = router_plan(T, H, E);
  return (size_t)p.splits * (size_t)T * (size_t)E * sizeof(double);
}

void launch_router_logits(const uint16_t* x, const float* w_router, int T, int H, int E,
                          const RouterPlan& plan, double* partial, hipStream_t stream) {
  dim3 grid((T + kTokPerWave - 1) / kTokPerWave, (E + kExpPerBlock - 1) / kExpPerBlock,
            plan.splits);
  hipLaunchKernelGGL(router_logits_partial, grid, dim3(256), 0, stream, x, w_router, T, H, E,
                     plan.split_len, partial);
}

void launch_router_topk(const double* partial, const float* bias, int T, int E, int k,
                        int splits, int32_t* topk_ids, float* topk_weights, double* logits,
                        hipStream_t stream) {
  dim3 grid((T + kWavesPerBlock - 1) / kWavesPerBlock);
  hipLaunchKernelGGL(router_topk_softmax, grid, dim3(256), 0, stream, partial, bias, T, E, k,
                     splits, topk_ids, topk_weights, logits);
}

}  // namespace moe
