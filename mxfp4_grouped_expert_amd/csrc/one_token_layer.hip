// The whole MoE layer for one token in a single launch: router logits,
// top-k, softmax and tile table, the grouped gate/up GEMM with SwiGLU, the
// grouped down GEMM and the weighted combine.
//
// The SimpleLLM write-up ("A 297-line kernel file that decodes faster than
// vLLM", section "Where the time went") books launch and host gaps as their
// own row of a decode step.  With one token each step is short, so the gaps
// between dependent launches and the time each launch takes to fill the GPU
// with workgroups are a large share of the layer.  Here one grid holds all
// of it:
//   routing   splits x ceil(E/16) workgroups compute fp64 partial logits (as
//             router_decode_fused does) and publish them.  The first
//             min(that, 32) of them, the publishers, then each read all the
//             partials, sum them in split order and run the wave top-k, all
//             in parallel and with identical results, and each publishes the
//             plan (expert and slot of each sorted position) in a line of
//             its own, then the routing weights; publisher 0 also writes the
//             routing outputs and the tile table for the caller.
//   GEMM      workgroup j polls the plan words it needs in replica
//             j % publishers, then runs gate/up job j (tile g = j / (I/16),
//             16-row block j % (I/16)) with exactly the arithmetic of the
//             one-token gate/up kernel (expert_gemm_kernel<gate/up, 1, 1>),
//             then the down job(s) of the tile t with (t+1) * I/16 <= j <
//             (t+1) * I/16 + H/16 with exactly the arithmetic of the
//             one-token down kernel.  The last tile's down job of each
//             16-row block also combines the block's k slots in ascending
//             slot order, as combine_kernel does.
// Every value is therefore bit-identical to moe_route_tiles + moe_forward.
//
// Handshakes and why they are sound.
//  * Progress.  A workgroup only ever waits for data produced by workgroups
//    with a lower index (routing below GEMM, a tile's gate/up jobs below its
//    down jobs, the other tiles' down jobs below the combining one), and the
//    dispatcher starts workgroups in index order, so the lowest-index
//    unfinished workgroup is always resident and never waits on anything
//    unfinished: the waits cannot deadlock however few workgroups fit at
//    once.  Every poll is also bounded (about a second); one that gives up
//    sets the sticky error word and its workgroup carries on with whatever
//    it read, so the launch ends even if the premise were broken.
//  * Visibility.  Values that cross workgroups are written and read with
//    agent-scope atomic stores and loads, which gfx950 serves from the
//    memory side of its caches (coherent across the XCDs' L2s), and each
//    value carries its own validity in the same 64-bit word: nothing relies
//    on the order in which two different stores become visible, so no
//    release/acquire fence (and no wait for a store to complete) is needed
//    on the critical path.  Partial logits are stored as their bit pattern
//    plus one in a buffer chosen by the call's parity, zero meaning "not yet
//    written" (no fp64 value that the router arithmetic can produce has all
//    bits set: NaNs that propagate from fp32 or bf16 inputs have their low
//    29 bits clear); the routing workgroups clear the other parity's buffer
//    for the next call.  h pairs and y values carry a stamp, the call's
//    epoch + 1, in their upper half.
//  * Epoch.  Thread 0 of each workgroup reads the epoch (in routing
//    workgroups every thread does, and all of them wait for the load before
//    the barrier that precedes the check-in); the others take it from LDS
//    after a barrier.  The last workgroup to check in (a two-level arrival
//    tree) advances it, so no workgroup of a call can see the next call's
//    value.
//
// Contention.  Atomics and polls on one address are serialised by the
// memory system (tens of nanoseconds per access to one line), so no line is
// read by many workgroups: the partials by the publishers only, each plan
// replica by about (GEMM workgroups / publishers) threads, and the arrival
// tree spreads its counters over 16 leaf lines and a top line.  (Every GEMM
// workgroup reading all partials itself measured slower than the old single
// tail: 900 workgroups polling the same 44 lines.)
#include "expert_common.h"
#include "moe_device.h"
#include "moe_launch.h"
#include "one_launch.h"
#include "router_body.h"

namespace moe {

namespace {

constexpr int kThreads = 256;           // every role: 4 waves
constexpr int kActRegion = (kMaxK * 2 + 16 + 1023) / 1024 * 1024;  // staged row + pad
constexpr int kRedBytes = 4 * 2 * 256 * 4;  // split-K table of the gate/up job
constexpr int kRegion0 = kActRegion > kRedBytes ? kActRegion : kRedBytes;

// words per parity buffer: [split][expert] at a fixed stride, bit pattern
// + 1 (0: not yet), so any shape finds its words where the last call of any
// shape cleared them
constexpr size_t kPartialWords = (size_t)kMaxSplits * kMaxExperts;
// the plan as a publisher leaves it, one 128-byte line each
constexpr int kMaxPublishers = 32;
struct PlanLine {
  u64 plan[kMaxTopk];    // sorted position g: stamp | slot << 16 | expert
  u64 weight[kMaxTopk];  // slot j: stamp | routing weight bits
};
static_assert(sizeof(PlanLine) == 128, "one line per replica");

struct Args {
  const uint16_t* x;
  const float* w_router;
  const float* bias;
  const uint8_t* w13_q;
  const uint8_t* w13_s;
  const uint8_t* w2_q;
  const uint8_t* w2_s;
  int H, I, E, k, gating;
  bool blocked;    // code matrices in the blocked layout
  int split_len, splits, n_route;
  int32_t* topk_ids;
  float* topk_weights;
  double* logits;
  int32_t* expert_offsets;
  int32_t* sorted_ids;
  int32_t* tiles;
  int32_t* num_tiles;
  Sync* sync;
  u64* partials;    // [2][kPartialWords]: parity buffers of published partial logits
  PlanLine* plans;  // [kMaxPublishers]
  int n_pub;        // publishers: min(n_route, kMaxPublishers)
  u64* h;           // [k][I/2] stamped bf16 pairs
  u64* y;           // [k][H] stamped fp32
  uint16_t* out;
};


// LDS of a workgroup's own routing: logits, the rank scratch of the wave
// top-k, and the selected experts and weights in slot order.
constexpr int kRankAllMaxE = 32;  // experts whose ranks the whole workgroup counts
constexpr int kRankParts = kThreads / kRankAllMaxE;
struct RouteLds {
  double logit[kMaxExperts];
  long long scratch[kRankScratch];
  int ids[kMaxTopk];
  float w[kMaxTopk];
  int cnt[kRankAllMaxE][kRankParts];
};

// The token's logits from the published partials, by the whole workgroup
// (barriers inside): wave w sums the partials of experts w*64 + lane in
// split order and adds the bias, exactly as token_logits does, into
// r->logit; then wave 0 runs the wave top-k, as moe_route_tiles does, and
// the selected ids end in r->ids (slot order).  With at most 32 experts the
// whole workgroup counts the ranks instead (thread t: expert t % 32 against
// keys 4*(t/32) .. +3; the eight counts of an expert are then added): the
// same ranks as the wave top-k's rank count (the number of experts with a
// larger order key, or an equal key and a lower index), so the same ids in
// the same slots, with a serial compare chain of 4 instead of 16.
__device__ void route_ids(const Args& a, const CallState& cs, RouteLds* r) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = lane + kWave * wave;
  const u64* cur = a.partials + (size_t)(cs.epoch & 1) * kPartialWords;
  if (e < a.E) {
    double sum = settle_partials(cur + e, (size_t)kMaxExperts, a.splits, &a.sync->error,
                                 cs.spin_limit);
    if (a.bias) sum += (double)a.bias[e];
    r->logit[e] = sum;
  }
  __syncthreads();
  if (a.E <= kRankAllMaxE) {  // uniform
    const int t = threadIdx.x;
    const int ex = t % kRankAllMaxE, part = t / kRankAllMaxE;
    const long long kx = ex < a.E ? order_key(r->logit[ex]) : LLONG_MIN;
    int c = 0;
#pragma unroll
    for (int q = 0; q < kRankAllMaxE / kRankParts; ++q) {
      const int j = (kRankAllMaxE / kRankParts) * part + q;
      const long long o = j < a.E ? order_key(r->logit[j]) : LLONG_MIN;
      c += (o > kx) | ((o == kx) & (j < ex));
    }
    r->cnt[ex][part] = c;
    __syncthreads();
    if (t < a.E) {
      int rank = 0;
#pragma unroll
      for (int p = 0; p < kRankParts; ++p) rank += r->cnt[t][p];
      if (rank < a.k) r->ids[rank] = t;
    }
  } else if (wave == 0) {
    double val[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) val[i] = lane + kWave * i < a.E ? r->logit[lane + kWave * i] : 0.0;
    topk_softmax_wave<false>(val, a.E, a.k, a.gating, 0, nullptr, nullptr, r->ids, nullptr,
                             r->scratch);
  }
  __syncthreads();
}

// The routing weights of the token (wave 0, after route_ids): the same wave
// top-k and gating as moe_route_tiles, so the ids (r->ids) are the same and
// the weights (r->w) identical.
__device__ void route_weights(const Args& a, RouteLds* r) {
  const int lane = threadIdx.x & 63;
  double val[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) val[i] = lane + kWave * i < a.E ? r->logit[lane + kWave * i] : 0.0;
  topk_softmax_wave<true>(val, a.E, a.k, a.gating, 0, nullptr, nullptr, r->ids, r->w,
                          r->scratch);
  wave_lds_sync();
}

// Publishes the plan of the ids in `ids` (slot order) into line L: the
// sorted position of slot j is the number of selected experts below its
// own (one wave; lanes < k store).
__device__ void publish_plan(const Args& a, const int* ids, PlanLine* L, unsigned stamp) {
  const int lane = threadIdx.x & 63;
  if (lane < a.k) {
    const int e = ids[lane];
    int pos = 0;
    for (int q = 0; q < a.k; ++q) pos += ids[q] < e;
    st64(&L->plan[pos], stamp, ((unsigned)lane << 16) | (unsigned)e);
  }
}

// ---------------------------------------------------------------- routing
__device__ void routing_role(const Args& a, int rid, RouteLds* r) {
  // every thread reads the epoch (it picks the parity buffer); all of those
  // loads have returned before the barrier that precedes the check-in
  const CallState cs = read_call_state(a.sync);
  u64* cur = a.partials + (size_t)(cs.epoch & 1) * kPartialWords;
  u64* nxt = a.partials + (size_t)((cs.epoch & 1) ^ 1) * kPartialWords;
  const int eb = (a.E + kExpPerBlock - 1) / kExpPerBlock;
  logits_partial_compute<1>(a.x, a.w_router, 1, a.H, a.E, a.split_len, 0, rid % eb, rid / eb,
                            [&](int s, int, int e, double v) {
                              st64w(cur + (size_t)s * kMaxExperts + e,
                                    (u64)__double_as_longlong(v) + 1ull);
                            });
  // the next call's buffer starts empty whatever shape wrote it last
  for (size_t i = (size_t)rid * kThreads + threadIdx.x; i < kPartialWords;
       i += (size_t)a.n_route * kThreads)
    st64w(nxt + i, 0ull);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 3 * kWave) check_in(a.sync, cs.epoch);
  if (rid >= a.n_pub) return;
  // a publisher: the ids first (the GEMM workgroups wait for them), then the
  // weights (only the combining workgroups need them)
  route_ids(a, cs, r);
  if (threadIdx.x >= kWave) return;
  const int lane = threadIdx.x;
  const unsigned stamp = (unsigned)cs.epoch + 1u;
  PlanLine* L = &a.plans[rid];
  publish_plan(a, r->ids, L, stamp);
  route_weights(a, r);
  if (lane < a.k) st64(&L->weight[lane], stamp, __float_as_uint(r->w[lane]));
  if (rid != 0) return;
  if (a.logits)
    for (int e = lane; e < a.E; e += kWave) a.logits[e] = r->logit[e];
  if (lane < a.k) {
    a.topk_ids[lane] = r->ids[lane];
    a.topk_weights[lane] = r->w[lane];
  }
  one_token_tables(a.E, a.k, r->ids, a.expert_offsets, a.sorted_ids, a.tiles, a.num_tiles);
}

// ----------------------------------------------------------------- gate/up
// Tile g (sorted position g, one row), 16-row block cb of the gate and up
// halves.  Same lane roles, loads, exchange (canonical layout only), MFMA
// order, split-K order and epilogue as expert_gemm_kernel<true, 1, 1, true,
// BLK> for one token.
struct GateupLoads {
  uint4 w[kChunk][2];  // this lane's weight pieces, per step and half
  uint4 spiece;        // this thread's piece of the two scale runs
};

// The token's activation row into LDS (16-byte slots, the pad slot
// repeating the last chunk).  It does not depend on the routing, so it is
// requested at the workgroup's start.
__device__ __forceinline__ void gateup_prefetch_act(const Args& a, unsigned char* act) {
  const int K = a.H;
  const int tid = threadIdx.x, lane = tid & 63, kq = tid >> 6;
  const int cpr = K / 8, spr = cpr + 1;
  for (int ins = kq; ins < (spr + 63) / 64; ins += 4) {
    const int c = min(ins * 64 + lane, cpr - 1);
    __builtin_amdgcn_global_load_lds(a.x + (size_t)c * 8,
                                     (__attribute__((address_space(3))) void*)(act + ins * 1024),
                                     16, 0, 0);
  }
}

// The scale piece, then the weights (the activations are already requested).
template <bool BLK>
__device__ __forceinline__ void gateup_issue(const Args& a, int cb, int e, GateupLoads& L) {
  const int I = a.I, K = a.H, KB = K / 32;
  const int tid = threadIdx.x, lane = tid & 63, kq = tid >> 6;
  const int n_base = cb * kRowsPerBlock;
  const int pr = min(tid / KB, 1), pp = tid - pr * KB;
  L.spiece = *reinterpret_cast<const uint4*>(
      a.w13_s + ((size_t)e * 2 * I + (size_t)pr * I + n_base) * KB + (size_t)min(pp, KB - 1) * 16);
  asm volatile("" ::: "memory");
  // canonical: 4 rows x 256 bytes per wave instruction, exchanged later;
  // blocked: the MFMA mapping itself, one contiguous kilobyte
  const int l_row = BLK ? n_base + (lane & 15) : n_base + 4 * kq + (lane >> 4);
  const size_t wrow[2] = {(size_t)e * 2 * I + l_row, (size_t)e * 2 * I + I + l_row};
#pragma unroll
  for (int c = 0; c < kChunk; ++c) {
    const int bc = min(BLK ? c * kBlocksPerStep + kq * 4 + (lane >> 4)
                           : c * kBlocksPerStep + (lane & 15), KB - 1);
#pragma unroll
    for (int w = 0; w < 2; ++w)
      L.w[c][w] = *reinterpret_cast<const uint4*>(a.w13_q + wq_row_offset(wrow[w], K / 2, BLK) +
                                                  (size_t)bc * wq_piece_stride(BLK));
  }
}

template <bool BLK>
__device__ __forceinline__ void gateup_finish(const Args& a, int g, int cb, unsigned stamp,
                                              unsigned char* lds, GateupLoads& L) {
  constexpr int NW = 2;
  const int I = a.I, K = a.H, KB = K / 32;
  const int n_base = cb * kRowsPerBlock;
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, grp = lane >> 4;
  const int kq = tid >> 6;
  unsigned char* act = lds;                          // x row, then the split-K table
  unsigned char* s_sc = lds + kRegion0;              // 2 scale runs
  unsigned char* s_ring = s_sc + NW * kScaleRunMax;  // 2 exchange slots

  wait_vmcnt<kChunk * NW>();  // activations and the scale piece
  const int pr = min(tid / KB, NW - 1), pp = tid - pr * KB;
  if (tid < NW * KB) *reinterpret_cast<uint4*>(s_sc + pr * kScaleRunMax + pp * 16) = L.spiece;
  lds_barrier();

  uint32_t sreg[kChunk][NW];
#pragma unroll
  for (int c = 0; c < kChunk; ++c) {
    const int bc = min(c * kBlocksPerStep + kq * 4 + grp, KB - 1);
#pragma unroll
    for (int w = 0; w < NW; ++w) sreg[c][w] = s_sc[w * kScaleRunMax + li * KB + bc];
  }
  floatx4 acc[NW] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int c = 0; c < kChunk; ++c) {
    if constexpr (!BLK) {
      unsigned char* slot = s_ring + (c & 1) * NW * kRowsPerBlock * 256;
      const int wr16 = 4 * kq + (lane >> 4);
#pragma unroll
      for (int w = 0; w < NW; ++w)
        *reinterpret_cast<uint4*>(slot + (w * kRowsPerBlock + wr16) * 256 +
                                  (((lane & 15) ^ wr16) << 4)) = L.w[c][w];
      lds_barrier();
#pragma unroll
      for (int w = 0; w < NW; ++w)
        L.w[c][w] = *reinterpret_cast<const uint4*>(
            slot + (w * kRowsPerBlock + li) * 256 + (((4 * kq + grp) ^ li) << 4));
    }
#pragma unroll
    for (int w = 0; w < NW; ++w)
      asm volatile("" : "+v"(L.w[c][w].x), "+v"(L.w[c][w].y), "+v"(L.w[c][w].z),
                   "+v"(L.w[c][w].w), "+v"(sreg[c][w]));
    const int b = c * kBlocksPerStep + kq * 4 + grp;
    const int bc = min(b, KB - 1);
    float scale[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) scale[w] = b < KB ? e8m0_to_float(sreg[c][w]) : 0.f;
    const uint4* ap = reinterpret_cast<const uint4*>(act + bc * 64);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 av = as_bf16x8(ap[j]);
#pragma unroll
      for (int w = 0; w < NW; ++w)
        acc[w] = mfma16x16x32(av, dequant8_bf16(word(L.w[c][w], j), scale[w]), acc[w]);
    }
  }

  // split-K sum in wave order, then SwiGLU of row 0 (the token)
  __syncthreads();
  float* red = reinterpret_cast<float*>(act);
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      red[(kq * NW + w) * 256 + (4 * grp + r) * kRowsPerBlock + li] = acc[w][r];
  __syncthreads();
  float v[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    v[w] = red[(0 * NW + w) * 256 + tid];
#pragma unroll
    for (int q = 1; q < 4; ++q) v[w] += red[(q * NW + w) * 256 + tid];
  }
  const uint32_t hv = float_to_bf16(silu(v[0]) * v[NW - 1]);
  const uint32_t hn = (uint32_t)__float_as_int(swap_pair(__int_as_float((int)hv)));
  if (tid < kRowsPerBlock && (tid & 1) == 0)  // one stamped word per bf16 pair
    st64(a.h + ((size_t)g * I + n_base + tid) / 2, stamp, hv | (hn << 16));
}

// -------------------------------------------------------------------- down
// Tile g, 16-row block cb of w2: the arithmetic of expert_gemm_kernel<false,
// 1, 1, true> for one token.  The last tile's job also combines the block.
struct DownLoads {
  uint4 w[kChunk];
  uint4 spiece;
};

__device__ __forceinline__ void down_issue(const Args& a, int cb, int e, DownLoads& L) {
  const int K = a.I, KB = K / 32;
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, grp = lane >> 4;
  const int kq = tid >> 6;
  const int n_base = cb * kRowsPerBlock;
  const size_t wrow = (size_t)e * a.H + n_base + li;
#pragma unroll
  for (int c = 0; c < kChunk; ++c) {
    const int bc = min(c * kBlocksPerStep + kq * 4 + grp, KB - 1);
    L.w[c] = *reinterpret_cast<const uint4*>(a.w2_q + wq_row_offset(wrow, K / 2, a.blocked) +
                                             (size_t)bc * wq_piece_stride(a.blocked));
  }
  L.spiece = *reinterpret_cast<const uint4*>(
      a.w2_s + ((size_t)e * a.H + n_base) * KB + (size_t)min(tid, KB - 1) * 16);
}

__device__ __forceinline__ void down_finish(const Args& a, int g, int cb, int slot,
                                            unsigned stamp, int spin_limit, const PlanLine* R,
                                            unsigned char* lds, DownLoads& L) {
  const int H = a.H, I = a.I, K = I, KB = K / 32;
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, grp = lane >> 4;
  const int kq = tid >> 6;
  const int n_base = cb * kRowsPerBlock;
  unsigned char* act = lds;                          // h row
  unsigned char* s_sc = lds + kRegion0;              // scale run
  float* red = reinterpret_cast<float*>(s_sc + kScaleRunMax);

  __syncthreads();  // the LDS of any earlier job is free
  // h row g into LDS as its stamped pairs arrive (16-byte slots, the pad
  // slot repeating the last chunk): every word of this thread requested at
  // once, then re-polled only where the stamp is not yet this call's
  {
    constexpr int kPer = ((kMaxK / 8 + 1) * 4 + kThreads - 1) / kThreads;
    const int cpr = K / 8, spr = cpr + 1;
    const u64* hrow = a.h + (size_t)g * I / 2;
    unsigned* dst = reinterpret_cast<unsigned*>(act);
    const u64* src[kPer];
    bool use[kPer];
    u64 v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int d = tid + i * kThreads;
      use[i] = d < spr * 4;
      src[i] = hrow + min(min(d, spr * 4 - 1) >> 2, cpr - 1) * 4 + (d & 3);
    }
    settle(src, use, v, stamp, &a.sync->error, spin_limit);
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (use[i]) dst[tid + i * kThreads] = (unsigned)v[i];
  }
  if (tid < KB) *reinterpret_cast<uint4*>(s_sc + tid * 16) = L.spiece;
  __syncthreads();

  uint32_t sreg[kChunk];
#pragma unroll
  for (int c = 0; c < kChunk; ++c)
    sreg[c] = s_sc[li * KB + min(c * kBlocksPerStep + kq * 4 + grp, KB - 1)];
  floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < kChunk; ++c) {
    asm volatile("" : "+v"(L.w[c].x), "+v"(L.w[c].y), "+v"(L.w[c].z), "+v"(L.w[c].w),
                 "+v"(sreg[c]));
    const int b = c * kBlocksPerStep + kq * 4 + grp;
    const float scale = b < KB ? e8m0_to_float(sreg[c]) : 0.f;
    const uint4* ap = reinterpret_cast<const uint4*>(act + min(b, KB - 1) * 64);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc = mfma16x16x32(as_bf16x8(ap[j]), dequant8_bf16(word(L.w[c], j), scale), acc);
  }
  if (grp == 0) red[kq * kRowsPerBlock + li] = acc[0];  // row 0: the token
  __syncthreads();
  if (tid >= kRowsPerBlock) return;  // no barrier below
  float yv = red[tid];
#pragma unroll
  for (int q = 1; q < 4; ++q) yv += red[q * kRowsPerBlock + tid];
  if (g != a.k - 1) {
    st64(a.y + (size_t)slot * H + n_base + tid, stamp, __float_as_uint(yv));
    return;
  }
  // the last tile's job combines the block: the routing weights and the
  // other slots' y as their stamped words arrive, then fma in ascending slot
  // order
  const u64* src[2 * kMaxTopk];
  bool use[2 * kMaxTopk];
  u64 v[2 * kMaxTopk];
#pragma unroll
  for (int j = 0; j < kMaxTopk; ++j) {
    const int jc = min(j, a.k - 1);
    src[j] = &R->weight[jc];
    use[j] = j < a.k;
    src[kMaxTopk + j] = a.y + (size_t)jc * H + n_base + tid;
    use[kMaxTopk + j] = j < a.k && j != slot;
  }
  settle(src, use, v, stamp, &a.sync->error, spin_limit);
  float wj[kMaxTopk], yj[kMaxTopk];
#pragma unroll
  for (int j = 0; j < kMaxTopk; ++j) {
    wj[j] = __uint_as_float((unsigned)v[j]);
    yj[j] = j == slot ? yv : __uint_as_float((unsigned)v[kMaxTopk + j]);
  }
  float acc_o = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxTopk; ++j)
    if (j < a.k) acc_o = fmaf(wj[j], yj[j], acc_o);
  a.out[n_base + tid] = float_to_bf16(acc_o);
}

// ------------------------------------------------------- GEMM workgroups
// Workgroup j (after the routing ones) runs gate/up job j when j < k * I/16,
// then the down jobs of every tile t with (t+1) * I/16 <= j <
// (t+1) * I/16 + H/16 (block j - (t+1) * I/16): a tile's down jobs sit above
// all of its gate/up jobs, and the last tile's down job of a block above the
// other tiles' jobs of that block.  A down job's weights are requested once
// the workgroup's gate/up job is done (requested together, the two streams
// measured slower).
template <bool BLK>
__device__ void gemm_role(const Args& a, int j, unsigned char* lds, CallState* s_call,
                          unsigned* s_plan) {
  const int ncbI = a.I / kRowsPerBlock, ncbH = a.H / kRowsPerBlock;
  const bool has_gu = j < a.k * ncbI;
  const int g_gu = min(j / ncbI, a.k - 1);
  int t0 = a.k;  // first tile with a down job here
  for (int t = a.k - 1; t >= 0; --t)
    if (j >= (t + 1) * ncbI && j < (t + 1) * ncbI + ncbH) t0 = t;

  if (has_gu) gateup_prefetch_act(a, lds);
  const PlanLine* R = &a.plans[blockIdx.x % a.n_pub];
  if (threadIdx.x == 0) {
    const CallState cs = read_call_state(a.sync);
    *s_call = cs;
    const u64* src[2] = {&R->plan[g_gu], &R->plan[min(t0, a.k - 1)]};
    const bool use[2] = {true, true};
    u64 v[2];
    settle(src, use, v, (unsigned)cs.epoch + 1u, &a.sync->error, cs.spin_limit);
    s_plan[0] = (unsigned)v[0];
    s_plan[1] = (unsigned)v[1];
  }
  __syncthreads();
  const CallState cs = *s_call;
  const unsigned stamp = (unsigned)cs.epoch + 1u;
  const int spin_limit = cs.spin_limit;
  // clamped: the indices stay in bounds whatever the words hold
  auto expert = [&](unsigned p) { return min((int)(p & 0xffffu), a.E - 1); };
  auto slot_of = [&](unsigned p) { return min((int)(p >> 16), a.k - 1); };
  const unsigned p_gu = s_plan[0], p_d0 = s_plan[1];

  if (has_gu) {
    GateupLoads gl;
    gateup_issue<BLK>(a, j - g_gu * ncbI, expert(p_gu), gl);
    gateup_finish<BLK>(a, g_gu, j - g_gu * ncbI, stamp, lds, gl);
  }
  // the check-in's atomics wait on wave 3 where it has nothing else to do
  if (threadIdx.x == 3 * kWave) check_in(a.sync, cs.epoch);
  for (int t = t0; t < a.k; ++t) {
    const int cb = j - (t + 1) * ncbI;
    if (cb < 0 || cb >= ncbH) continue;
    unsigned p = p_d0;
    if (t != t0) {  // only when H/16 > I/16
      __syncthreads();
      if (threadIdx.x == 0) {
        const u64* src[1] = {&R->plan[t]};
        const bool use[1] = {true};
        u64 v[1];
        settle(src, use, v, stamp, &a.sync->error, spin_limit);
        s_plan[2] = (unsigned)v[0];
      }
      __syncthreads();
      p = s_plan[2];
    }
    if (!has_gu) {
      // a workgroup with no gate/up job requests its down weights only once
      // its tile's h has begun to arrive (one word, a different one per
      // workgroup), so they do not compete with the gate/up stream at its
      // start; they still land before the tile's h is complete (0.1 us per
      // call faster at 20b; requesting every down job's weights together with
      // the gate/up ones, straight into LDS, measured 2.3 us slower: the
      // mixed stream ran at 4.4 TB/s instead of 5.3)
      if (threadIdx.x == 0) {
        const u64* src[1] = {a.h + (size_t)t * a.I / 2 + (size_t)(cb % (a.I / 32)) * 16};
        const bool use[1] = {true};
        u64 v[1];
        settle(src, use, v, stamp, &a.sync->error, spin_limit);
      }
      __syncthreads();
    }
    DownLoads dl;
    down_issue(a, cb, expert(p), dl);
    down_finish(a, t, cb, slot_of(p), stamp, spin_limit, R, lds, dl);
  }
}

template <bool BLK>
constexpr int lds_bytes() {
  // GEMM workgroups: region 0 (x row / split-K table / h row), two scale
  // runs (the down job's reduction table sits in the second), the canonical
  // layout's exchange ring.  Routing workgroups use the start of the same
  // space for their RouteLds.
  return kRegion0 + 2 * kScaleRunMax + (BLK ? 0 : 2 * 2 * kRowsPerBlock * 256) + 16;
}
static_assert(sizeof(RouteLds) <= lds_bytes<true>(), "routing scratch fits");

template <bool BLK>
__global__ __launch_bounds__(kThreads, 4) void moe_layer_one_token_kernel(Args a) {
  __shared__ __align__(16) unsigned char lds[lds_bytes<BLK>()];
  __shared__ CallState s_call;
  __shared__ unsigned s_plan[4];
  if ((int)blockIdx.x < a.n_route)
    routing_role(a, blockIdx.x, reinterpret_cast<RouteLds*>(lds));
  else
    gemm_role<BLK>(a, blockIdx.x - a.n_route, lds, &s_call, s_plan);
}

size_t round_up(size_t n) { return (n + 255) / 256 * 256; }

}  // namespace

bool layer_one_token_ok(int H, int I, int E, int k) {
  if (!(H % 32 == 0 && I % 32 == 0 && H > 0 && I > 0 && H <= kMaxK && I <= kMaxK && E >= 1 &&
        E <= kMaxExperts && k >= 1 && k <= kMaxTopk && k <= E))
    return false;
  const RouterPlan p = router_plan(1, H, E);
  return p.splits <= kMaxSplits;
}

size_t layer_one_token_sync_bytes(int H) {
  (void)H;
  return round_up(sizeof(Sync)) + 2 * kPartialWords * sizeof(u64) +
         kMaxPublishers * sizeof(PlanLine);
}

size_t layer_one_token_bytes(int H, int I, int E, int k) {
  (void)E;
  return layer_one_token_sync_bytes(H) + round_up((size_t)k * (I / 2) * sizeof(u64)) +
         round_up((size_t)k * H * sizeof(u64));
}

void launch_layer_one_token(const uint16_t* x, const float* w_router, const float* bias,
                            const uint8_t* w13_q, const uint8_t* w13_s, const uint8_t* w2_q,
                            const uint8_t* w2_s, int H, int I, int E, int k, int gating,
                            bool blocked, int32_t* topk_ids,
                            float* topk_weights, double* logits, int32_t* expert_offsets,
                            int32_t* sorted_ids, int32_t* tiles, int32_t* num_tiles,
                            void* workspace, uint16_t* out, hipStream_t stream) {
  const RouterPlan p = router_plan(1, H, E);
  char* ws = static_cast<char*>(workspace);
  Args a;
  a.x = x; a.w_router = w_router; a.bias = bias;
  a.w13_q = w13_q; a.w13_s = w13_s; a.w2_q = w2_q; a.w2_s = w2_s;
  a.H = H; a.I = I; a.E = E; a.k = k; a.gating = gating; a.blocked = blocked;
  a.split_len = p.split_len;
  a.splits = p.splits;
  a.n_route = p.splits * ((E + kExpPerBlock - 1) / kExpPerBlock);
  a.topk_ids = topk_ids; a.topk_weights = topk_weights; a.logits = logits;
  a.expert_offsets = expert_offsets; a.sorted_ids = sorted_ids; a.tiles = tiles;
  a.num_tiles = num_tiles;
  a.sync = reinterpret_cast<Sync*>(ws);
  a.partials = reinterpret_cast<u64*>(ws + round_up(sizeof(Sync)));
  a.plans = reinterpret_cast<PlanLine*>(ws + round_up(sizeof(Sync)) +
                                        2 * kPartialWords * sizeof(u64));
  a.n_pub = a.n_route < kMaxPublishers ? a.n_route : kMaxPublishers;
  size_t off = layer_one_token_sync_bytes(H);
  a.h = reinterpret_cast<u64*>(ws + off);
  off += round_up((size_t)k * (I / 2) * sizeof(u64));
  a.y = reinterpret_cast<u64*>(ws + off);
  a.out = out;
  const int ncbI = I / kRowsPerBlock, ncbH = H / kRowsPerBlock;
  const int grid = a.n_route + k * ncbI + ncbH;
  if (blocked)
    hipLaunchKernelGGL(moe_layer_one_token_kernel<true>, dim3(grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(moe_layer_one_token_kernel<false>, dim3(grid), dim3(kThreads), 0, stream,
                       a);
}

}  // namespace moe
