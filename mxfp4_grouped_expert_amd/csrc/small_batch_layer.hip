// The whole MoE layer for a small batch (2 to 4 tokens) in a single launch:
// the one-launch scheme of the one-token layer (one_token_layer.hip) with
// tiles of several rows.
//
// The SimpleLLM write-up ("A 297-line kernel file that decodes faster than
// vLLM", section "Where the time went") books launch and host gaps as their
// own row of a decode step; with a handful of tokens the four dependent
// launches of the separate path (routing + tiles, gate/up, down, combine)
// each pay a launch and a ramp-up.  Here one grid holds all of it:
//   routing   splits x ceil(E/16) workgroups compute the fp64 partial logits
//             of every token (the 4-token body of router_logits_partial)
//             and publish them.  The first min(that, 32) of them, the
//             publishers, then each read all the partials; wave t sums token
//             t's in split order and runs the unfused path's wave top-k and
//             gating, one wave builds the tile table (build_tiles_wave, one
//             tile per selected expert: every expert gets at most T <= 4
//             rows), and each publisher publishes the plan in lines of its
//             own: per tile one word with its expert, row count, first sorted
//             position and the slots of its rows; per slot its routing
//             weight.  Publisher 0 also writes the routing outputs and the
//             table for the caller.
//   GEMM      workgroups run one job each: first every gate/up job (tile g,
//             16-row block), whose workgroups stage every token's x row at
//             their start (they do not depend on the routing), for the
//             tile's rows with the arithmetic of expert_gemm_kernel<gate/up,
//             1, XR>; then every down job, with that of
//             expert_gemm_kernel<down, 1, XR>.  The last tile's down job of
//             each 16-column block also combines the block for every token,
//             in ascending slot order, as combine_kernel does.
// Every value is bit-identical to moe_route_tiles + moe_forward: the router
// partials and their sums, the top-k and gating, the table, the GEMMs' lane
// mapping, MFMA order and split-K order, and the combine are the same
// arithmetic (the rows that share an MFMA do not change any row's result).
//
// Handshakes follow the one-token layer (one_launch.h): a workgroup only
// waits for workgroups with a lower index, every crossing value carries its
// validity in the same 64-bit word (partials: bits + 1 in a parity buffer;
// plan words, h pairs, y values: the call's epoch + 1), every poll is
// bounded, and the last workgroup to check in advances the epoch.
#include "expert_common.h"
#include "moe_device.h"
#include "moe_launch.h"
#include "one_launch.h"
#include "router_body.h"
#include "tiles_block.h"

namespace moe {

namespace {

constexpr int kThreads = 256;        // every role: 4 waves
constexpr int kMaxT = 4;             // tokens
constexpr int kMaxSlots = 16;        // T * k
constexpr int kMaxPub = 32;          // publishers
// The table's BM.  Every expert gets at most T <= kMaxT rows, so the table is
// the same for every BM the tile builder takes (one tile per expert).
constexpr int kTileRows = 16;
// staged rows (x at gate/up, h at down): up to kMaxT rows of K <= kMaxK
// bf16 with a 16-byte pad each, in 1 KB wave-instruction slots
constexpr int kActBytes = (kMaxT * (kMaxK * 2 + 16) + 1023) / 1024 * 1024;
constexpr int kRedBytes = 4 * 2 * 256 * 4;  // split-K table of a gate/up job
constexpr int kLdsBytes = kActBytes + 2 * kScaleRunMax + kRedBytes;

// partial words per parity buffer: [split][token][expert] at fixed strides
constexpr size_t kPartialWords = (size_t)kMaxSplits * kMaxT * kMaxExperts;

// A publisher's plan: per tile one word, per slot its routing weight.
// Tile word payload: expert (8 bits) | (rows - 1) << 8 | first sorted
// position << 10 | slot of row r << (14 + 4r); kNoTile for tiles past the
// table's end.
struct PlanBlock {
  u64 tile[kMaxSlots];
  u64 weight[kMaxSlots];
};
static_assert(sizeof(PlanBlock) == 256, "two lines per replica");
constexpr unsigned kNoTile = 1u << 31;

struct Args {
  const uint16_t* x;
  const float* w_router;
  const float* bias;
  const uint8_t* w13_q;
  const uint8_t* w13_s;
  const uint8_t* w2_q;
  const uint8_t* w2_s;
  int T, H, I, E, k, gating;
  int split_len, splits, n_route, n_pub, G;  // G: tiles the grid has jobs for
  int32_t* topk_ids;
  float* topk_weights;
  double* logits;
  int32_t* expert_offsets;
  int32_t* sorted_ids;
  int32_t* tiles;
  int32_t* num_tiles;
  Sync* sync;
  u64* partials;     // [2][kPartialWords]
  PlanBlock* plans;  // [kMaxPub]
  u64* h;            // [kMaxSlots][I/2] stamped bf16 pairs, by sorted position
  u64* y;            // [kMaxSlots][H] stamped fp32, by slot
  uint16_t* out;
};

struct TileInfo {
  int e, rows, r0;
  int slot[kMaxT];
  bool valid;
};
__device__ __forceinline__ TileInfo decode_tile(unsigned p, int E, int k, int T) {
  TileInfo t;
  t.valid = (p & kNoTile) == 0;
  t.e = min((int)(p & 0xffu), E - 1);  // clamped: indices stay in bounds
  t.rows = min((int)((p >> 8) & 3u) + 1, T);
  t.r0 = min((int)((p >> 10) & 15u), T * k - t.rows);
#pragma unroll
  for (int r = 0; r < kMaxT; ++r) t.slot[r] = min((int)((p >> (14 + 4 * r)) & 15u), T * k - 1);
  return t;
}

// ---------------------------------------------------------------- routing
struct RouteLds {
  long long rank[4][kRankScratch];
  int ids[kMaxSlots];
  float w[kMaxSlots];
  int tab[kWaveTablesScratch];
  int off[kBuckets + 1];
  int sorted[kMaxSlots];
  int tiles[3 * kMaxSlots];
  int ntiles;
};

__device__ void routing_role(const Args& a, int rid, RouteLds* r) {
  const CallState cs = read_call_state(a.sync);
  u64* cur = a.partials + (size_t)(cs.epoch & 1) * kPartialWords;
  u64* nxt = a.partials + (size_t)((cs.epoch & 1) ^ 1) * kPartialWords;
  const int eb = (a.E + kExpPerBlock - 1) / kExpPerBlock;
  logits_partial_compute<kTokPerWave>(
      a.x, a.w_router, a.T, a.H, a.E, a.split_len, 0, rid % eb, rid / eb,
      [&](int s, int t, int e, double v) {
        st64w(cur + ((size_t)s * kMaxT + t) * kMaxExperts + e, (u64)__double_as_longlong(v) + 1ull);
      });
  // the next call's buffer starts empty whatever shape wrote it last
  for (size_t i = (size_t)rid * kThreads + threadIdx.x; i < kPartialWords;
       i += (size_t)a.n_route * kThreads)
    st64w(nxt + i, 0ull);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 3 * kWave) check_in(a.sync, cs.epoch);
  if (rid >= a.n_pub) return;

  // a publisher: wave t takes token t
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & (kWave - 1);
  const unsigned stamp = (unsigned)cs.epoch + 1u;
  if (wave < a.T) {
    // one expert slot (64 experts) at a time: each settles up to
    // kMaxSplits words per lane, and all four at once would not fit the
    // registers of the GEMM roles' occupancy
    double val[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 1
    for (int i = 0; i < 4; ++i) {
      if (kWave * i >= a.E) break;  // uniform
      const int e = lane + kWave * i;
      double v = 0.0;
      if (e < a.E) {
        v = settle_partials(cur + (size_t)wave * kMaxExperts + e, (size_t)kMaxT * kMaxExperts,
                            a.splits, &a.sync->error, cs.spin_limit);
        if (a.bias) v += (double)a.bias[e];
      }
      val[i] = v;
    }
    if (a.logits && rid == 0)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lane + kWave * i < a.E) a.logits[(size_t)wave * a.E + lane + kWave * i] = val[i];
    topk_softmax_wave<true>(val, a.E, a.k, a.gating, wave, nullptr, nullptr, r->ids, r->w,
                            r->rank[wave]);
  }
  __syncthreads();
  if (wave != 0) return;
  const int N = a.T * a.k;
  build_tiles_wave(r->ids, N, a.E, kTileRows, r->tab, r->off, r->sorted, r->tiles, &r->ntiles);
  wave_lds_sync();
  PlanBlock* P = &a.plans[rid];
  const int nt = r->ntiles;
  if (lane < a.G) {
    unsigned p = kNoTile;
    if (lane < nt) {
      const int e = r->tiles[3 * lane], r0 = r->tiles[3 * lane + 1], rows = r->tiles[3 * lane + 2];
      p = (unsigned)e | (unsigned)(rows - 1) << 8 | (unsigned)r0 << 10;
      for (int q = 0; q < rows; ++q) p |= (unsigned)r->sorted[r0 + q] << (14 + 4 * q);
    }
    st64(&P->tile[lane], stamp, p);
  }
  if (lane < N) st64(&P->weight[lane], stamp, __float_as_uint(r->w[lane]));
  if (rid != 0) return;
  // publisher 0: the routing outputs and the table for the caller
  if (lane < N) {
    a.topk_ids[lane] = r->ids[lane];
    a.topk_weights[lane] = r->w[lane];
    a.sorted_ids[lane] = r->sorted[lane];
  }
  if (lane < nt) {
#pragma unroll
    for (int c = 0; c < 3; ++c) a.tiles[3 * lane + c] = r->tiles[3 * lane + c];
  }
  for (int e = lane; e <= a.E; e += kWave) a.expert_offsets[e] = r->off[e];
  if (lane == 0) a.num_tiles[0] = nt;
}

// --------------------------------------------------------------- staging
// The x rows of every token into LDS (16-byte slots, K/8 + 1 per row, the
// pad slot repeating the row's last chunk), requested at the workgroup's
// start with direct global->LDS loads.
__device__ __forceinline__ void stage_x(const Args& a, unsigned char* act) {
  const int cpr = a.H / 8, spr = cpr + 1;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int ninst = (a.T * spr + kWave - 1) / kWave;
  for (int ins = wave; ins < ninst; ins += 4) {  // wave-uniform
    const int slot = ins * kWave + lane;
    const int r = min(slot / spr, a.T - 1);
    const int c = min(slot - (slot / spr) * spr, cpr - 1);
    __builtin_amdgcn_global_load_lds(a.x + (size_t)r * a.H + (size_t)c * 8,
                                     (__attribute__((address_space(3))) void*)(act + ins * 1024),
                                     16, 0, 0);
  }
}

// ----------------------------------------------------------------- gate/up
// Tile g, 16-row block cb of the gate and up halves: the lane roles, loads,
// MFMA order, split-K order and epilogue of expert_gemm_kernel<true, 1, XR,
// true, true> (blocked codes) for the tile's rows.
struct GateupLoads {
  uint4 w[kChunk][2];
  uint4 spiece;
};

__device__ __forceinline__ void gateup_issue(const Args& a, int cb, int e, GateupLoads& L) {
  const int I = a.I, K = a.H, KB = K / 32;
  const int tid = threadIdx.x, lane = tid & 63, kq = tid >> 6;
  const int n_base = cb * kRowsPerBlock;
  const int pr = min(tid / KB, 1), pp = tid - pr * KB;
  L.spiece = *reinterpret_cast<const uint4*>(
      a.w13_s + ((size_t)e * 2 * I + (size_t)pr * I + n_base) * KB + (size_t)min(pp, KB - 1) * 16);
  asm volatile("" ::: "memory");
  const int l_row = n_base + (lane & 15);
  const size_t wrow[2] = {(size_t)e * 2 * I + l_row, (size_t)e * 2 * I + I + l_row};
#pragma unroll
  for (int c = 0; c < kChunk; ++c) {
    const int bc = min(c * kBlocksPerStep + kq * 4 + (lane >> 4), KB - 1);
#pragma unroll
    for (int w = 0; w < 2; ++w)
      L.w[c][w] = *reinterpret_cast<const uint4*>(a.w13_q + wq_row_offset(wrow[w], K / 2, true) +
                                                  (size_t)bc * wq_piece_stride(true));
  }
}

__device__ __forceinline__ void gateup_finish(const Args& a, const TileInfo& t, int cb,
                                              unsigned stamp, unsigned char* lds,
                                              GateupLoads& L) {
  constexpr int NW = 2;
  const int I = a.I, K = a.H, KB = K / 32;
  const int n_base = cb * kRowsPerBlock;
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, grp = lane >> 4;
  const int kq = tid >> 6;
  const int stride = act_stride_bytes(K);
  unsigned char* act = lds;                          // every token's x row
  unsigned char* s_sc = lds + kActBytes;             // 2 scale runs
  float* red = reinterpret_cast<float*>(s_sc + 2 * kScaleRunMax);

  wait_vmcnt<kChunk * NW>();  // the x rows and the scale piece
  const int pr = min(tid / KB, NW - 1), pp = tid - pr * KB;
  if (tid < NW * KB) *reinterpret_cast<uint4*>(s_sc + pr * kScaleRunMax + pp * 16) = L.spiece;
  // LDS-only barrier: every wave's share of the x rows has landed (waited
  // above) and the scale runs are stored; a full __syncthreads would also
  // wait for the weight stream the first steps' MFMAs overlap
  lds_barrier();

  uint32_t sreg[kChunk][NW];
#pragma unroll
  for (int c = 0; c < kChunk; ++c) {
    const int bc = min(c * kBlocksPerStep + kq * 4 + grp, KB - 1);
#pragma unroll
    for (int w = 0; w < NW; ++w) sreg[c][w] = s_sc[w * kScaleRunMax + li * KB + bc];
  }
  // MFMA row li: tile row min(li, rows - 1), i.e. the x row of its token
  int tok = t.slot[0] / a.k;
#pragma unroll
  for (int r = 1; r < kMaxT; ++r)
    if (r < t.rows && li >= r) tok = t.slot[r] / a.k;
  const unsigned char* arow = act + (size_t)min(tok, a.T - 1) * stride;
  floatx4 acc[NW] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int c = 0; c < kChunk; ++c) {
#pragma unroll
    for (int w = 0; w < NW; ++w)
      asm volatile("" : "+v"(L.w[c][w].x), "+v"(L.w[c][w].y), "+v"(L.w[c][w].z),
                   "+v"(L.w[c][w].w), "+v"(sreg[c][w]));
    const int b = c * kBlocksPerStep + kq * 4 + grp;
    const int bc = min(b, KB - 1);
    float scale[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) scale[w] = b < KB ? e8m0_to_float(sreg[c][w]) : 0.f;
    const uint4* ap = reinterpret_cast<const uint4*>(arow + bc * 64);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 av = as_bf16x8(ap[j]);
#pragma unroll
      for (int w = 0; w < NW; ++w)
        acc[w] = mfma16x16x32(av, dequant8_bf16(word(L.w[c][w], j), scale[w]), acc[w]);
    }
  }

  // split-K sum in wave order, then SwiGLU of each tile row
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
  const int tm = tid / kRowsPerBlock, tn = tid % kRowsPerBlock;
  const uint32_t hv = float_to_bf16(silu(v[0]) * v[NW - 1]);
  const uint32_t hn = (uint32_t)__float_as_int(swap_pair(__int_as_float((int)hv)));
  if (tm < t.rows && (tn & 1) == 0)  // one stamped word per bf16 pair
    st64(a.h + ((size_t)(t.r0 + tm) * I + n_base + tn) / 2, stamp, hv | (hn << 16));
}

// -------------------------------------------------------------------- down
// Tile t, 16-row block cb of w2: the arithmetic of expert_gemm_kernel<false,
// 1, XR, true, true> for the tile's rows.  The last tile's job also combines
// the block.
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
    L.w[c] = *reinterpret_cast<const uint4*>(a.w2_q + wq_row_offset(wrow, K / 2, true) +
                                             (size_t)bc * wq_piece_stride(true));
  }
  L.spiece = *reinterpret_cast<const uint4*>(
      a.w2_s + ((size_t)e * a.H + n_base) * KB + (size_t)min(tid, KB - 1) * 16);
}

// words of one staged h row a thread polls: (K/8 + 1) 16-byte slots of 4
// words
constexpr int kHPerRow = ((kMaxK / 8 + 1) * 4 + kThreads - 1) / kThreads;

__device__ __forceinline__ void down_finish(const Args& a, const TileInfo& t, int cb, bool last,
                                            unsigned stamp, int spin_limit,
                                            const PlanBlock* P, unsigned char* lds,
                                            DownLoads& L) {
  const int H = a.H, I = a.I, K = I, KB = K / 32;
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, grp = lane >> 4;
  const int kq = tid >> 6;
  const int n_base = cb * kRowsPerBlock;
  unsigned char* act = lds;                  // the tile's h rows
  unsigned char* s_sc = lds + kActBytes;     // scale run
  float* red = reinterpret_cast<float*>(s_sc + 2 * kScaleRunMax);
  const int stride = act_stride_bytes(K);

  __syncthreads();  // the LDS of any earlier job is free
  // the tile's h rows into LDS as their stamped pairs arrive, one row at a
  // time (all of a row's words requested at once, then re-polled where
  // still stale): the rows come from the same gate/up jobs, so once the
  // first has arrived the others normally have too, and polling all rows at
  // once would not fit the registers of this occupancy
  {
    const int cpr = K / 8, wpr = (cpr + 1) * 4;  // words per staged row, pad slot included
    unsigned* dst = reinterpret_cast<unsigned*>(act);
    const u64* src[kHPerRow];
    bool use[kHPerRow];
    u64 v[kHPerRow];
#pragma unroll 1
    for (int r = 0; r < t.rows; ++r) {
      const u64* hrow = a.h + (size_t)(t.r0 + r) * (I / 2);
#pragma unroll
      for (int i = 0; i < kHPerRow; ++i) {
        const int d = tid + i * kThreads;
        use[i] = d < wpr;
        src[i] = hrow + min(min(d, wpr - 1) >> 2, cpr - 1) * 4 + (d & 3);
      }
      settle(src, use, v, stamp, &a.sync->error, spin_limit);
#pragma unroll
      for (int i = 0; i < kHPerRow; ++i)
        if (use[i]) dst[r * wpr + tid + i * kThreads] = (unsigned)v[i];
    }
  }
  if (tid < KB) *reinterpret_cast<uint4*>(s_sc + tid * 16) = L.spiece;
  __syncthreads();

  uint32_t sreg[kChunk];
#pragma unroll
  for (int c = 0; c < kChunk; ++c)
    sreg[c] = s_sc[li * KB + min(c * kBlocksPerStep + kq * 4 + grp, KB - 1)];
  const unsigned char* arow = act + (size_t)min(li, t.rows - 1) * stride;
  floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < kChunk; ++c) {
    asm volatile("" : "+v"(L.w[c].x), "+v"(L.w[c].y), "+v"(L.w[c].z), "+v"(L.w[c].w),
                 "+v"(sreg[c]));
    const int b = c * kBlocksPerStep + kq * 4 + grp;
    const float scale = b < KB ? e8m0_to_float(sreg[c]) : 0.f;
    const uint4* ap = reinterpret_cast<const uint4*>(arow + min(b, KB - 1) * 64);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc = mfma16x16x32(as_bf16x8(ap[j]), dequant8_bf16(word(L.w[c], j), scale), acc);
  }
  __syncthreads();  // every wave done reading the h rows
#pragma unroll
  for (int r = 0; r < 4; ++r) red[kq * 256 + (4 * grp + r) * kRowsPerBlock + li] = acc[r];
  __syncthreads();
  const int tm = tid / kRowsPerBlock, tn = tid % kRowsPerBlock;
  float yv = red[tid];
#pragma unroll
  for (int q = 1; q < 4; ++q) yv += red[q * 256 + tid];
  if (tm < t.rows) {
    int slot = t.slot[0];
#pragma unroll
    for (int r = 1; r < kMaxT; ++r)
      if (r == tm) slot = t.slot[r];
    st64(a.y + (size_t)slot * H + n_base + tn, stamp, __float_as_uint(yv));
  }
  if (!last) return;
  // the last tile's job combines the block for every token: thread q polls
  // the routing weight and the y value of (slot q / 16, column q % 16) as
  // their stamped words arrive and parks them in LDS, then thread (token u,
  // column) runs the fma over u's slots in ascending order
  __builtin_amdgcn_s_waitcnt(0);  // this workgroup's own y words are out
  __syncthreads();                // and every thread is done with the table
  const int N = a.T * a.k;        // slots: N * 16 <= kThreads
  float* cw = red;
  float* cy = red + kMaxSlots * kRowsPerBlock;
  {
    const int sl = min(tid / kRowsPerBlock, N - 1);
    const u64* src[2] = {&P->weight[sl], a.y + (size_t)sl * H + n_base + tn};
    const bool use[2] = {tid < N * kRowsPerBlock, tid < N * kRowsPerBlock};
    u64 v[2];
    settle(src, use, v, stamp, &a.sync->error, spin_limit);
    if (use[0]) {
      cw[tid] = __uint_as_float((unsigned)v[0]);
      cy[tid] = __uint_as_float((unsigned)v[1]);
    }
  }
  __syncthreads();
  if (tid >= a.T * kRowsPerBlock) return;  // no barrier below
  const int u = tm;                        // token, column tn
  float acc_o = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxTopk; ++j)
    if (j < a.k)
      acc_o = fmaf(cw[(u * a.k + j) * kRowsPerBlock + tn], cy[(u * a.k + j) * kRowsPerBlock + tn],
                   acc_o);
  a.out[(size_t)u * H + n_base + tn] = float_to_bf16(acc_o);
}

// ------------------------------------------------------- GEMM workgroups
// Workgroup j (after the routing ones) runs one job: gate/up job j (tile
// j / (I/16), block j % (I/16)) when j < G * I/16, else down job d = j -
// G * I/16 (tile d / (H/16), block d % (H/16)).  Every down job sits above
// every gate/up job, and the last tile's down job of a block above the other
// tiles' jobs of that block.  (With one token, where all workgroups fit on
// the GPU at once, a workgroup pairs a gate/up job with a down job; here
// the grid is several times what fits, and down jobs that wait for their
// tile's h would hold their CU while gate/up jobs of later tiles wait to be
// dispatched.)  Jobs of tiles past the table's end return at once.
__device__ void gemm_role(const Args& a, int j, unsigned char* lds, CallState* s_call,
                          unsigned* s_plan) {
  const int ncbI = a.I / kRowsPerBlock, ncbH = a.H / kRowsPerBlock;
  const bool gu = j < a.G * ncbI;
  const int d = j - a.G * ncbI;
  const int tile = gu ? j / ncbI : min(d / ncbH, a.G - 1);
  const int cb = gu ? j - tile * ncbI : d - tile * ncbH;

  if (gu) stage_x(a, lds);
  const PlanBlock* P = &a.plans[blockIdx.x % a.n_pub];
  if (threadIdx.x == 0) {
    const CallState cs = read_call_state(a.sync);
    *s_call = cs;
    // the job's tile and, for a down job, the next one (whether the tile
    // is the table's last)
    const u64* src[2] = {&P->tile[tile], &P->tile[min(tile + 1, a.G - 1)]};
    const bool use[2] = {true, !gu && tile + 1 < a.G};
    u64 v[2];
    settle(src, use, v, (unsigned)cs.epoch + 1u, &a.sync->error, cs.spin_limit);
    s_plan[0] = (unsigned)v[0];
    s_plan[1] = use[1] ? (unsigned)v[1] : kNoTile;
  }
  __syncthreads();
  const CallState cs = *s_call;
  const unsigned stamp = (unsigned)cs.epoch + 1u;
  // the check-in's atomics wait on wave 3 where it has nothing else to do
  if (threadIdx.x == 3 * kWave) check_in(a.sync, cs.epoch);
  const TileInfo t = decode_tile(s_plan[0], a.E, a.k, a.T);
  if (!t.valid) {  // uniform; no barrier below for this workgroup
    __builtin_amdgcn_s_waitcnt(0);  // the x rows land before the workgroup ends
    return;
  }
  if (gu) {
    GateupLoads gl;
    gateup_issue(a, cb, t.e, gl);
    gateup_finish(a, t, cb, stamp, lds, gl);
  } else {
    DownLoads dl;
    down_issue(a, cb, t.e, dl);
    down_finish(a, t, cb, (s_plan[1] & kNoTile) != 0, stamp, cs.spin_limit, P, lds, dl);
  }
}

static_assert(sizeof(RouteLds) <= kLdsBytes, "routing scratch fits");

__global__ __launch_bounds__(kThreads, 4) void moe_layer_small_batch_kernel(Args a) {
  __shared__ __align__(16) unsigned char lds[kLdsBytes];
  __shared__ CallState s_call;
  __shared__ unsigned s_plan[8];
  if ((int)blockIdx.x < a.n_route)
    routing_role(a, blockIdx.x, reinterpret_cast<RouteLds*>(lds));
  else
    gemm_role(a, blockIdx.x - a.n_route, lds, &s_call, s_plan);
}

size_t round_up(size_t n) { return (n + 255) / 256 * 256; }

}  // namespace

bool layer_small_batch_ok(int T, int H, int I, int E, int k) {
  if (!(T >= 2 && T <= kMaxT && T * k <= kMaxSlots && H % 32 == 0 && I % 32 == 0 && H > 0 &&
        I > 0 && H <= kMaxK && I <= kMaxK && E >= 1 && E <= kMaxExperts && k >= 1 &&
        k <= kMaxTopk && k <= E))
    return false;
  const RouterPlan p = router_plan(T, H, E);
  return p.splits <= kMaxSplits;
}

size_t layer_small_batch_sync_bytes() {
  return round_up(sizeof(Sync)) + 2 * kPartialWords * sizeof(u64) + kMaxPub * sizeof(PlanBlock);
}

size_t layer_small_batch_bytes(int H, int I) {
  return layer_small_batch_sync_bytes() + round_up((size_t)kMaxSlots * (I / 2) * sizeof(u64)) +
         round_up((size_t)kMaxSlots * H * sizeof(u64));
}

void launch_layer_small_batch(const uint16_t* x, const float* w_router, const float* bias,
                              const uint8_t* w13_q, const uint8_t* w13_s, const uint8_t* w2_q,
                              const uint8_t* w2_s, int T, int H, int I, int E, int k,
                              int gating, int32_t* topk_ids, float* topk_weights, double* logits,
                              int32_t* expert_offsets, int32_t* sorted_ids, int32_t* tiles,
                              int32_t* num_tiles, void* workspace, uint16_t* out,
                              hipStream_t stream) {
  const RouterPlan p = router_plan(T, H, E);
  char* ws = static_cast<char*>(workspace);
  Args a;
  a.x = x; a.w_router = w_router; a.bias = bias;
  a.w13_q = w13_q; a.w13_s = w13_s; a.w2_q = w2_q; a.w2_s = w2_s;
  a.T = T; a.H = H; a.I = I; a.E = E; a.k = k; a.gating = gating;
  a.split_len = p.split_len;
  a.splits = p.splits;
  a.n_route = p.splits * ((E + kExpPerBlock - 1) / kExpPerBlock);
  a.n_pub = a.n_route < kMaxPub ? a.n_route : kMaxPub;
  a.G = T * k < E ? T * k : E;
  a.topk_ids = topk_ids; a.topk_weights = topk_weights; a.logits = logits;
  a.expert_offsets = expert_offsets; a.sorted_ids = sorted_ids; a.tiles = tiles;
  a.num_tiles = num_tiles;
  a.sync = reinterpret_cast<Sync*>(ws);
  a.partials = reinterpret_cast<u64*>(ws + round_up(sizeof(Sync)));
  a.plans = reinterpret_cast<PlanBlock*>(ws + round_up(sizeof(Sync)) +
                                         2 * kPartialWords * sizeof(u64));
  size_t off = layer_small_batch_sync_bytes();
  a.h = reinterpret_cast<u64*>(ws + off);
  off += round_up((size_t)kMaxSlots * (I / 2) * sizeof(u64));
  a.y = reinterpret_cast<u64*>(ws + off);
  a.out = out;
  const int ncbI = I / kRowsPerBlock, ncbH = H / kRowsPerBlock;
  const int grid = a.n_route + a.G * (ncbI + ncbH);
  hipLaunchKernelGGL(moe_layer_small_batch_kernel, dim3(grid), dim3(kThreads), 0, stream, a);
}

}  // namespace moe
