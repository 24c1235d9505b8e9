// Grouped MXFP4 expert GEMMs for large token tiles (prefill).
//
// The SimpleLLM write-up grows the MoE token tile with tokens per expert so
// that a weight tile is unpacked once for many tokens instead of once per
// small tile ("A 297-line kernel file that decodes faster than vLLM",
// section "Optimizations", "MoE token tile follows tokens per expert"; a
// 4k-token prefill is its example).  This kernel is the MI355X form of that
// regime: per expert the work is a dense bf16 contraction, so it is built
// around the matrix cores and LDS.
//
// Unit of work: one workgroup of 8 waves takes a tile of up to 128 token
// rows of one expert and 384 weight rows (4 slices of 96).  Waves w and w+4
// (the two waves of one SIMD) share slice w & 3 and take three of its six
// 16-row weight fragments each, against all of the tile's token fragments
// (16 rows each, as many as the tile has rows): every weight is decoded by
// one wave only, and while one wave of a SIMD waits (on LDS, a barrier or its
// decoding) the other keeps the matrix core busy.
//   gate/up: a fragment holds 8 output columns, gate and up rows interleaved
//     (even row: gate, odd row: up, of the same column), so a lane and its
//     neighbour hold the two halves of SwiGLU; 192 output columns per unit.
//   down: a fragment is 16 rows of w2; 384 output columns per unit.
//
// K loop: 64 K per stage (two MX blocks), four stages in LDS, all of them in
// flight.  MFMA 16x16x32: lane group g supplies K elements
// 32*(g>>1) + 16*(g&1) + 8j .. +8 of the stage for step j = 0, 1 (any K order
// works as long as both operands use it), so a lane's weight operand is one
// 8-byte half of one MX block and its scale is one byte.  All loads in the
// loop are direct global->LDS 16-byte loads (global_load_lds_dwordx4), a
// fixed number per wave and stage, so a stage wait is an exact vmcnt:
//   * activations: 64 or 128 rows x 128 B (as many as the tile needs),
//     gathered by a row table, row r's eight 16-byte chunks stored at
//     chunk ^ ((r >> 1) & 7): a 128-bit read is served 16 lanes (one 256-byte
//     bank row) at a time, and the 16 rows a fragment read touches then cover
//     all 64 banks once (rows of one parity share a bank half);
//   * weights: per slice 96 rows x 32 B, row r's two MX blocks stored at
//     block ^ ((r >> 3) & 1) (conflict-free 64-bit reads).
// The E8M0 scales of the unit's rows (contiguous runs of the scale matrix)
// are loaded once, as raw 16-byte pieces, into an LDS slab.  Weights are
// decoded to bf16 in registers (v_cvt_scalef32_pk_bf16_fp4) right before
// their MFMAs.
//
// Grid: one workgroup per (tile, column block) unit, 1-D.  Workgroup w runs
// on XCD w % 8; units are renumbered so that each XCD takes a contiguous
// range, i.e. the column blocks of one token tile run side by side on one
// XCD and its activation rows are fetched into that XCD's L2 once.
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

namespace {

constexpr int kMT = 128;                           // token rows per tile (largest BM)
constexpr int kThreads = 512;                      // 8 waves, two per SIMD
constexpr int kBK = 64;                            // K per stage: two MX blocks
constexpr int kStages = 4;
constexpr int kXStage = kMT * kBK * 2;             // 16 KB of bf16 activations
constexpr int kWRowsSlice = 96;                    // weight rows staged per slice
constexpr int kWSlice = kWRowsSlice * kBK / 2;     // 3 KB of e2m1 codes per slice
constexpr int kWStage = 4 * kWSlice;
constexpr int kStage = kXStage + kWStage;          // 28 KB
constexpr int kWLoadsSlice = kWSlice / 1024;       // direct loads per slice and stage (3)
constexpr int kMaxKB = 96;                         // K <= 3072
constexpr int kSlabUnits = 5;                      // of kThreads pieces of 16 B
constexpr int kSlabBytes = kSlabUnits * kThreads * 16;  // 40 KB of raw scale bytes
constexpr int kLdsBytes = kStages * kStage + kSlabBytes + kMT * 8 + kMT * 4;
constexpr int kNFW = 3;                            // weight fragments per wave
constexpr int kColsGateUp = 48;                    // output columns per slice
constexpr int kColsDown = 96;

static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
static_assert(kWLoadsSlice == 3, "slice loads split 2 + 1 between the two waves of a SIMD");
static_assert(2 * kNFW * 16 == kWRowsSlice, "two waves of three fragments per slice");
// slab pieces: gate/up two runs of 192 rows, down one run of 384 rows
static_assert(2 * ((15 + 4 * kColsGateUp * kMaxKB + 15) / 16) <= kSlabUnits * kThreads, "slab");
static_assert((15 + 4 * kColsDown * kMaxKB + 15) / 16 <= kSlabUnits * kThreads, "slab size");

__device__ __forceinline__ bool tile_ok(int e, int r0, int rows, int E, long long nslots) {
  return e >= 0 && e < E && r0 >= 0 && rows > 0 && rows <= kMT && (long long)r0 + rows <= nslots;
}

// Direct global->LDS 16-byte load: lane l's data lands at lds + 16*l (lds is
// wave-uniform).  Issued as inline asm so that the compiler neither counts it
// nor adds its own vmcnt(0) before LDS reads; the kernel waits for its loads
// explicitly (vm_wait / wait_vm) before the barrier that publishes them.  No
// memory clobber: the target buffer is read only after a later wait and
// barrier (volatile asm statements keep their order), so LDS reads of other
// buffers may be scheduled across the load.
__device__ __forceinline__ void lds_load16(const void* g, unsigned char* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)lds);
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(m0));
}

// Wait until at most N of this wave's vector-memory loads are outstanding.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Same with a wave-uniform runtime count (0..15; larger counts wait for all).
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
    case 15: vm_wait<15>(); break;
    case 14: vm_wait<14>(); break;
    case 13: vm_wait<13>(); break;
    case 12: vm_wait<12>(); break;
    case 11: vm_wait<11>(); break;
    case 10: vm_wait<10>(); break;
    case 9: vm_wait<9>(); break;
    case 8: vm_wait<8>(); break;
    case 7: vm_wait<7>(); break;
    case 6: vm_wait<6>(); break;
    case 5: vm_wait<5>(); break;
    case 4: vm_wait<4>(); break;
    case 3: vm_wait<3>(); break;
    case 2: vm_wait<2>(); break;
    case 1: vm_wait<1>(); break;
    default: vm_wait<0>(); break;
  }
}

__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Everything a wave needs for the K loop and the epilogue of one unit.
struct UnitCtx {
  unsigned char* smem;
  const unsigned char* slab;
  const int* s_slot;
  const long long* s_rowoff;
  const uint16_t* act;
  const uint8_t* w_row[2];  // this lane's weight row for each of the wave's direct loads
  int w_swz[2];             // the MX block (0/1) of the stage it fetches
  int w_dst[2];             // its 1 KB slot within the stage's weight area
  int soff[kNFW];           // slab offset of this lane's row, per fragment
  int K, KB, niters, wave, lane, mg, wn, n0, N, H, I, r0, rows;
  long long nslots;
  void* out;
};

// Weight direct loads of stage `it` into buffer st: slice loads 0, 1 go to
// the first wave of the SIMD (mg = 0), load 2 to the second (WW = 2 - mg).
__device__ __forceinline__ void issue_w(const UnitCtx& c, int it, int st) {
  unsigned char* wsb = c.smem + st * kStage + kXStage;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (t < 2 - c.mg) {
      const int blk = min(2 * it + c.w_swz[t], c.KB - 1);  // past K: any data, scale 0
      lds_load16(c.w_row[t] + (size_t)blk * 16, wsb + c.w_dst[t]);
    }
  }
}

__device__ __forceinline__ void lds_wait_all() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// K loop and epilogue of one wave: its kNFW weight fragments (3*mg .. +2 of
// slice wn) against NM token fragments, XCW activation loads per wave and
// stage (1: rows 0..63 of the tile, 2: rows 0..127).  NM and XCW are
// compile-time constants so the loop body is straight-line code.
//
// Software pipeline, per iteration it (stage it in buffer it % 4):
//   step 0: read the step-1 activation operands of stage it; dequantize the
//           weights of step 0 and run its MFMAs;
//   sync:   stage it is fully read (lgkmcnt 0) and stage it+1 has landed
//           (vmcnt): barrier;
//   step 1: refill buffer it % 4 with stage it+4; read the step-0 operands
//           and the weights of stage it+1; dequantize and run the MFMAs of
//           step 1.
// LDS reads of the next step are in flight under the MFMAs of the current
// one, and one barrier per iteration both publishes a stage and frees a
// buffer.  Scheduling fences keep MFMAs from drifting across the sync.
template <bool GATEUP, int NM, int XCW>
__device__ __forceinline__ void unit_main(const UnitCtx& c) {
  constexpr int NF = kNFW;
  const int li = c.lane & 15;
  const int grp = c.lane >> 4;
  const int half = grp >> 1;  // MX block of the stage this lane feeds
  const int sub = grp & 1;    // which 8-byte half of it
  const int ww = 2 - c.mg;    // weight loads of this wave per stage
  const int niters = c.niters;
  // loads per stage of this wave; stages 0..3 had their weights in the prologue
  auto loads = [&](int s) { return s >= niters ? 0 : (s <= 3 ? XCW : XCW + ww); };

  // this lane's source rows of the activation loads (load t covers rows
  // 8L .. 8L+7, L = 8t + wave, the lane's row being 8L + (lane >> 3)); its
  // 16-byte slot (lane & 7) of the row holds chunk slot ^ ((row >> 1) & 7),
  // and (row >> 1) & 7 = (4 * (wave & 1) + (lane >> 4)) & 7 for every t
  const uint16_t* xsrc[XCW];
#pragma unroll
  for (int t = 0; t < XCW; ++t)
    xsrc[t] = c.act + c.s_rowoff[8 * (8 * t + c.wave) + (c.lane >> 3)];
  const int xchunk = (c.lane & 7) ^ ((4 * (c.wave & 1) + (c.lane >> 4)) & 7);
  auto issue_x = [&](int it, int st) {
    unsigned char* xs = c.smem + st * kStage;
    const int kel = min(it * kBK + 8 * xchunk, c.K - 8);
#pragma unroll
    for (int t = 0; t < XCW; ++t) lds_load16(xsrc[t] + kel, xs + (8 * t + c.wave) * 1024);
  };

  // LDS operand reads
  auto read_a = [&](const unsigned char* xs, int j, bf16x8 (&a)[NM]) {
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      const int r = 16 * i + li;
      a[i] = as_bf16x8(*reinterpret_cast<const uint4*>(
          xs + r * 128 + 16 * ((2 * grp + j) ^ ((r >> 1) & 7))));
    }
  };
  auto read_w = [&](const unsigned char* xs, int it, uint2 (&wr)[NF], float (&sc)[NF]) {
    const unsigned char* wsb = xs + kXStage + c.wn * kWSlice;
    const int blk = 2 * it + half;
    const uint32_t vmask = blk < c.KB ? ~0u : 0u;  // a missing last block scales to 0
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int rl = 16 * (NF * c.mg + f) + li;  // staged row within the slice
      wr[f] = *reinterpret_cast<const uint2*>(wsb + rl * 32 + 16 * (half ^ ((rl >> 3) & 1)) +
                                              8 * sub);
      const uint32_t sbits = __float_as_uint(e8m0_to_float(c.slab[c.soff[f] + blk]));
      sc[f] = __uint_as_float(sbits & vmask);
    }
  };

  floatx4 acc[NM][NF];
#pragma unroll
  for (int i = 0; i < NM; ++i)
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[i][f] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto step = [&](const bf16x8 (&a)[NM], const uint2 (&wr)[NF], const float (&sc)[NF], int j) {
    bf16x8 b[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) b[f] = dequant8_bf16(j ? wr[f].y : wr[f].x, sc[f]);
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int i = 0; i < NM; ++i) acc[i][f] = mfma16x16x32(a[i], b[f], acc[i][f]);
  };

  // stages 0..3 in flight (their weights were loaded in the prologue)
  for (int s = 0; s < 4 && s < niters; ++s) issue_x(s, s);
  wait_vm(loads(1) + loads(2) + loads(3));
  wg_barrier();  // stage 0 landed

  bf16x8 a0[NM], a1[NM];
  uint2 wcur[NF];
  float scur[NF];
  read_a(c.smem, 0, a0);
  read_w(c.smem, 0, wcur, scur);

  for (int it = 0; it < niters; ++it) {
    const unsigned char* xs = c.smem + (it & (kStages - 1)) * kStage;
    read_a(xs, 1, a1);
    step(a0, wcur, scur, 0);
    __builtin_amdgcn_sched_barrier(0);

    lds_wait_all();  // this wave is done reading stage it
    // its share of stage it+1 landed: only stages it+2, it+3 may be pending
    if (it >= 2 && it + 3 < niters) {
      if (c.mg == 0)
        vm_wait<2 * (XCW + 2)>();
      else
        vm_wait<2 * (XCW + 1)>();
    } else {
      wait_vm(loads(it + 2) + loads(it + 3));
    }
    wg_barrier();
    __builtin_amdgcn_sched_barrier(0);

    if (it + 4 < niters) {
      const int st = it & (kStages - 1);
      issue_x(it + 4, st);
      issue_w(c, it + 4, st);
    }
    // operands of stage it+1 (a stale buffer on the last iteration: unused)
    const unsigned char* xn = c.smem + ((it + 1) & (kStages - 1)) * kStage;
    uint2 wnext[NF];
    float snext[NF];
    read_a(xn, 0, a0);
    read_w(xn, it + 1, wnext, snext);

    step(a1, wcur, scur, 1);
#pragma unroll
    for (int f = 0; f < NF; ++f) { wcur[f] = wnext[f]; scur[f] = snext[f]; }
    __builtin_amdgcn_sched_barrier(0);
  }

  // epilogue straight from the accumulators: the lane holds D[4*grp + r][li]
  // of each (token fragment, weight fragment)
  const int cbase = c.n0 + (GATEUP ? kColsGateUp : kColsDown) * c.wn;
#pragma unroll
  for (int i = 0; i < NM; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * i + 4 * grp + r;
      if (GATEUP) {
        // even lane: gate, odd lane: up, of column cbase + 8*(3*mg + f) + li/2
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const float v = acc[i][f][r];
          const float up = __shfl_xor(v, 1);
          const int col = cbase + 8 * (NF * c.mg + f) + (li >> 1);
          if (row < c.rows && (li & 1) == 0 && col < c.N)
            reinterpret_cast<uint16_t*>(c.out)[(size_t)(c.r0 + row) * c.I + col] =
                float_to_bf16(silu(v) * up);
        }
      } else {
        if (row >= c.rows) continue;
        const long long p = c.s_slot[row];
        if (p < 0 || p >= c.nslots) continue;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const int col = cbase + 16 * (NF * c.mg + f) + li;
          if (col < c.N) reinterpret_cast<float*>(c.out)[(size_t)p * c.H + col] = acc[i][f][r];
        }
      }
    }
  }
}

template <bool GATEUP>
__global__ __launch_bounds__(kThreads, 1) void expert_mma_kernel(
    const uint16_t* __restrict__ act, const uint8_t* __restrict__ wq,
    const uint8_t* __restrict__ ws, const int32_t* sorted_ids,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ num_tiles, int T, int H,
    int I, int E, int k, int ncb, void* __restrict__ out) {
  constexpr int kCols = GATEUP ? kColsGateUp : kColsDown;  // output columns per slice
  constexpr int kRunRows = 4 * kCols;                        // rows per scale run
  constexpr int kRuns = GATEUP ? 2 : 1;                      // gate + up, or w2
  extern __shared__ __align__(16) unsigned char smem[];

  const int units = min(num_tiles[0] * ncb, (int)gridDim.x);
  const int w = blockIdx.x;
  if (w >= units) return;  // uniform over the workgroup
  const int xcd = w & 7;
  const int unit = xcd * (units >> 3) + min(xcd, units & 7) + (w >> 3);
  const int tile = unit / ncb;
  const int cb = unit - tile * ncb;

  const int e = tiles[3 * tile + 0];
  const int r0 = tiles[3 * tile + 1];
  const int rows = tiles[3 * tile + 2];
  const long long nslots = (long long)T * k;
  if (!tile_ok(e, r0, rows, E, nslots)) return;  // uniform

  UnitCtx c;
  c.smem = smem;
  c.act = act;
  c.K = GATEUP ? H : I;
  c.N = GATEUP ? I : H;
  c.KB = c.K / 32;
  c.niters = (c.KB + 1) / 2;
  c.n0 = cb * 4 * kCols;
  c.H = H; c.I = I; c.r0 = r0; c.rows = rows; c.nslots = nslots; c.out = out;
  const int tid = threadIdx.x;
  c.wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so branches on
  c.lane = tid & 63;                                   // it stay scalar
  c.wn = c.wave & 3;
  c.mg = c.wave >> 2;
  const int KB = c.KB;
  const int li = c.lane & 15;

  unsigned char* slab = smem + kStages * kStage;
  long long* s_rowoff = reinterpret_cast<long long*>(slab + kSlabBytes);
  int* s_slot = reinterpret_cast<int*>(s_rowoff + kMT);
  c.slab = slab;
  c.s_rowoff = s_rowoff;
  c.s_slot = s_slot;

  // rows of one expert's weight matrix (2I for gate/up, H for down), and the
  // rows of one run's half (I or H)
  const int mrows = GATEUP ? 2 * I : H;
  const int nvalid = GATEUP ? I : H;
  // slice row rl (0..95) of slice wn -> run (0: gate or w2, 1: up) and run row
  auto slice_row = [&](int wn, int rl, int& ch, int& rr) {
    const int f = rl >> 4, l = rl & 15;
    if (GATEUP) {
      ch = l & 1;
      rr = kCols * wn + 8 * f + (l >> 1);
    } else {
      ch = 0;
      rr = kCols * wn + 16 * f + l;
    }
  };

  // ---- prologue 1: the scale slab, raw 16-byte pieces of the runs of the
  // scale matrix that hold this unit's rows.  Run ch covers bytes
  // [c0, c0 + kRunRows*KB) and is fetched from a0 = c0 rounded down to 16.
  // Pieces past the last whole 16 bytes of the matrix are clamped in bounds;
  // the bytes they miss are read one by one after the wait below.
  const size_t total = (size_t)E * mrows * KB;
  const size_t whole = total & ~(size_t)15;
  size_t a0[kRuns];
  int skip[kRuns], npc[kRuns], pbase[kRuns];
  int npieces = 0;
#pragma unroll
  for (int ch = 0; ch < kRuns; ++ch) {
    const size_t c0 = ((size_t)e * mrows + (size_t)ch * I + c.n0) * KB;
    a0[ch] = c0 & ~(size_t)15;
    skip[ch] = (int)(c0 - a0[ch]);
    npc[ch] = (skip[ch] + kRunRows * KB + 15) >> 4;
    pbase[ch] = npieces;
    npieces += npc[ch];
  }
  const bool dma_slab = whole >= 16;
  if (dma_slab) {
    const int nunits = (npieces + kThreads - 1) / kThreads;  // <= kSlabUnits
    for (int u = 0; u < nunits; ++u) {
      const int p = min(u * kThreads + tid, npieces - 1);
      const int ch = (kRuns > 1 && p >= pbase[kRuns - 1]) ? kRuns - 1 : 0;
      const size_t g = min(a0[ch] + (size_t)(p - pbase[ch]) * 16, whole - 16);
      lds_load16(ws + g, slab + (size_t)(u * kThreads + c.wave * 64) * 16);
    }
  }

  // ---- prologue 2: weights of stages 0..3 (independent of the row table).
  // Slice load q covers staged rows 32q + (lane >> 1) of slice wn; the lane's
  // 16-byte slot (lane & 1) holds MX block slot ^ ((row >> 3) & 1).  Loads
  // 0, 1 belong to the wave with mg = 0, load 2 to the one with mg = 1.
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int q = c.mg ? 2 : t;
    const int rl = 32 * q + (c.lane >> 1);
    int ch, rr;
    slice_row(c.wn, rl, ch, rr);
    const size_t gr = (size_t)e * mrows + (size_t)ch * I + min(c.n0 + rr, nvalid - 1);
    c.w_row[t] = wq + gr * (size_t)(c.K / 2);
    c.w_swz[t] = (c.lane & 1) ^ ((rl >> 3) & 1);
    c.w_dst[t] = c.wn * kWSlice + q * 1024;
  }
  for (int s = 0; s < 4 && s < c.niters; ++s) issue_w(c, s, s);

  // ---- prologue 3: the row table
  if (tid < kMT) {
    const int rr = min(tid, rows - 1);
    const int slot = sorted_ids[r0 + rr];
    s_rowoff[tid] = GATEUP ? (long long)min(max(slot / k, 0), T - 1) * H
                           : (long long)(r0 + rr) * I;
    s_slot[tid] = slot;
  }
  vm_wait<0>();  // slab pieces and the first four weight stages are in LDS
  __syncthreads();

  // slab bytes the clamped pieces missed: [whole, total) when the matrix is
  // not a multiple of 16 bytes (all of it when it is under 16 bytes)
  const size_t tail0 = dma_slab ? whole : 0;
  bool fixed = false;
#pragma unroll
  for (int ch = 0; ch < kRuns; ++ch) {
    const size_t lo = max(a0[ch], tail0);
    const size_t hi = min(a0[ch] + (size_t)npc[ch] * 16, total);
    if (lo < hi) {
      fixed = true;
      for (size_t b = lo + tid; b < hi; b += kThreads)
        slab[(size_t)pbase[ch] * 16 + (b - a0[ch])] = ws[b];
    }
  }
  if (fixed) __syncthreads();  // uniform

  // slab offset of this lane's row, per fragment of the wave
#pragma unroll
  for (int f = 0; f < kNFW; ++f) {
    int ch, rr;
    slice_row(c.wn, 16 * (kNFW * c.mg + f) + li, ch, rr);
    c.soff[f] = pbase[ch] * 16 + skip[ch] + rr * KB;
  }

  // token fragments of the tile (all waves take all of them)
  switch ((rows + 15) >> 4) {
    case 8: unit_main<GATEUP, 8, 2>(c); break;
    case 7: unit_main<GATEUP, 7, 2>(c); break;
    case 6: unit_main<GATEUP, 6, 2>(c); break;
    case 5: unit_main<GATEUP, 5, 2>(c); break;
    case 4: unit_main<GATEUP, 4, 1>(c); break;
    case 3: unit_main<GATEUP, 3, 1>(c); break;
    case 2: unit_main<GATEUP, 2, 1>(c); break;
    default: unit_main<GATEUP, 1, 1>(c); break;
  }
}

}  // namespace

bool expert_mma_ok(int T, int H, int I, int E, int k, int BM) {
  // large token tiles, K small enough for the scale slab, and the expected
  // rows per expert large enough that 128-row tiles are mostly full
  const int Kmax = H > I ? H : I;
  return BM == kMT && Kmax <= 32 * kMaxKB && (long long)T * k >= 32LL * E;
}

void launch_expert_mma(bool gateup, const uint16_t* act, const uint8_t* wq, const uint8_t* ws,
                       const int32_t* sorted_ids, const int32_t* tiles, const int32_t* num_tiles,
                       int tiles_max, int T, int H, int I, int E, int k, void* out,
                       hipStream_t stream) {
  const int N = gateup ? I : H;
  const int ncol = 4 * (gateup ? kColsGateUp : kColsDown);
  const int ncb = (N + ncol - 1) / ncol;
  const dim3 grid((unsigned)tiles_max * (unsigned)ncb);
  if (gateup)
    hipLaunchKernelGGL(expert_mma_kernel<true>, grid, dim3(kThreads), kLdsBytes, stream, act, wq, ws,
                       sorted_ids, tiles, num_tiles, T, H, I, E, k, ncb, out);
  else
    hipLaunchKernelGGL(expert_mma_kernel<false>, grid, dim3(kThreads), kLdsBytes, stream, act, wq, ws,
                       sorted_ids, tiles, num_tiles, T, H, I, E, k, ncb, out);
}

}  // namespace moe
