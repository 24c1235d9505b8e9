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
// rows of one expert (160 when it takes over the expert's remainder tile,
// see the kernel) and 384 weight rows (4 slices of 96).  Waves w and w+4
// (the two waves of one SIMD) share slice w & 3: each decodes all six 16-row
// weight fragments of the slice and multiplies them against its own half of
// the tile's token fragments (16 rows each; the first ceil(n/2) of the n
// fragments go to the wave with mg = 0).  The two waves of a SIMD run
// ping-pong: while one issues the MFMAs of a stage the other reads and
// decodes its operands of the next one, and the roles swap at every
// workgroup barrier.
//   gate/up: a fragment holds 8 output columns, gate and up rows interleaved
//     (even row: gate, odd row: up, of the same column), so a lane and its
//     neighbour hold the two halves of SwiGLU; 192 output columns per unit.
//   down: a fragment is 16 rows of w2, fragment f of slice s being the
//     unit's 16-row group 4f + s; 384 output columns per unit (a unit whose
//     columns end within the first 192 runs three fragments per wave).
//
// K loop: 64 K per stage (two MX blocks), three stage buffers in LDS: the
// stage being read and two in flight.  MFMA 16x16x32: lane group g supplies
// K elements 32*(g>>1) + 16*(g&1) + 8j .. +8 of the stage for step j = 0, 1
// (any K order works as long as both operands use it), so a lane's weight
// operand is one 8-byte half of one MX block and its scale is one byte.  All loads in the
// loop are direct global->LDS 16-byte loads (global_load_lds_dwordx4), a
// fixed number per wave and stage, so a stage wait is an exact vmcnt:
//   * activations: 64, 128 or 192 rows x 128 B (as many as the unit needs),
//     gathered by a row table, row r's eight 16-byte chunks stored at
//     chunk ^ ((r >> 1) & 7): a 128-bit read is served 16 lanes (one 256-byte
//     bank row) at a time, and the 16 rows a fragment read touches then cover
//     all 64 banks once (rows of one parity share a bank half);
//   * weights: per slice 96 rows x 32 B, row r's two MX blocks stored at
//     block ^ ((r >> 3) & 1) (conflict-free 64-bit reads).
// The E8M0 scales of the unit's rows (contiguous runs of the scale matrix)
// are loaded once, as raw 16-byte pieces, into an LDS slab.  Weights are
// decoded to bf16 in registers (v_cvt_scalef32_pk_bf16_fp4) in the load
// phase before their MFMAs.
//
// Grid: one workgroup per (tile, column block) unit, 1-D.  Workgroup w runs
// on XCD w % 8; units are renumbered so that each XCD takes a contiguous
// range, i.e. the column blocks of one token tile run side by side on one
// XCD and its activation rows are fetched into that XCD's L2 once.
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

namespace {

constexpr int kMT = 128;                           // token rows per tile (the tile table's BM)
constexpr int kUnitRows = 160;                     // token rows per unit (a tile + remainder)
constexpr int kXRows = 192;                        // activation rows staged (3 loads of 64)
constexpr int kThreads = 512;                      // 8 waves, two per SIMD
constexpr int kBK = 64;                            // K per stage: two MX blocks
constexpr int kStages = 3;
constexpr int kXStage = kXRows * kBK * 2;          // 24 KB of bf16 activations
constexpr int kWRowsSlice = 96;                    // weight rows staged per slice
constexpr int kWSlice = kWRowsSlice * kBK / 2;     // 3 KB of e2m1 codes per slice
constexpr int kWStage = 4 * kWSlice;
constexpr int kStage = kXStage + kWStage;          // 28 KB
constexpr int kWLoadsSlice = kWSlice / 1024;       // direct loads per slice and stage (3)
constexpr int kSlabUnits = 6;                      // of kThreads pieces of 16 B
constexpr int kSlabBytes = kSlabUnits * kThreads * 16;  // 48 KB of raw scale bytes
constexpr int kLdsBytes = kStages * kStage + kSlabBytes + kXRows * 8 + kXRows * 4;
constexpr int kNFW = 6;                            // weight fragments per wave
constexpr int kColsGateUp = 48;                    // output columns per slice
constexpr int kColsDown = 96;

static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
static_assert(kWLoadsSlice == 3, "slice loads split 2 + 1 between the two waves of a SIMD");
static_assert(kNFW * 16 == kWRowsSlice, "one wave decodes a whole slice");
// 16-byte pieces of the scale slab for K = 32 * KB: gate/up two runs of 192
// rows, down one run of 384 rows, each run fetched from its first byte
// rounded down to 16 (a run starts at a multiple of KB bytes, so at a
// multiple of 16 when KB is one)
__host__ __device__ constexpr int slab_pieces(bool gateup, int KB) {
  const int run_rows = gateup ? 4 * kColsGateUp : 4 * kColsDown;
  return (gateup ? 2 : 1) * (((KB % 16 ? 15 : 0) + run_rows * KB + 15) / 16);
}
// every K up to 3072 fits, and K = 4096 (KB = 128, runs 16-byte aligned)
static_assert(slab_pieces(true, 96) <= kSlabUnits * kThreads, "slab size");
static_assert(slab_pieces(false, 96) <= kSlabUnits * kThreads, "slab size");
static_assert(slab_pieces(true, 128) <= kSlabUnits * kThreads, "slab size");
static_assert(slab_pieces(false, 128) <= kSlabUnits * kThreads, "slab size");

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
  int w_pstride;            // bytes between consecutive MX blocks of a row (layout)
  int w_swz[2];             // the MX block (0/1) of the stage it fetches
  int w_dst[2];             // its 1 KB slot within the stage's weight area
  int soff[kNFW];           // slab offset of this lane's row, per fragment
  int K, KB, niters, wave, lane, mg, wn, n0, N, H, I, r0, rows, e;
  long long nslots;
  void* out;
  ExpertAct fn;
};

// Weight direct loads of stage `it` into buffer st: slice loads 0, 1 go to
// the first wave of the SIMD (mg = 0), load 2 to the second (WW = 2 - mg).
__device__ __forceinline__ void issue_w(const UnitCtx& c, int it, int st) {
  unsigned char* wsb = c.smem + st * kStage + kXStage;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (t < 2 - c.mg) {
      const int blk = min(2 * it + c.w_swz[t], c.KB - 1);  // past K: any data, scale 0
      lds_load16(c.w_row[t] + (size_t)blk * c.w_pstride, wsb + c.w_dst[t]);
    }
  }
}

__device__ __forceinline__ void lds_wait_all() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// K loop and epilogue of one wave: the first NF weight fragments of slice
// wn (all kNFW, or 3 in a down unit whose columns end within the first three
// fragments of every slice) against NMW token fragments starting at tile row
// mrow0, with XCW activation loads per wave and stage (1: rows 0..63 of the
// unit, 2: rows 0..127, 3: rows 0..191).  NMW (0..5), XCW and NF are
// compile-time constants so the loop body is straight-line code; a wave with
// NMW = 0 only loads and syncs.
template <bool GATEUP, int NMW, int XCW, int NF = kNFW>
__device__ __forceinline__ void unit_main(const UnitCtx& c, int mrow0) {
  static_assert(NF == kNFW || (!GATEUP && NF == 3), "short units: down only");
  constexpr int NA = NMW > 0 ? NMW : 1;  // array extent
  const int li = c.lane & 15;
  const int grp = c.lane >> 4;
  const int half = grp >> 1;  // MX block of the stage this lane feeds
  const int sub = grp & 1;    // which 8-byte half of it
  const int ww = 2 - c.mg;    // weight loads of this wave per stage
  const int niters = c.niters;
  // loads per stage of this wave: stages 0 and 1 are issued before the loop
  // (their weights, and those of stage 2, came with the prologue);
  // stage s >= 2 is issued in iteration s - 2 with its weights.  Stages past
  // the last one are loaded too (clamped, in-bounds addresses, into a buffer
  // that is not read again), so the loop issues a fixed number of loads per
  // iteration.  Two stages ahead measured faster than three (fewer loads in
  // flight compete less with the MFMA phases).
  auto loads = [&](int s) { return s <= 1 ? XCW : XCW + ww; };

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

  // activation operands of step j of a stage
  auto read_a = [&](const unsigned char* xs, int j, bf16x8 (&a)[NA]) {
#pragma unroll
    for (int i = 0; i < NMW; ++i) {
      const int r = mrow0 + 16 * i + li;
      a[i] = as_bf16x8(*reinterpret_cast<const uint4*>(
          xs + r * 128 + 16 * ((2 * grp + j) ^ ((r >> 1) & 7))));
    }
  };
  // weights (8-byte halves of MX blocks) and raw E8M0 bytes of stage `it`
  auto read_w = [&](const unsigned char* xs, int it, uint2 (&wr)[NF], uint32_t (&sr)[NF]) {
    const unsigned char* wsb = xs + kXStage + c.wn * kWSlice;
    const int blk = 2 * it + half;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int rl = 16 * f + li;  // staged row within the slice
      wr[f] = *reinterpret_cast<const uint2*>(wsb + rl * 32 + 16 * (half ^ ((rl >> 3) & 1)) +
                                              8 * sub);
      sr[f] = c.slab[c.soff[f] + blk];
    }
  };
  // E8M0 bytes -> float scales of stage `it`; a missing last MX block (odd
  // K / 32) scales to 0
  auto scales = [&](int it, const uint32_t (&sr)[NF], float (&sc)[NF]) {
    const uint32_t vmask = 2 * it + half < c.KB ? ~0u : 0u;
#pragma unroll
    for (int f = 0; f < NF; ++f) sc[f] = __uint_as_float(__float_as_uint(e8m0_to_float(sr[f])) & vmask);
  };
  // bf16 weight operands of step j
  auto decode = [&](int j, const uint2 (&wr)[NF], const float (&sc)[NF], bf16x8 (&b)[NF]) {
#pragma unroll
    for (int f = 0; f < NF; ++f) b[f] = dequant8_bf16(j ? wr[f].y : wr[f].x, sc[f]);
  };

  floatx4 acc[NA][NF];
#pragma unroll
  for (int i = 0; i < NA; ++i)
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[i][f] = floatx4{0.f, 0.f, 0.f, 0.f};

  // MFMAs of weight fragments f0 .. f1-1 against the wave's token fragments
  auto mfmas = [&](const bf16x8 (&a)[NA], const bf16x8 (&b)[NF], int f0, int f1) {
#pragma unroll
    for (int f = f0; f < f1; ++f)
#pragma unroll
      for (int i = 0; i < NMW; ++i) acc[i][f] = mfma16x16x32(a[i], b[f], acc[i][f]);
  };

  // Ping-pong between the two waves of a SIMD.  Phases are separated by
  // workgroup barriers; in every phase one group of waves (one wave per
  // SIMD) runs MFMAs while the other reads and decodes the operands of its
  // next stage, so each SIMD's matrix core and its VALU/LDS work overlap
  // without relying on the two waves drifting apart.  Group 0 (mg = 0)
  // loads stage it in phase 2it and multiplies it in phase 2it+1; group 1
  // runs half a stage behind (load in 2it+1, multiply in 2it+2).
  bf16x8 a[2][NA], b[2][NF];
  // load phase: all operands of stage `it`, decoded, in registers
  auto load_phase = [&](int it) {
    if (NMW > 0) {
      const unsigned char* xs = c.smem + (it % kStages) * kStage;
      uint2 wr[NF];
      uint32_t sr[NF];
      float sc[NF];
      read_w(xs, it, wr, sr);
      read_a(xs, 0, a[0]);
      read_a(xs, 1, a[1]);
      scales(it, sr, sc);
      decode(0, wr, sc, b[0]);
      decode(1, wr, sc, b[1]);
      lds_wait_all();  // the stage may be refilled two phases on
      // the decoded operands are complete here, not sunk into the MFMA phase
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int f = 0; f < NF; ++f) asm volatile("" : "+v"(b[j][f]));
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // MFMA phase: stage `it`; this wave also issues its share of stage it+2,
  // into the buffer of stage it-1 (group 0 read it two phases earlier, group
  // 1 in the phase that ended at the previous barrier)
  auto mfma_phase = [&](int it) {
    const int st = (it + 2) % kStages;
    issue_x(it + 2, st);
    issue_w(c, it + 2, st);
    if (NMW > 0) {
      __builtin_amdgcn_s_setprio(1);
      mfmas(a[0], b[0], 0, NF);
      mfmas(a[1], b[1], 0, NF);
      __builtin_amdgcn_s_setprio(0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    wg_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // stages 0 and 1 in flight; every wave's share of stage 0 lands before the
  // first barrier.  Before phase 2s (group 0 reads stage s) every wave's
  // share of stage s has landed: group 0 then has stage s+1 pending at most,
  // group 1 (which issued up to stage s) nothing.
  for (int s = 0; s < 2; ++s) issue_x(s, s);
  wait_vm(loads(1));
  barrier();
  if (c.mg == 0) {
    for (int it = 0; it < niters; ++it) {
      load_phase(it);                       // phase 2it
      barrier();
      mfma_phase(it);                       // phase 2it+1
      wait_vm(loads(it + 2));
      barrier();
    }
    // phase 2*niters: group 1's last MFMA phase
  } else {
    barrier();                              // phase 0: group 0's first load
    for (int it = 0; it < niters; ++it) {
      load_phase(it);                       // phase 2it+1
      vm_wait<0>();
      barrier();
      mfma_phase(it);                       // phase 2it+2
      if (it + 1 < niters) barrier();
    }
  }
  vm_wait<0>();  // the loads past the last stage

  // epilogue straight from the accumulators: the lane holds D[4*grp + r][li]
  // of each (token fragment, weight fragment)
  const int cbase = c.n0 + kColsGateUp * c.wn;  // gate/up: the slice's 48 columns
  if (GATEUP) {
    // A lane pair (even: gate, odd: up, of column cbase + 8*f + li/2) swaps
    // half of its rows, so that the even lane finishes rows 0, 1 of its four
    // and the odd lane rows 2, 3: each SwiGLU is evaluated once.
    const bool odd = li & 1;
    const int col0 = cbase + (li >> 1);
#pragma unroll
    for (int i = 0; i < NMW; ++i) {
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const floatx4 v = acc[i][f];
        const float send0 = odd ? v[0] : v[2];
        const float send1 = odd ? v[1] : v[3];
        const float got0 = swap_pair(send0);
        const float got1 = swap_pair(send1);
        // (gate, up) of rows q = 0, 1 (even lane) or q = 2, 3 (odd lane)
        const float g0 = odd ? got0 : v[0], u0 = odd ? v[2] : got0;
        const float g1 = odd ? got1 : v[1], u1 = odd ? v[3] : got1;
        const int row = mrow0 + 16 * i + 4 * grp + (odd ? 2 : 0);
        const int col = col0 + 8 * f;
        uint16_t* o = reinterpret_cast<uint16_t*>(c.out) + (size_t)(c.r0 + row) * c.I + col;
        if (col < c.N) {
          float h0, h1;
          if (c.fn.kind == 0) {
            h0 = silu_fast(g0) * u0;
            h1 = silu_fast(g1) * u1;
          } else {
            const float bg = c.fn.b13 ? c.fn.b13[(size_t)c.e * 2 * c.I + col] : 0.f;
            const float bu = c.fn.b13 ? c.fn.b13[(size_t)c.e * 2 * c.I + c.I + col] : 0.f;
            h0 = act_gptoss_fast(g0 + bg, u0 + bu, c.fn.alpha, c.fn.limit);
            h1 = act_gptoss_fast(g1 + bg, u1 + bu, c.fn.alpha, c.fn.limit);
          }
          if (row < c.rows) o[0] = float_to_bf16(h0);
          if (row + 1 < c.rows) o[c.I] = float_to_bf16(h1);
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < NMW; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = mrow0 + 16 * i + 4 * grp + r;
        if (row >= c.rows) continue;
        const long long p = c.s_slot[row];
        if (p < 0 || p >= c.nslots) continue;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const int col = c.n0 + 16 * (4 * f + c.wn) + li;  // fragment f of slice wn
          if (col < c.N) {
            const float bias =
                c.fn.kind != 0 && c.fn.b2 ? c.fn.b2[(size_t)c.e * c.H + col] : 0.f;
            reinterpret_cast<float*>(c.out)[(size_t)p * c.H + col] =
                c.fn.kind != 0 ? acc[i][f][r] + bias : acc[i][f][r];
          }
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
    int I, int E, int k, int ncb, bool blocked, void* __restrict__ out, ExpertAct fn) {
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
  const int trows = tiles[3 * tile + 2];
  const long long nslots = (long long)T * k;
  if (!tile_ok(e, r0, trows, E, nslots)) return;  // uniform
  // An expert's rows past its last full tile (a remainder tile of at most
  // kUnitRows - kMT rows) are computed by the unit of that full tile, so the
  // expert's weights are staged and decoded once for all its rows: tile b is
  // absorbed by tile a = b - 1 when both hold rows of one expert, b's rows
  // continue a's, a is full and the two fit one unit.  (A full tile cannot
  // itself be absorbed, so no chains form; both units test the same rows.)
  auto absorbs = [&](int ea, int ra, int na, int eb, int rb, int nb) {
    return ea == eb && ra + na == rb && na == kMT && na + nb <= kUnitRows &&
           tile_ok(ea, ra, na, E, nslots) && tile_ok(eb, rb, nb, E, nslots);
  };
  const int ntl = units / ncb;  // whole tiles of the table (tile < ntl)
  if (tile > 0 && absorbs(tiles[3 * tile - 3], tiles[3 * tile - 2], tiles[3 * tile - 1], e, r0,
                          trows))
    return;  // uniform: computed by the previous tile's unit
  int rows = trows;
  if (tile + 1 < ntl && absorbs(e, r0, trows, tiles[3 * tile + 3], tiles[3 * tile + 4],
                                tiles[3 * tile + 5]))
    rows += tiles[3 * tile + 5];

  UnitCtx c;
  c.smem = smem;
  c.act = act;
  c.K = GATEUP ? H : I;
  c.N = GATEUP ? I : H;
  c.KB = c.K / 32;
  c.niters = (c.KB + 1) / 2;
  c.n0 = cb * 4 * kCols;
  c.H = H; c.I = I; c.r0 = r0; c.rows = rows; c.nslots = nslots; c.out = out;
  c.e = e;
  c.fn = fn;
  const int tid = threadIdx.x;
  c.wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so branches on
  c.lane = tid & 63;                                   // it stay scalar
  c.wn = c.wave & 3;
  c.mg = c.wave >> 2;
  const int KB = c.KB;
  const int li = c.lane & 15;

  unsigned char* slab = smem + kStages * kStage;
  long long* s_rowoff = reinterpret_cast<long long*>(slab + kSlabBytes);
  int* s_slot = reinterpret_cast<int*>(s_rowoff + kXRows);
  c.slab = slab;
  c.s_rowoff = s_rowoff;
  c.s_slot = s_slot;

  // rows of one expert's weight matrix (2I for gate/up, H for down), and the
  // rows of one run's half (I or H).  Down: fragment f of slice wn is the
  // unit's 16-column group 4f + wn, so that a unit whose columns end early
  // (the last of 2880 = 7.5 x 384) spreads its valid groups over all four
  // SIMDs and runs short (NF = 3) instead of leaving two SIMDs idle.
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
      rr = 16 * (4 * f + wn) + l;
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
    const int nunits = (npieces + kThreads - 1) / kThreads;  // <= kSlabUnits (expert_mma_ok)
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
    c.w_row[t] = wq + wq_row_offset(gr, (size_t)(c.K / 2), blocked);
    c.w_swz[t] = (c.lane & 1) ^ ((rl >> 3) & 1);
    c.w_dst[t] = c.wn * kWSlice + q * 1024;
  }
  c.w_pstride = wq_piece_stride(blocked);
  for (int s = 0; s < kStages && s < c.niters; ++s) issue_w(c, s, s);

  // ---- prologue 3: the row table
  if (tid < kXRows) {
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
    slice_row(c.wn, 16 * f + li, ch, rr);
    c.soff[f] = pbase[ch] * 16 + skip[ch] + rr * KB;
  }

  // token fragments: the first ceil(nm/2) go to the waves with mg = 0, the
  // rest to those with mg = 1
  const int nm = (rows + 15) >> 4;
  const int nm0 = (nm + 1) >> 1;
  const int mine = c.mg ? nm - nm0 : nm0;  // wave-uniform
  const int mrow0 = c.mg ? 16 * nm0 : 0;
  if constexpr (!GATEUP) {
    if (c.N - c.n0 <= 3 * 4 * 16) {  // uniform: every slice's valid fragments are its first 3
      if (nm > 8) {
        switch (mine) {
          case 5: unit_main<false, 5, 3, 3>(c, mrow0); break;
          default: unit_main<false, 4, 3, 3>(c, mrow0); break;
        }
      } else if (nm > 4) {
        switch (mine) {
          case 4: unit_main<false, 4, 2, 3>(c, mrow0); break;
          case 3: unit_main<false, 3, 2, 3>(c, mrow0); break;
          default: unit_main<false, 2, 2, 3>(c, mrow0); break;
        }
      } else {
        switch (mine) {
          case 2: unit_main<false, 2, 1, 3>(c, mrow0); break;
          case 1: unit_main<false, 1, 1, 3>(c, mrow0); break;
          default: unit_main<false, 0, 1, 3>(c, mrow0); break;
        }
      }
      return;
    }
  }
  if (nm > 8) {
    switch (mine) {
      case 5: unit_main<GATEUP, 5, 3>(c, mrow0); break;
      default: unit_main<GATEUP, 4, 3>(c, mrow0); break;
    }
  } else if (nm > 4) {
    switch (mine) {
      case 4: unit_main<GATEUP, 4, 2>(c, mrow0); break;
      case 3: unit_main<GATEUP, 3, 2>(c, mrow0); break;
      default: unit_main<GATEUP, 2, 2>(c, mrow0); break;
    }
  } else {
    switch (mine) {
      case 2: unit_main<GATEUP, 2, 1>(c, mrow0); break;
      case 1: unit_main<GATEUP, 1, 1>(c, mrow0); break;
      default: unit_main<GATEUP, 0, 1>(c, mrow0); break;
    }
  }
}

}  // namespace

bool expert_mma_ok(bool gateup, int T, int H, int I, int E, int k, int BM) {
  // large token tiles, the scale slab of K = H (gate/up) or I (down) within
  // its LDS area, and the expected rows per expert large enough that
  // 128-row tiles are mostly full
  const int KB = (gateup ? H : I) / 32;
  return BM == kMT && KB > 0 && slab_pieces(gateup, KB) <= kSlabUnits * kThreads &&
         (long long)T * k >= 32LL * E;
}

void launch_expert_mma(bool gateup, const uint16_t* act, const uint8_t* wq, const uint8_t* ws,
                       const int32_t* sorted_ids, const int32_t* tiles, const int32_t* num_tiles,
                       int tiles_max, int T, int H, int I, int E, int k, bool blocked,
                       void* out, const ExpertAct& fn, hipStream_t stream) {
  const int N = gateup ? I : H;
  const int ncol = 4 * (gateup ? kColsGateUp : kColsDown);
  const int ncb = (N + ncol - 1) / ncol;
  const dim3 grid((unsigned)tiles_max * (unsigned)ncb);
  if (gateup)
    hipLaunchKernelGGL(expert_mma_kernel<true>, grid, dim3(kThreads), kLdsBytes, stream, act, wq, ws,
                       sorted_ids, tiles, num_tiles, T, H, I, E, k, ncb, blocked, out, fn);
  else
    hipLaunchKernelGGL(expert_mma_kernel<false>, grid, dim3(kThreads), kLdsBytes, stream, act, wq, ws,
                       sorted_ids, tiles, num_tiles, T, H, I, E, k, ncb, blocked, out, fn);
}

}  // namespace moe
