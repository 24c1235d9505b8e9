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
// Work split.  A workgroup owns one tile (<= BM slots of one expert) and
// NBW blocks of 16 output rows of the weight matrix (for gate/up: gate rows
// n..n+15 with the matching up rows I+n..I+n+15, so SwiGLU fuses into the
// epilogue).  Each 16-row block is served by 4 waves that split the
// reduction dimension: it is cut into 32-element MX blocks and block
// b = 16*step + 4*kq + group goes to lane group `group` (lanes 16*group ..
// +15) of the block's wave kq.  A lane thus loads exactly one MX block (16
// bytes, 32 codes) plus its scale byte per weight row and step, and a wave
// needs 64 bytes of each of its 16 rows: one contiguous kilobyte in the
// blocked weight layout, 16 separate runs in the canonical one (where the
// one-chunk gate/up kernel loads a faster pattern and regroups it through
// LDS, as described at its loads).  An MFMA sums over its
// whole K range, so the K order is free as long as the activation operand
// uses the same assignment: for MFMA j (0..3) of a step, group g supplies
// elements 32*b + 8*j .. +8 of both operands.
//
// Workgroup (x, y) is column block x of tile y, so the workgroups of one
// tile are dispatched together and stream neighbouring rows of one
// expert's weights; at 64 tokens this measured 6-13% faster than
// dispatching column block by column block across all tiles.
//
// Memory behaviour.  All weight loads of a wave (up to kChunk steps) are
// issued branch-free before the first MFMA (out-of-range blocks read a
// clamped address and get a zero scale), and they stay in registers across
// the tile's M-passes, so each weight byte is fetched once per tile.  The
// activation rows of a pass (XR rows, XR = 1..16) are staged once per
// workgroup in LDS with a 16-byte row pad (conflict-free 128-bit reads; at
// XR = 1 every lane reads the same row, a broadcast).  The split-K partial
// sums meet in LDS in a fixed order, so results are bit-reproducible.
#include "expert_common.h"
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

namespace {

// GATEUP: A rows are x[token of sorted_ids[r]], K = H, weights are the gate
//         and up rows of w13, output h[r][n] = bf16(silu(g) * u).
// !GATEUP: A rows are h[r], K = I, weights are rows of w2, output
//         y[sorted_ids[r]][n] in fp32.
// BLK: the code matrix is in the blocked layout (see wq_row_offset).
// G: passes that share each load of a K chunk's weights (several chunks).
template <bool GATEUP, int NBW, int XR, bool ONECHUNK, bool BLK, int G = 1>
__global__ __launch_bounds__(256 * NBW) void expert_gemm_kernel(
    const uint16_t* __restrict__ act, const uint8_t* __restrict__ wq,
    const uint8_t* __restrict__ ws, const int32_t* sorted_ids,  // not restrict: see below
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ num_tiles, int T, int H,
    int I, int E, int k, void* __restrict__ out, ExpertAct fn) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int NW = GATEUP ? 2 : 1;  // weight rows per lane per step (gate + up)

  // The tile count and the tile's row are read together (one round trip
  // instead of two dependent ones); the row exists for every workgroup, as
  // the grid has one workgroup per possible tile.
  const int tile = blockIdx.y;
  const int ntiles = num_tiles[0];
  const int e = tiles[3 * tile + 0];
  const int r0 = tiles[3 * tile + 1];
  const int rows = tiles[3 * tile + 2];
  asm volatile("" ::"s"(ntiles), "s"(e), "s"(r0), "s"(rows));  // all four loads, one wait
  const long long nslots = (long long)T * k;
  if (tile >= ntiles || !tile_ok(e, r0, rows, E, nslots)) return;  // uniform

  const int K = GATEUP ? H : I;       // reduction length
  const int N = GATEUP ? I : H;       // output rows (row pairs for gate/up)
  const int KB = K / 32;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int li = lane & 15;
  const int grp = lane >> 4;
  const int nb = wave >> 2;           // 16-row block within the workgroup
  const int kq = wave & 3;            // K quarter of this wave
  const int n_base = (blockIdx.x * NBW + nb) * kRowsPerBlock;
  const int n_row = n_base < N ? n_base + li : li;  // blocks past N compute, never store

  // Weight rows this lane loads.  In the blocked layout the MFMA mapping
  // (row li, block 16*step + 4*kq + grp) is one contiguous kilobyte per wave
  // instruction, in lane order.  In the canonical layout it is 16 rows x 64
  // bytes; there the gate/up kernel with one K chunk and one 16-row block
  // per workgroup instead reads 4 rows x 256 contiguous bytes per wave
  // instruction (lane l: row 4*kq + l/16 of the block, MX block
  // 16*step + l%16), which streams from HBM markedly faster, and exchanges
  // each step's pieces through LDS so that every lane holds the MFMA
  // mapping.  The other canonical variants load the mapping directly: for
  // down the exchange's per-step barriers and LDS cost more than the faster
  // stream gains, and with 4 blocks per workgroup its LDS would lower
  // occupancy.
  const size_t q_stride = (size_t)K / 2;
  const size_t s_stride = (size_t)K / 32;
  constexpr bool XCHG = GATEUP && ONECHUNK && NBW == 1 && !BLK;
  const int l_row = XCHG ? (n_base < N ? n_base : 0) + 4 * kq + (lane >> 4) : n_row;
  size_t wrow[NW];
  if (GATEUP) {
    wrow[0] = (size_t)e * 2 * I + l_row;
    if (NW > 1) wrow[NW - 1] = (size_t)e * 2 * I + I + l_row;
  } else {
    wrow[0] = (size_t)e * H + l_row;
  }

  const int nsteps = (KB + kBlocksPerStep - 1) / kBlocksPerStep;
  const int nchunks = ONECHUNK ? 1 : (nsteps + kChunk - 1) / kChunk;
  // Staged activations: the whole of K with one chunk; with several, one
  // chunk's K-range at a time (so a pass can hold 16 rows at any K).
  const int stride = act_stride_bytes(ONECHUNK ? K : min(K, kChunkK));
  const int npass = (rows + XR - 1) / XR;

  uint4 wreg[kChunk][NW];
  uint32_t sreg[kChunk][NW];

  auto load_weights = [&](int ch, int c0 = 0, int c1 = kChunk) {
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
      if (c < c0 || c >= c1) continue;
      const int b = XCHG ? c * kBlocksPerStep + (lane & 15)
                             : (ch * kChunk + c) * kBlocksPerStep + kq * 4 + grp;
      const int bc = min(b, KB - 1);  // clamped: always a valid address
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        wreg[c][w] = *reinterpret_cast<const uint4*>(wq + wq_row_offset(wrow[w], q_stride, BLK) +
                                                     (size_t)bc * wq_piece_stride(BLK));
        if constexpr (!ONECHUNK) sreg[c][w] = ws[wrow[w] * s_stride + bc];
      }
    }
  };

  // ONECHUNK: the workgroup's scale runs (run nb*NW + w: rows of block nb,
  // half w; KB pieces of 16 bytes each), piece `tid` of the concatenation
  // per thread, loaded with the weight stream and written to LDS after it
  // has landed
  constexpr int kRuns = ONECHUNK ? NBW * NW : 1;
  static_assert(!ONECHUNK || kRuns * kChunk * kBlocksPerStep <= 256 * NBW,
                "one scale piece per thread");
  __shared__ __align__(16) unsigned char s_sc[ONECHUNK ? NBW * NW * kScaleRunMax : 16];

  // XCHG: LDS slots through which one step of the workgroup's weights is
  // exchanged between its 4 waves: [slot][half][row][16 pieces of 16
  // bytes], piece p of row r stored at position p ^ r so that both the
  // row-wise writes and the column-wise reads spread over all banks.  With
  // one staged token, two slots let step c+1 be written while step c is
  // read; with more, one slot (and a second barrier per step) keeps the
  // LDS footprint low enough for as many workgroups per CU as the
  // registers allow, which measured faster.
  constexpr int kRing = XR == 1 ? 2 : 1;
  constexpr int kSlotBytes = NW * NBW * kRowsPerBlock * 256;
  __shared__ __align__(16) unsigned char s_ring[XCHG ? kRing * kSlotBytes : 16];
  uint4 spiece = uint4{0u, 0u, 0u, 0u};
  const int pr = min(tid / KB, kRuns - 1);  // this thread's run and piece
  const int pp = tid - pr * KB;
  const bool has_piece = tid < kRuns * KB;
  auto load_scale_runs = [&]() {
    const int rb = pr / NW, rw = pr % NW;
    const int nb0 = (blockIdx.x * NBW + rb) * kRowsPerBlock;
    const int row0 = nb0 < N ? nb0 : 0;  // blocks past N read block 0's rows
    const size_t grow0 = GATEUP ? (size_t)e * 2 * I + (size_t)rw * I + row0
                                : (size_t)e * H + row0;
    const int piece = min(pp, KB - 1);  // threads past the runs repeat a piece
    spiece = *reinterpret_cast<const uint4*>(ws + grow0 * s_stride + (size_t)piece * 16);
  };
  auto store_scale_runs = [&]() {
    if (has_piece)
      *reinterpret_cast<uint4*>(s_sc + pr * kScaleRunMax + pp * 16) = spiece;
  };

  // Per-tile row table in LDS: the element offset of each row's activations
  // and (down) the slot id its output goes to.  The index loads are issued
  // before the weight stream so they never wait behind it.
  __shared__ long long s_rowoff[kMaxRows];
  __shared__ int s_slot[kMaxRows];
  // Branch-free and in bounds.  The memory clobber keeps this load ahead of
  // the weight stream (sorted_ids is deliberately not __restrict__, which
  // would let the compiler sink the load past the clobber).
  const int my_slot = sorted_ids[r0 + min(tid, rows - 1)];
  asm volatile("" ::: "memory");

  // Stage activation rows [p0, p0 + nrows) of this tile into LDS with
  // direct global->LDS 128-bit loads (no registers hold the data).  The
  // padded rows form one array of 16-byte slots, K/8 + 1 per row (the last is
  // the pad, filled with a copy of the row's last chunk); one wave
  // instruction fills 64 consecutive slots = 1 KB.  Slots past the last row
  // repeat it; the LDS allocation is rounded up to whole kilobytes.
  constexpr int kWavesWG = 4 * NBW;
  // (Elements [k0, k0 + klen) of each row; rows then sit klen*2 + 16 bytes
  // apart.)
  auto stage_acts = [&](int p0, int nrows, int k0, int klen) {
    const int cpr = klen / 8;
    const int spr = cpr + 1;
    const int ninst = (nrows * spr + 63) / 64;
    for (int ins = wave; ins < ninst; ins += kWavesWG) {  // wave-uniform
      const int slot = ins * 64 + lane;
      const int r = min(slot / spr, nrows - 1);
      const int c = min(slot - (slot / spr) * spr, cpr - 1);
      __builtin_amdgcn_global_load_lds(
          act + s_rowoff[p0 + r] + (long long)(k0 + c * 8),
          (__attribute__((address_space(3))) void*)(smem + (size_t)ins * 1024), 16, 0, 0);
    }
  };

  // With one K chunk and activation rows that do not depend on the slot ids
  // (down, or a single token), the activations and the scale piece are
  // issued ahead of the weights and waited for alone; each step's MFMAs then
  // start as soon as that step's weights land.  Otherwise the weights go
  // first and everything is waited for at once.
  const bool early = ONECHUNK && (!GATEUP || T == 1);  // uniform
  if (early) {
    if (tid < rows) s_rowoff[tid] = GATEUP ? 0LL : (long long)(r0 + tid) * I;
    lds_barrier();
    stage_acts(0, min(XR, rows), 0, K);
    load_scale_runs();
    asm volatile("" ::: "memory");  // the weight loads stay behind
    load_weights(0);
    wait_vmcnt<kChunk * NW>();      // all but the weight loads
  } else {
    // SPLIT (several 16-row blocks per workgroup, which then runs alone on
    // its CU): the first half of the steps' weights and the scale piece go
    // first, the second half after the activation staging, so the wait below
    // leaves it in flight while the first steps' MFMAs run (20b T = 64
    // gate/up 62.4 -> 58.9 us; with one block per workgroup other
    // workgroups already fill that gap and the split measured slower)
    constexpr bool SPLIT = ONECHUNK && NBW > 1;
    if constexpr (ONECHUNK) {  // depends only on the tile row
      load_weights(0, 0, SPLIT ? kChunk / 2 : kChunk);
      load_scale_runs();
    }
    // Row offsets: for down they are the tile's own rows of h, and with one
    // token every gate/up row is token 0, so neither waits for the slot ids
    // (which queue behind the weight stream).
    if (tid < rows) {
      long long off;
      if (GATEUP) {
        const int t = T == 1 ? 0 : min(max(my_slot / k, 0), T - 1);
        off = (long long)t * H;
      } else {
        off = (long long)(r0 + tid) * I;
      }
      s_rowoff[tid] = off;
    }
    // LDS-only barrier: __syncthreads would also wait for the whole weight
    // stream issued above, and the activation staging below would no longer
    // overlap it (the slot-id load was issued first, so using it waited only
    // for that load)
    lds_barrier();
    // Pass 0's activations are staged while the weight stream is in flight;
    // one wait covers both.  (With several chunks each chunk stages its own.)
    if constexpr (ONECHUNK) stage_acts(0, min(XR, rows), 0, K);
    if constexpr (SPLIT) {
      asm volatile("" ::: "memory");  // the second half stays behind the staging
      load_weights(0, kChunk / 2, kChunk);
      wait_vmcnt<(kChunk - kChunk / 2) * NW>();
    } else {
      __builtin_amdgcn_s_waitcnt(0);
    }
  }
  if constexpr (ONECHUNK) store_scale_runs();
  if (tid < rows) s_slot[tid] = my_slot;
  lds_barrier();  // this wave's staging loads have landed (waited above)

  // With several K chunks a lane holds one chunk of weights at a time, so
  // G passes share each load of a chunk (their accumulators stay in
  // registers across the chunks) instead of every pass fetching all of K
  // again.  Each pass still accumulates its chunks and steps in order, so
  // the results do not depend on G.
  static_assert(G == 1 || !ONECHUNK, "pass groups only with several chunks");
  for (int g0 = 0; g0 < npass; g0 += G) {
    if (ONECHUNK && g0 > 0) {
      __syncthreads();  // previous pass done with LDS
      stage_acts(g0 * XR, min(XR, rows - g0 * XR), 0, K);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }

    if constexpr (ONECHUNK) {
      // scale bytes of this lane's rows from the table
#pragma unroll
      for (int c = 0; c < kChunk; ++c) {
        const int bc = min(c * kBlocksPerStep + kq * 4 + grp, KB - 1);
#pragma unroll
        for (int w = 0; w < NW; ++w) sreg[c][w] = s_sc[(nb * NW + w) * kScaleRunMax + li * KB + bc];
      }
    }
    floatx4 acc[G][NW];
#pragma unroll
    for (int pg = 0; pg < G; ++pg)
#pragma unroll
      for (int w = 0; w < NW; ++w) acc[pg][w] = floatx4{0.f, 0.f, 0.f, 0.f};
    const unsigned char* arow = smem + min(li, min(XR, rows - g0 * XR) - 1) * stride;
    int chunk_kb = KB;  // MX blocks of the staged K-range

    for (int ch = 0; ch < nchunks; ++ch) {
#pragma unroll
      for (int pg = 0; pg < G; ++pg) {
        const int pass = g0 + pg;
        if (pass >= npass) break;  // uniform
        if constexpr (!ONECHUNK) {
          const int p0 = pass * XR;
          const int prow = min(XR, rows - p0);
          const int k0 = ch * kChunkK, klen = min(K - k0, kChunkK);
          if (g0 > 0 || ch > 0 || pg > 0) __syncthreads();  // every wave done with the LDS
          if (pg == 0) load_weights(ch);
          stage_acts(p0, prow, k0, klen);
          __builtin_amdgcn_s_waitcnt(0);
          __syncthreads();
          arow = smem + min(li, prow - 1) * act_stride_bytes(klen);
          chunk_kb = klen / 32;
        }
#pragma unroll
        for (int c = 0; c < kChunk; ++c) {
          if (XCHG && pass == 0) {  // uniform: exchange step c's pieces
            unsigned char* slot = s_ring + (c % kRing) * kSlotBytes;
            if (kRing == 1 && c > 0) lds_barrier();  // every wave done reading step c-1
            const int wr16 = 4 * kq + (lane >> 4);
#pragma unroll
            for (int w = 0; w < NW; ++w)
              *reinterpret_cast<uint4*>(slot + ((w * NBW + nb) * kRowsPerBlock + wr16) * 256 +
                                        (((lane & 15) ^ wr16) << 4)) = wreg[c][w];
            lds_barrier();
#pragma unroll
            for (int w = 0; w < NW; ++w)
              wreg[c][w] = *reinterpret_cast<const uint4*>(
                  slot + ((w * NBW + nb) * kRowsPerBlock + li) * 256 + (((4 * kq + grp) ^ li) << 4));
          }
          // Step c's weights are decoded here and no earlier: an empty asm that
          // "modifies" them stops the compiler from hoisting the decode (which
          // would quadruple their register footprint) and makes this step wait
          // for its own loads only.
#pragma unroll
          for (int w = 0; w < NW; ++w)
            asm volatile("" : "+v"(wreg[c][w].x), "+v"(wreg[c][w].y), "+v"(wreg[c][w].z),
                         "+v"(wreg[c][w].w), "+v"(sreg[c][w]));
          const int b = (ch * kChunk + c) * kBlocksPerStep + kq * 4 + grp;
          const bool valid = b < KB;
          // block within the staged K-range (the whole of K with one chunk)
          const int bl = min(c * kBlocksPerStep + kq * 4 + grp, chunk_kb - 1);
          float scale[NW];
#pragma unroll
          for (int w = 0; w < NW; ++w) scale[w] = valid ? e8m0_to_float(sreg[c][w]) : 0.f;
          const uint4* ap = reinterpret_cast<const uint4*>(arow + bl * 64);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bf16x8 a = as_bf16x8(ap[j]);
#pragma unroll
            for (int w = 0; w < NW; ++w)
              acc[pg][w] = mfma16x16x32(a, dequant8_bf16(word(wreg[c][w], j), scale[w]), acc[pg][w]);
          }
        }
      }
    }

#pragma unroll
    for (int pg = 0; pg < G; ++pg) {
      const int pass = g0 + pg;
      if (pass >= npass) break;  // uniform
      const int p0 = pass * XR;
      const int prow = min(XR, rows - p0);
      // split-K reduction: waves kq = 0..3 of each 16-row block, fixed order
      __syncthreads();  // every wave done reading the staged activations
      float* red = reinterpret_cast<float*>(smem);  // [NBW][4][NW][256]
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          red[((nb * 4 + kq) * NW + w) * 256 + (4 * grp + r) * kRowsPerBlock + li] = acc[pg][w][r];
      __syncthreads();
      {
        const int obl = tid >> 8;       // output block handled by this thread
        const int idx = tid & 255;      // 16 tokens x 16 rows
        const int tm = idx / kRowsPerBlock;
        const int tn = idx % kRowsPerBlock;
        const int on = (blockIdx.x * NBW + obl) * kRowsPerBlock + tn;
        float v[NW];
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          v[w] = red[((obl * 4 + 0) * NW + w) * 256 + idx];
#pragma unroll
          for (int q = 1; q < 4; ++q) v[w] += red[((obl * 4 + q) * NW + w) * 256 + idx];
        }
        if (tm < prow && on < N) {
          const int r = r0 + p0 + tm;
          if (GATEUP) {
            float hv;
            if (fn.kind == 0) {
              hv = silu(v[0]) * v[NW - 1];
            } else {
              const float bg = fn.b13 ? fn.b13[(size_t)e * 2 * I + on] : 0.f;
              const float bu = fn.b13 ? fn.b13[(size_t)e * 2 * I + I + on] : 0.f;
              hv = act_gptoss(v[0] + bg, v[NW - 1] + bu, fn.alpha, fn.limit);
            }
            reinterpret_cast<uint16_t*>(out)[(size_t)r * I + on] = float_to_bf16(hv);
          } else {
            const long long p = s_slot[p0 + tm];
            const float yv = fn.kind != 0 && fn.b2 ? v[0] + fn.b2[(size_t)e * H + on] : v[0];
            if (p >= 0 && p < nslots) reinterpret_cast<float*>(out)[(size_t)p * H + on] = yv;
          }
        }
      }
    }
  }
}

// Down GEMM and combine of a single token in one launch (T = 1, k <= 4).
// Workgroup n owns output rows 16n .. 16n+15 of w2 for all k tiles at once:
// waves 4g .. 4g+3 are tile g's split-K group and run exactly the arithmetic
// of expert_gemm_kernel<false, 1, 1, true> for that tile (same blocks per
// lane, same MFMA order, same fixed-order split-K sum), so each slot's y
// value is bit-identical to the unfused down GEMM's; the k values then meet
// in LDS and are combined as combine_kernel does (fp32 fma in ascending slot
// order, one bf16 rounding).  No y buffer and no extra launch.
constexpr int kFuseMaxK = 4;
__host__ __device__ __forceinline__ int fuse_row_region(int K) {
  return (act_stride_bytes(K) + 1023) / 1024 * 1024;
}

__global__ __launch_bounds__(256 * kFuseMaxK) void down_combine_one_token_kernel(
    const uint16_t* __restrict__ h, const uint8_t* __restrict__ wq,
    const uint8_t* __restrict__ ws, const int32_t* sorted_ids,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ num_tiles,
    const float* __restrict__ topk_weights, int H, int I, int E, int k, bool blocked,
    uint16_t* __restrict__ out, ExpertAct fn) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int li = lane & 15;
  const int grp = lane >> 4;
  const int g = wave >> 2;   // tile (slot group) of this wave
  const int kq = wave & 3;   // K quarter
  const int K = I, KB = K / 32;
  const int n_row = blockIdx.x * kRowsPerBlock + li;  // grid covers H / 16 blocks exactly

  // every tile row in one round trip; a tile outside the table (g >= count)
  // or malformed computes nothing and contributes nothing
  const int ntiles = num_tiles[0];
  const int gt = min(g, k - 1);
  const int e = tiles[3 * gt + 0];
  const int r0 = tiles[3 * gt + 1];
  const int rows = tiles[3 * gt + 2];
  asm volatile("" ::"s"(ntiles), "s"(e), "s"(r0), "s"(rows));
  const bool live = g < k && g < ntiles && tile_ok(e, r0, rows, E, k) && rows == 1;  // uniform per wave
  const int slot = live ? sorted_ids[r0] : -1;

  // LDS: tile g's staged h row (I bf16 + 16-byte pad, in a region rounded
  // up to whole kilobytes: the last load instruction's surplus slots land
  // there) | its scale run (16 rows x KB bytes) | the split-K table
  const int region = fuse_row_region(K);
  unsigned char* arow = smem + g * region;
  unsigned char* s_sc = smem + kFuseMaxK * region + g * kScaleRunMax;
  float* red = reinterpret_cast<float*>(smem + kFuseMaxK * (region + kScaleRunMax));
  __shared__ int s_slot[kFuseMaxK];
  __shared__ int s_exp[kFuseMaxK];

  uint4 wreg[kChunk];
  uint32_t sreg[kChunk];
  if (live) {
    // activations first (row r0 of h, one 16-byte slot per lane of the group,
    // the pad slot repeating the last chunk), then the scale run, then the
    // weights, so that each step waits for its own weights only
    const int cpr = K / 8, spr = cpr + 1;
    const int gl = tid & 255;
    for (int ins = kq; ins < (spr + 63) / 64; ins += 4) {  // wave-uniform
      const int sl = ins * 64 + lane;
      const int c = min(sl, cpr - 1);
      __builtin_amdgcn_global_load_lds(
          h + (size_t)r0 * I + (size_t)c * 8,
          (__attribute__((address_space(3))) void*)(arow + (size_t)ins * 1024), 16, 0, 0);
    }
    const size_t grow0 = (size_t)e * H + (size_t)blockIdx.x * kRowsPerBlock;
    const int piece = min(gl, KB - 1);
    const uint4 sp = *reinterpret_cast<const uint4*>(ws + grow0 * KB + (size_t)piece * 16);
    asm volatile("" ::: "memory");
    const size_t wrow = (size_t)e * H + n_row;
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
      const int bc = min(c * kBlocksPerStep + kq * 4 + grp, KB - 1);
      wreg[c] = *reinterpret_cast<const uint4*>(wq + wq_row_offset(wrow, K / 2, blocked) +
                                                (size_t)bc * wq_piece_stride(blocked));
    }
    wait_vmcnt<kChunk>();  // activations and the scale piece
    if (gl < KB) *reinterpret_cast<uint4*>(s_sc + gl * 16) = sp;
  }
  if (tid < kFuseMaxK) s_slot[tid] = -1;
  lds_barrier();
  if (live && kq == 0 && lane == 0) {
    s_slot[g] = slot;
    s_exp[g] = e;
  }

  floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
  if (live) {
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
      const int bc = min(c * kBlocksPerStep + kq * 4 + grp, KB - 1);
      sreg[c] = s_sc[li * KB + bc];
    }
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
      asm volatile("" : "+v"(wreg[c].x), "+v"(wreg[c].y), "+v"(wreg[c].z), "+v"(wreg[c].w),
                   "+v"(sreg[c]));
      const int b = c * kBlocksPerStep + kq * 4 + grp;
      const int bc = min(b, KB - 1);
      const float scale = b < KB ? e8m0_to_float(sreg[c]) : 0.f;
      const uint4* ap = reinterpret_cast<const uint4*>(arow + bc * 64);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc = mfma16x16x32(as_bf16x8(ap[j]), dequant8_bf16(word(wreg[c], j), scale), acc);
    }
  }
  // split-K table: row 0 (the token) of each group's 16x16 result
  if (live && grp == 0) red[(g * 4 + kq) * 16 + li] = acc[0];
  __syncthreads();
  if (tid < kRowsPerBlock) {
    // y of slot j = fixed-order sum over the K quarters of its tile's table
    float y[kFuseMaxK];
#pragma unroll
    for (int gg = 0; gg < kFuseMaxK; ++gg) {
      float v = red[(gg * 4 + 0) * 16 + tid];
#pragma unroll
      for (int q = 1; q < 4; ++q) v += red[(gg * 4 + q) * 16 + tid];
      if (fn.kind != 0 && fn.b2 && s_slot[gg] >= 0)
        v += fn.b2[(size_t)s_exp[gg] * H + blockIdx.x * kRowsPerBlock + tid];
      y[gg] = v;
    }
    float a = 0.f;
    for (int j = 0; j < k; ++j) {
      float yj = 0.f;
#pragma unroll
      for (int gg = 0; gg < kFuseMaxK; ++gg)
        if (s_slot[gg] == j) yj = y[gg];
      a = fmaf(topk_weights[j], yj, a);
    }
    out[blockIdx.x * kRowsPerBlock + tid] = float_to_bf16(a);
  }
}

// Rows of activations staged per pass, by the mean rows per expert
// m = T*k/E: 4 below m = 2, 8 below m = 8, else 16 (with 16-row blocks per
// workgroup: 1, 2 and 4 respectively; the one-chunk down kernel takes 12
// rows and 3 blocks in place of 16 and 4, see the launcher); bounded by the
// tile's row bound (an expert gets at most one slot per token, so rows <=
// min(BM, T), rounded up to a power of two) and small enough that the
// staged rows fit in 96 KB (whole-K rows) or 100 KB (one chunk's K-range per
// row when K > 3072, so 16 rows fit).  Measured on MI355X over decode
// shapes from 2 to 128 tokens (gpt-oss-20b and -120b, Mixtral- and
// DeepSeek-shaped): 8-row passes in 8-wave workgroups gained 5-30% over
// 4-row or 16-row passes wherever m is between 2 and 8 (DeepSeek-shaped
// T = 128 gate/up 1,163 -> 983 us, down 612 -> 453 us; gpt-oss-120b T = 64
// gate/up 166 -> 160 us), and 16-row passes in 16-wave workgroups stayed
// best from m = 8 (gpt-oss-20b T = 64 under its biased router,
// Mixtral-shaped T = 128).  Smaller passes keep the LDS footprint low enough
// for several workgroups per CU (one's loads overlap another's compute);
// tiles with more rows take extra passes over weights held in registers.
int pick_xr(int T, int BM, int K, int E, int k) {
  const long long tk = (long long)T * k;
  int xr = tk < 2LL * E ? 4 : tk < 8LL * E ? 8 : 16;
  const int cap = T < BM ? T : BM;
  int c2 = 1;
  while (c2 < cap && c2 < 16) c2 <<= 1;
  if (xr > c2) xr = c2;
  const bool one_chunk = K <= kChunkK;
  const size_t row_bytes = act_stride_bytes(one_chunk ? K : kChunkK);
  const size_t budget = (one_chunk ? 96 : 100) * 1024;
  while (xr > 1 && (size_t)xr * row_bytes > budget) xr >>= 1;
  return xr;
}

template <bool GATEUP, bool BLK>
void launch_expert_gemm(const uint16_t* act, const uint8_t* wq, const uint8_t* ws,
                        const int32_t* sorted_ids, const int32_t* tiles,
                        const int32_t* num_tiles, int tiles_max, int T, int H, int I, int E,
                        int k, int BM, void* out, const ExpertAct& fn, hipStream_t stream) {
  const int K = GATEUP ? H : I;
  const int N = GATEUP ? I : H;
  const int xr = pick_xr(T, BM, K, E, k);
  const int nblk16 = N / kRowsPerBlock;
  const bool one_chunk = K <= kChunk * kBlocksPerStep * 32;
  const size_t red_bytes_1 = (size_t)4 * (GATEUP ? 2 : 1) * 256 * sizeof(float);
  // several chunks and more expected rows per expert than one pass holds:
  // two passes share each chunk's weights (with one pass expected, the
  // larger register footprint only costs)
  const bool group2 = (long long)T * k > (long long)xr * E;
#define MOE_LAUNCH(NBW_, XR_)                                                                  \
  do {                                                                                          \
    size_t lds = ((size_t)(XR_) * act_stride_bytes(one_chunk ? K : kChunkK) + 1023) / 1024 * 1024; \
    if (lds < red_bytes_1 * (NBW_)) lds = red_bytes_1 * (NBW_);                                 \
    dim3 grid((nblk16 + (NBW_) - 1) / (NBW_), tiles_max);                                       \
    if (one_chunk)                                                                              \
      hipLaunchKernelGGL((expert_gemm_kernel<GATEUP, NBW_, XR_, true, BLK>), grid, dim3(256 * (NBW_)), \
                         lds, stream, act, wq, ws, sorted_ids, tiles, num_tiles, T, H, I, E, k,  \
                         out, fn);                                                              \
    else if (group2)                                                                            \
      hipLaunchKernelGGL((expert_gemm_kernel<GATEUP, NBW_, XR_, false, BLK, 2>), grid,          \
                         dim3(256 * (NBW_)), lds, stream, act, wq, ws, sorted_ids, tiles,       \
                         num_tiles, T, H, I, E, k, out, fn);                                    \
    else                                                                                        \
      hipLaunchKernelGGL((expert_gemm_kernel<GATEUP, NBW_, XR_, false, BLK, 1>), grid,          \
                         dim3(256 * (NBW_)), lds, stream, act, wq, ws, sorted_ids, tiles,       \
                         num_tiles, T, H, I, E, k, out, fn);                                    \
  } while (0)
  switch (xr) {
    case 1: MOE_LAUNCH(1, 1); break;
    case 2: MOE_LAUNCH(1, 2); break;
    case 4: MOE_LAUNCH(1, 4); break;
    case 8: MOE_LAUNCH(2, 8); break;
    default:
      // down with one K chunk: three blocks and 12-row passes, so that two
      // 768-thread workgroups fit on a CU (registers and LDS) and one's
      // weight stream overlaps the other's compute; bit-identical, and at
      // 20b T = 64 under its biased router down 36.9 -> 35.2 us (gpt-oss-120b
      // T = 512: layer 497 -> 490 us), where 4 x 8 (registers spill at 64),
      // 2 x 8, 2 x 12, 2 x 16, 3 x 8, 3 x 10, 3 x 16 and 4 x 12 measured
      // slower; gate/up (124 registers) keeps 4 x 16
      if (!GATEUP && one_chunk)
        MOE_LAUNCH(3, 12);
      else
        MOE_LAUNCH(4, 16);
      break;
  }
#undef MOE_LAUNCH
}

}  // namespace

void launch_gateup_swiglu(const uint16_t* x, const uint8_t* w13_q, const uint8_t* w13_s,
                          const int32_t* sorted_ids, const int32_t* tiles,
                          const int32_t* num_tiles, int tiles_max, int T, int H, int I, int E,
                          int k, int BM, bool blocked, uint16_t* h, const ExpertAct& fn,
                          hipStream_t stream) {
  if (expert_mma_ok(true, T, H, I, E, k, BM)) {
    launch_expert_mma(true, x, w13_q, w13_s, sorted_ids, tiles, num_tiles, tiles_max, T, H, I, E,
                      k, blocked, h, fn, stream);
    return;
  }
  if (blocked)
    launch_expert_gemm<true, true>(x, w13_q, w13_s, sorted_ids, tiles, num_tiles, tiles_max, T,
                                   H, I, E, k, BM, h, fn, stream);
  else
    launch_expert_gemm<true, false>(x, w13_q, w13_s, sorted_ids, tiles, num_tiles, tiles_max, T,
                                    H, I, E, k, BM, h, fn, stream);
}

bool down_combine_one_token_ok(int T, int H, int I, int k) {
  return T == 1 && k <= kFuseMaxK && I <= kChunk * kBlocksPerStep * 32 && H % kRowsPerBlock == 0;
}

void launch_down_combine_one_token(const uint16_t* h, const uint8_t* w2_q, const uint8_t* w2_s,
                                   const int32_t* sorted_ids, const int32_t* tiles,
                                   const int32_t* num_tiles, const float* topk_weights, int H,
                                   int I, int E, int k, bool blocked, uint16_t* out,
                                   const ExpertAct& fn, hipStream_t stream) {
  const size_t red_bytes = (size_t)kFuseMaxK * 4 * 16 * sizeof(float);
  const size_t lds = (size_t)kFuseMaxK * (fuse_row_region(I) + kScaleRunMax) + red_bytes;
  hipLaunchKernelGGL(down_combine_one_token_kernel, dim3(H / kRowsPerBlock),
                     dim3(256 * kFuseMaxK), lds, stream, h, w2_q, w2_s, sorted_ids, tiles,
                     num_tiles, topk_weights, H, I, E, k, blocked, out, fn);
}

void launch_down(const uint16_t* h, const uint8_t* w2_q, const uint8_t* w2_s,
                 const int32_t* sorted_ids, const int32_t* tiles, const int32_t* num_tiles,
                 int tiles_max, int T, int H, int I, int E, int k, int BM, bool blocked,
                 float* y, const ExpertAct& fn, hipStream_t stream) {
  if (expert_mma_ok(false, T, H, I, E, k, BM)) {
    launch_expert_mma(false, h, w2_q, w2_s, sorted_ids, tiles, num_tiles, tiles_max, T, H, I, E,
                      k, blocked, y, fn, stream);
    return;
  }
  if (blocked)
    launch_expert_gemm<false, true>(h, w2_q, w2_s, sorted_ids, tiles, num_tiles, tiles_max, T, H,
                                    I, E, k, BM, y, fn, stream);
  else
    launch_expert_gemm<false, false>(h, w2_q, w2_s, sorted_ids, tiles, num_tiles, tiles_max, T,
                                     H, I, E, k, BM, y, fn, stream);
}

}  // namespace moe
