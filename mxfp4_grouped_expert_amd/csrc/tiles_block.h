// Block-level builder of the per-expert tile table (shared by the standalone
// tile kernel and the fused decode router).
//
// The SimpleLLM write-up ("A 297-line kernel file that decodes faster than
// vLLM", section "Optimizations", "Per-expert routing tile table") has each
// expert write its own tiles instead of the expert GEMM searching a
// tiles x experts grid.  One workgroup of NT threads does it in LDS, with no
// order-dependent atomics, so the result is bit-exact and deterministic:
//   1. each wave counts the slots of its own contiguous range per expert
//      (LDS integer adds: totals do not depend on order); ids outside
//      [0, E) go to a trash bucket E;
//   2. exclusive scans of the counts (row offsets, and per expert over the
//      waves in order) and of ceil(count/BM) (tile offsets);
//   3. stable scatter: each wave walks its range in rounds of 64 slots;
//      lanes with the same expert find each other with nine ballots (one
//      per bit of the bucket index) and rank themselves with mbcnt, after
//      the wave's own running position in that expert;
//   4. each tile index finds its expert by binary search over the tile
//      offsets and writes (expert, row_start, rows).
// Many slots (a prefill) split over several workgroups, each scattering one
// contiguous range of slots: a workgroup also counts the slots before and
// after its range per expert (order-free LDS adds over the ids, read from
// L2), so it knows every expert's offset and its own first position in each
// expert without hearing from the others, and the result is the same table.
#pragma once

#include "moe_device.h"

namespace moe {

constexpr int kBuckets = kMaxExperts + 1;  // experts + trash bucket

template <int NT>
struct TilesScratch {
  int cnt[kBuckets];
  int ntile[kBuckets];
  int off[kBuckets + 1];
  int toff[kBuckets + 1];
  int run[kBuckets];
  int wcnt[NT / kWave][kBuckets];
};

// Exclusive scan of n <= 320 ints by one wave (5 per lane); writes out[0..n]
// with out[n] = total.
__device__ inline void wave_exclusive_scan(const int* in, int* out, int n, int lane) {
  const int base = lane * 5;
  int loc[5];
  int sum = 0;
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    loc[j] = (base + j < n) ? in[base + j] : 0;
    sum += loc[j];
  }
  int incl = sum;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  int run = incl - sum;
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    if (base + j < n) out[base + j] = run;
    run += loc[j];
  }
  if (lane == kWave - 1) out[n] = incl;
}

// The part of the slots [0, N) one workgroup scatters: [q0, q1).  With
// q0 > 0 or q1 < N, `before` and `after` are LDS arrays of kBuckets ints
// for the counts outside the range; only the workgroup with `writer` set
// stores expert_offsets, the tiles and num_tiles (identical in every one).
struct TilesRange {
  int q0, q1;
  int* before;
  int* after;
  bool writer;
};

// Builds the table from ids[0..N) (any address space).  Every thread of the
// NT-thread workgroup must call it; it ends with a barrier.  Phases exchange
// data through LDS only, so the barriers do not wait for global stores.
//
// Wave w owns the contiguous slot range [w*L, (w+1)*L): it counts its slots
// per bucket (LDS integer adds), an exclusive scan over (bucket, wave) in
// bucket-major order gives every wave its first position in each bucket, and
// the wave then scatters its range in rounds of 64 slots, ranking equal
// buckets within a round by ballots and advancing its own per-bucket cursor.
// Only the wave touches its cursors, so the scatter needs no workgroup
// barrier, and slot order inside a bucket stays ascending.
template <int NT, typename IdPtr>
__device__ void build_tiles_block(IdPtr ids, int N, int E, int BM, TilesScratch<NT>& S,
                                  int32_t* __restrict__ expert_offsets,
                                  int32_t* __restrict__ sorted_ids, int32_t* __restrict__ tiles,
                                  int32_t* __restrict__ num_tiles,
                                  TilesRange R = TilesRange{0, -1, nullptr, nullptr, true}) {
  constexpr int kW = NT / kWave;
  static_assert(kW >= 2, "needs two waves for the scans");
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int NB = E + 1;  // buckets in use
  const int q0 = R.q0, q1 = R.q1 < 0 ? N : R.q1;
  const bool split = q0 > 0 || q1 < N;  // uniform
  const int L = ((q1 - q0 + kW - 1) / kW + kWave - 1) / kWave * kWave;  // slots per wave
  const int p0 = q0 + wave * L;
  const int p1 = min(q1, p0 + L);
  auto bucket = [&](int p) {
    const int e = ids[p];
    return (e < 0 || e >= E) ? E : e;
  };

  for (int i = tid; i < kW * NB; i += NT) S.wcnt[i / NB][i % NB] = 0;
  if (split)
    for (int i = tid; i < NB; i += NT) R.before[i] = R.after[i] = 0;
  lds_barrier();
#pragma unroll 8
  for (int p = p0 + lane; p < p1; p += kWave) atomicAdd(&S.wcnt[wave][bucket(p)], 1);
  if (split) {
#pragma unroll 8
    for (int p = tid; p < q0; p += NT) atomicAdd(&R.before[bucket(p)], 1);
#pragma unroll 8
    for (int p = q1 + tid; p < N; p += NT) atomicAdd(&R.after[bucket(p)], 1);
  }
  lds_barrier();
  // per bucket: total, and each wave's first position relative to the
  // bucket (the slots before the range, then an exclusive scan over the
  // waves, in wave order)
  for (int i = tid; i < NB; i += NT) {
    int run = split ? R.before[i] : 0;
    for (int w = 0; w < kW; ++w) {
      const int c = S.wcnt[w][i];
      S.wcnt[w][i] = run;
      run += c;
    }
    if (split) run += R.after[i];
    S.cnt[i] = run;
    S.ntile[i] = (i < E) ? (run + BM - 1) / BM : 0;
  }
  lds_barrier();
  if (wave == 0) wave_exclusive_scan(S.cnt, S.off, NB, lane);
  if (wave == 1) wave_exclusive_scan(S.ntile, S.toff, NB, lane);
  lds_barrier();
  if (R.writer)
    for (int i = tid; i <= E; i += NT) expert_offsets[i] = S.off[i];

  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  constexpr int kBatch = 8;  // rounds whose ids are loaded together
  for (int c1 = p0; c1 < p1; c1 += kBatch * kWave) {  // wave-uniform
    int eb[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int p = c1 + j * kWave + lane;
      eb[j] = p < p1 ? bucket(p) : 0;
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int c0 = c1 + j * kWave;
      if (c0 >= p1) break;  // wave-uniform
      const int p = c0 + lane;
      const bool valid = p < p1;
      const int e = eb[j];
      uint64_t same = __ballot(valid);
#pragma unroll
      for (int bit = 0; bit < 9; ++bit) {
        const bool b = (e >> bit) & 1;
        const uint64_t bal = __ballot(b);
        same &= b ? bal : ~bal;
      }
      const int rank = lanes_below(same);
      int cur = 0;
      if (valid) {
        cur = S.wcnt[wave][e];
        sorted_ids[S.off[e] + cur + rank] = p;
      }
      // the group's last lane moves the wave's cursor past the group (read
      // above, written here, read again next round: one wave, in order)
      if (valid && (same & ~lt_mask & ~(1ull << lane)) == 0) S.wcnt[wave][e] = cur + rank + 1;
    }
  }

  const int total = R.writer ? S.toff[E] : 0;
  for (int i = tid; i < total; i += NT) {
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (S.toff[mid] <= i) lo = mid; else hi = mid - 1;
    }
    const int j = i - S.toff[lo];
    tiles[3 * i + 0] = lo;
    tiles[3 * i + 1] = S.off[lo] + j * BM;
    tiles[3 * i + 2] = min(BM, S.cnt[lo] - j * BM);
  }
  if (tid == 0 && R.writer) num_tiles[0] = total;
  lds_barrier();
}

// The same table for small slot counts (N <= NT slots, e.g. a decode batch)
// with the ids already in LDS, in all-pairs form: every quantity is an
// independent count over LDS, so the table takes two barriers and no scans.
//   slot p:    position = #{q : (b_q, q) < (b_p, p)}, b = bucket of the id
//              (ids outside [0, E) go to bucket E), so sorted_ids is the
//              stable counting sort of build_tiles_block;
//   expert e:  offset = #{q : b_q < e}, count = #{q : b_q = e};
//   expert e:  tile offset = sum over e' < e of ceil(count_e' / BM).
// Results are identical to build_tiles_block.  Every thread of the
// NT-thread workgroup must call it (NT > E); it ends with a barrier.
template <int NT>
__device__ void build_tiles_small(const int* ids, int N, int E, int BM, TilesScratch<NT>& S,
                                  int32_t* __restrict__ expert_offsets,
                                  int32_t* __restrict__ sorted_ids, int32_t* __restrict__ tiles,
                                  int32_t* __restrict__ num_tiles) {
  static_assert(NT > kMaxExperts, "one thread per bucket");
  const int tid = threadIdx.x;
  int* bk = &S.wcnt[0][0];  // bucket of each slot (N <= NT <= NT/64 * kBuckets)
  for (int p = tid; p < N; p += NT) {
    const int e = ids[p];
    bk[p] = (e < 0 || e >= E) ? E : e;
  }
  lds_barrier();
  for (int p = tid; p < N; p += NT) {
    const int b = bk[p];
    int pos = 0;
#pragma unroll 8
    for (int q = 0; q < N; ++q) {
      const int c = bk[q];
      pos += (c < b) | ((c == b) & (q < p));
    }
    sorted_ids[pos] = p;
  }
  if (tid <= E) {
    int off = 0, cnt = 0;
#pragma unroll 8
    for (int q = 0; q < N; ++q) {
      const int c = bk[q];
      off += c < tid;
      cnt += c == tid;
    }
    expert_offsets[tid] = off;
    S.off[tid] = off;
    S.cnt[tid] = cnt;
    S.ntile[tid] = (tid < E) ? (cnt + BM - 1) / BM : 0;
  }
  lds_barrier();
  if (tid <= E) {
    int toff = 0;
#pragma unroll 8
    for (int e = 0; e < tid; ++e) toff += S.ntile[e];
    if (tid == E) {
      num_tiles[0] = toff;
    } else {
      const int off = S.off[tid], cnt = S.cnt[tid];
      for (int j = 0; j < S.ntile[tid]; ++j) {
        tiles[3 * (toff + j) + 0] = tid;
        tiles[3 * (toff + j) + 1] = off + j * BM;
        tiles[3 * (toff + j) + 2] = min(BM, cnt - j * BM);
      }
    }
  }
  lds_barrier();
}

// The same table for at most 128 slots, built by one wave with no barrier
// (the fused decode router's tail): lane l owns slots l and l + 64.  Slots
// of one bucket find each other with nine ballots (one per bucket bit) per
// half; the first slot of a bucket stores the bucket's count, and two
// exclusive scans over the E + 1 buckets give the row offsets and the tile
// offsets.  Every quantity is a count over the ids, so the table equals
// build_tiles_small's.  scratch: >= kWaveTablesScratch ints of LDS private
// to the wave.
constexpr int kWaveTablesScratch = 4 * (kBuckets + 1);
__device__ inline void build_tiles_wave(const int* ids, int N, int E, int BM, int* scratch,
                                        int32_t* __restrict__ expert_offsets,
                                        int32_t* __restrict__ sorted_ids,
                                        int32_t* __restrict__ tiles,
                                        int32_t* __restrict__ num_tiles) {
  const int lane = threadIdx.x & (kWave - 1);
  int* cnt = scratch;                 // [E + 1] slots per bucket
  int* off = cnt + kBuckets;          // [E + 2] exclusive scan of cnt
  int* nt = off + kBuckets + 1;       // [E + 1] tiles per bucket
  int* toff = nt + kBuckets;          // [E + 2] exclusive scan of nt
  for (int e = lane; e <= E; e += kWave) cnt[e] = 0;
  const int halves = N > kWave ? 2 : 1;  // uniform
  int b[2];
  uint64_t valid[2], bal[2][9];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int p = lane + kWave * s;
    const bool v = p < N;
    b[s] = 0;
    if (v) {
      const int e = ids[p];
      b[s] = (e < 0 || e >= E) ? E : e;
    }
    valid[s] = __ballot(v);
#pragma unroll
    for (int i = 0; i < 9; ++i) bal[s][i] = __ballot(v && ((b[s] >> i) & 1));
  }
  // same-bucket masks of slot (s, lane) within half h
  int before[2], same[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    uint64_t m[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      m[h] = valid[h];
#pragma unroll
      for (int i = 0; i < 9; ++i) m[h] &= ((b[s] >> i) & 1) ? bal[h][i] : ~bal[h][i];
    }
    same[s] = __popcll(m[0]) + __popcll(m[1]);
    before[s] = s == 0 ? lanes_below(m[0]) : __popcll(m[0]) + lanes_below(m[1]);
    if (s + 1 >= halves) {  // uniform: no second half
      if (s == 0) { same[1] = 0; before[1] = 1; }
      break;
    }
  }
  wave_lds_sync();  // the zeroed counts before the first slots' stores
#pragma unroll
  for (int s = 0; s < 2; ++s)
    if (((valid[s] >> lane) & 1) && before[s] == 0) cnt[b[s]] = same[s];
  wave_lds_sync();
  wave_exclusive_scan(cnt, off, E + 1, lane);
  for (int e = lane; e <= E; e += kWave) nt[e] = e < E ? (cnt[e] + BM - 1) / BM : 0;
  wave_lds_sync();
  wave_exclusive_scan(nt, toff, E + 1, lane);
  wave_lds_sync();
  for (int e = lane; e <= E; e += kWave) expert_offsets[e] = off[e];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    if (!((valid[s] >> lane) & 1)) continue;
    const int o = off[b[s]];
    sorted_ids[o + before[s]] = lane + kWave * s;
    if (before[s] == 0 && b[s] < E) {
      const int t0 = toff[b[s]];
      const int n = (same[s] + BM - 1) / BM;
      for (int j = 0; j < n; ++j) {
        tiles[3 * (t0 + j) + 0] = b[s];
        tiles[3 * (t0 + j) + 1] = o + j * BM;
        tiles[3 * (t0 + j) + 2] = min(BM, same[s] - j * BM);
      }
    }
  }
  if (lane == 0) num_tiles[0] = toff[E];
}

}  // namespace moe
