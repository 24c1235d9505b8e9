// Cross-workgroup hand-offs inside one launch (the single-launch layers):
// agent-scope atomic words, stamped polls with a bounded wait, the arrival
// tree and the per-call epoch.  Every value that crosses workgroups carries
// its own validity in the same 64-bit word (a stamp, or bits + 1 in a buffer
// that starts zeroed), so no release/acquire fence is needed: agent-scope
// accesses are served at the memory side of gfx950's caches, coherent across
// the XCDs' L2s.
#pragma once

#include "moe_device.h"

namespace moe {

namespace {

constexpr int kSpinLimit = 1 << 20;     // polls (about 1 us each) before a wait gives up
constexpr int kMaxK = 3072;             // K of either GEMM: one chunk of weights
typedef unsigned long long u64;

// The sync region at the start of the workspace, in 128-byte lines, then
// the two parity buffers of published partial logits (zero before the first
// call; afterwards each call leaves the region consistent for the next).
constexpr int kLine = 32;      // ints per line
constexpr int kLeaves = 16;    // leaves of the arrival tree
struct Tree {
  int leaf[kLeaves][kLine];
  int top[kLine];
};
struct Sync {
  int reserved;
  int epoch;             // calls begun by every workgroup
  int error;             // set (sticky) when a poll gives up
  int poll_limit;        // 0: kSpinLimit; n > 0: waits give up after n - 1 re-polls
  int pad0[kLine - 4];
  Tree arrivals;         // every workgroup, once it has read the epoch
};
static_assert(sizeof(Sync) % 128 == 0, "whole lines");

// K-ranges of the router: router_plan keeps each >= 128 elements, and these
// kernels take H <= kMaxK.
constexpr int kMaxSplits = kMaxK / 128;

__device__ __forceinline__ int ld_agent(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int add_agent(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u64 ld64(const u64* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st64w(u64* p, u64 v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st64(u64* p, unsigned stamp, unsigned payload) {
  st64w(p, ((u64)stamp << 32) | payload);
}

// Reads the N stamped words p[i] (those with use[i]) until every stamp is
// this call's, in rounds: each round requests all words still stale at
// once, so once the producers are done one round trip suffices.  Returns
// the payloads in v's low halves.
template <int N>
__device__ __forceinline__ void settle(const u64* const (&p)[N], const bool (&use)[N], u64 (&v)[N],
                                       unsigned stamp, int* error, int spin_limit) {
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = use[i] ? ld64(p[i]) : ((u64)stamp << 32);
  for (int round = 0;; ++round) {
    bool stale = false;
#pragma unroll
    for (int i = 0; i < N; ++i) stale |= (unsigned)(v[i] >> 32) != stamp;
    if (!stale) return;
    if (round >= spin_limit) {
      st_agent(error, 1);
      return;
    }
    // a short back-off (about 50 ns): a poll is itself a memory round trip,
    // and longer sleeps measured slower (0.2 us: +0.25 us per call)
    __builtin_amdgcn_s_sleep(2);
#pragma unroll
    for (int i = 0; i < N; ++i)
      if ((unsigned)(v[i] >> 32) != stamp) v[i] = ld64(p[i]);
  }
}

// The partial logits of expert e, splits words at base + c * stride: read
// until each is nonzero (published), every stale word re-requested at once
// per round (all loads unconditional, surplus ones at a clamped address).
// Returns the sum of the decoded values in split order.
__device__ __forceinline__ double settle_partials(const u64* base, size_t stride, int splits,
                                                  int* error, int spin_limit) {
  u64 v[kMaxSplits];
#pragma unroll
  for (int c = 0; c < kMaxSplits; ++c) v[c] = ld64(base + (size_t)min(c, splits - 1) * stride);
  for (int round = 0;; ++round) {
    bool stale = false;
#pragma unroll
    for (int c = 0; c < kMaxSplits; ++c) stale |= v[c] == 0ull;
    if (!stale) break;
    if (round >= spin_limit) {
      st_agent(error, 1);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
#pragma unroll
    for (int c = 0; c < kMaxSplits; ++c)
      if (v[c] == 0ull) v[c] = ld64(base + (size_t)min(c, splits - 1) * stride);
  }
  double sum = 0.0;
#pragma unroll
  for (int c = 0; c < kMaxSplits; ++c)
    if (c < splits) sum += __longlong_as_double((long long)(v[c] - 1ull));
  return sum;
}

// Arrival i of n at the tree (one thread).  True for exactly one arrival,
// the last; every counter touched is reset by its last arrival.
__device__ bool tree_arrive(Tree* t, int i, int n) {
  const int leaf = i % kLeaves;
  const int per_leaf = n / kLeaves + (leaf < n % kLeaves ? 1 : 0);
  if (add_agent(&t->leaf[leaf][0], 1) != per_leaf - 1) return false;
  st_agent(&t->leaf[leaf][0], 0);
  const int leaves = n < kLeaves ? n : kLeaves;
  if (add_agent(&t->top[0], 1) != leaves - 1) return false;
  st_agent(&t->top[0], 0);
  return true;
}

// This workgroup has read `epoch`; the last of the call to check in
// advances it for the next call.
__device__ void check_in(Sync* S, int epoch) {
  if (tree_arrive(&S->arrivals, blockIdx.x, gridDim.x)) st_agent(&S->epoch, epoch + 1);
}

// This call's epoch and poll bound.
struct CallState {
  int epoch;
  int spin_limit;
};
__device__ __forceinline__ CallState read_call_state(const Sync* S) {
  const int epoch = ld_agent(&S->epoch);
  const int pl = ld_agent(&S->poll_limit);
  return CallState{epoch, pl > 0 ? pl - 1 : kSpinLimit};
}

}  // namespace

}  // namespace moe
