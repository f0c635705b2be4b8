// The cache resolve as a workgroup-wide device function (the LRU rules are
// stated where the resolve kernel is defined, cache.hip): the resolve kernel
// runs it alone, and a capped decode layer of a single token runs it in
// the workgroup that has just finished the router's top-k.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_util.h"

namespace moe {

constexpr int kResolveThreads = 1024;
constexpr uint64_t kResolveNone = ~0ull;

__device__ inline uint64_t block_min_u64(uint64_t v, uint64_t *sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint64_t o = __shfl_xor(v, off, 64);
    v = o < v ? o : v;
  }
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t m = sh[0];
    for (int w = 1; w < kResolveThreads / 64; ++w) m = sh[w] < m ? sh[w] : m;
    sh[16] = m;
  }
  __syncthreads();
  const uint64_t r = sh[16];
  __syncthreads();
  return r;
}

// counters are added without reading them back (no round trip before the
// kernel can end); one thread of one workgroup adds, so the sums are exact
__device__ inline void add_stat(int64_t *p, int64_t v) {
  atomicAdd(reinterpret_cast<unsigned long long *>(p), static_cast<unsigned long long>(v));
}

// stats: [0] unique identities, [1] hits, [2] misses, [3] calls, [4] calls that
// could not pin their working set, [5] the clock.  The whole workgroup
// (kResolveThreads threads) runs it; idx may have been written by the same
// workgroup before a barrier.
__device__ inline void resolve_block(const int32_t *__restrict__ idx, int n, int layer, int E, int S, int resident,
                                     int clear_on_fail, int32_t *__restrict__ slot_of, int32_t *__restrict__ id_of,
                                     uint32_t *__restrict__ stamp, int32_t *__restrict__ slot_of_pair,
                                     int32_t *__restrict__ dmiss, int64_t *__restrict__ stats) {
  __shared__ int mark[1024];
  __shared__ int miss_e[1024];
  __shared__ int victim[1024];
  __shared__ int scan_sh[17];
  __shared__ int nuniq_sh;
  __shared__ uint64_t shred[17];
  const int tid = threadIdx.x;
  const int base = layer * E;
  mark[tid] = 0;
  if (tid == 0) nuniq_sh = 0;
  __syncthreads();
  for (int p = tid; p < n; p += kResolveThreads) {
    const int e = idx[p];
    if (e >= 0 && e < E) mark[e] = 1;  // same value from every writer
    // resident: the slot is the identity, known from the id alone
    if (resident && slot_of_pair) slot_of_pair[p] = (e >= 0 && e < E) ? base + e : -1;
  }
  __syncthreads();
  if (resident) {
    // unique count: one ballot per wave, one LDS add per wave
    const uint64_t b = __ballot(tid < E && mark[tid]);
    if ((tid & 63) == 0 && b) atomicAdd(&nuniq_sh, __popcll(b));
    __syncthreads();
    if (tid == 0) {
      dmiss[0] = nuniq_sh;
      dmiss[1] = 0;
      dmiss[2] = 0;
      add_stat(stats + 0, nuniq_sh);
      add_stat(stats + 1, nuniq_sh);
      add_stat(stats + 3, 1);
    }
    return;
  }
  const uint32_t clock = (uint32_t)stats[5] + 1u;  // written back (by thread 0, last) only on success
  // capped: unique identities, hits and the ascending list of misses
  const int is_u = (tid < E) && mark[tid];
  const int s_e = is_u ? slot_of[base + tid] : -1;
  const int is_miss = is_u && s_e < 0;
  int nuniq, nmiss;
  (void)moe::block_excl_scan_1024(is_u, &nuniq, scan_sh);
  const int mpos = moe::block_excl_scan_1024(is_miss, &nmiss, scan_sh);
  if (is_miss) miss_e[mpos] = tid;
  if (nuniq > S) {  // cannot pin this call's working set: change nothing
    if (clear_on_fail)  // no host reads the error: the call's pairs get no slot (no output)
      for (int p = tid; p < n; p += kResolveThreads) slot_of_pair[p] = -1;
    if (tid == 0) {
      dmiss[0] = nuniq;
      dmiss[1] = 0;
      dmiss[2] = 1;
      add_stat(stats + 4, 1);
    }
    return;
  }
  if (is_u && s_e >= 0) stamp[s_e] = clock;  // hits leave the eligible set
  __threadfence_block();
  __syncthreads();
  // victims: the nmiss smallest keys, by nmiss rounds of a block min over the
  // keys strictly above the previous winner (keys are unique).  The table is
  // not written during the rounds, so every key stays fixed.
  uint64_t prev = 0;
  for (int i = 0; i < nmiss; ++i) {
    uint64_t best = kResolveNone;
    for (int s = tid; s < S; s += kResolveThreads) {
      uint64_t key;
      if (id_of[s] < 0)
        key = (uint64_t)s;
      else if (stamp[s] < clock)
        key = (1ull << 56) | ((uint64_t)stamp[s] << 24) | (uint64_t)s;
      else
        key = kResolveNone;
      if ((i == 0 || key > prev) && key < best) best = key;
    }
    best = block_min_u64(best, shred);
    if (best == kResolveNone) {  // cannot happen on a consistent table; never write out of range
      if (clear_on_fail)
        for (int p = tid; p < n; p += kResolveThreads) slot_of_pair[p] = -1;
      if (tid == 0) {
        dmiss[0] = nuniq;
        dmiss[1] = 0;
        dmiss[2] = 2;
        add_stat(stats + 4, 1);
      }
      return;
    }
    prev = best;
    if (tid == 0) victim[i] = (int)(best & 0xffffffu);
  }
  __syncthreads();
  // apply: victims are distinct, evicted identities are resident ones not
  // touched by this call, misses are not resident -- no two threads collide
  if (tid < nmiss) {
    const int v = victim[tid];
    const int id = base + miss_e[tid];
    const int old = id_of[v];
    if (old >= 0) slot_of[old] = -1;
    id_of[v] = id;
    slot_of[id] = v;
    stamp[v] = clock;
    dmiss[3 + 2 * tid] = id;
    dmiss[4 + 2 * tid] = v;
  }
  __threadfence_block();
  __syncthreads();
  for (int p = tid; p < n; p += kResolveThreads) {
    const int e = idx[p];
    slot_of_pair[p] = (e >= 0 && e < E) ? slot_of[base + e] : -1;
  }
  if (tid == 0) {
    dmiss[0] = nuniq;
    dmiss[1] = nmiss;
    dmiss[2] = 0;
    add_stat(stats + 0, nuniq);
    add_stat(stats + 1, nuniq - nmiss);
    add_stat(stats + 2, nmiss);
    add_stat(stats + 3, 1);
    stats[5] = clock;
  }
}

}  // namespace moe
