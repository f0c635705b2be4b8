// Expert-cache slot table in HBM: (layer, expert) identity -> VRAM slot.
//
// The pages' engine keeps a hot cache of expert slots in VRAM and fetches a
// miss over PCIe from host RAM ("一张 RTX 4090 跑千亿模型，Strata 实测
// 155 tok/s", section 如何做到：三层存储).  The eviction policy is not stated;
// the reading here is LRU with these exact rules, for one call:
//   clock += 1; U = sorted unique identities; every hit gets stamp = clock;
//   each miss, ascending identity, takes the lowest free slot, else the slot
//   with the smallest (stamp, slot) among slots whose stamp < clock.
// Because a slot taken by a miss gets stamp = clock and leaves the eligible
// set, the misses simply take the |misses| smallest keys in ascending order,
// where a free slot s has key s and an occupied eligible slot has key
// 2^56 + stamp * 2^24 + s.  So one pass finds them all.  Every miss finds a
// slot iff |U| <= n_slots; otherwise nothing changes and the call fails.
// The clock lives in device memory (stats[5]) so that a call needs no host
// state and can sit in a captured graph; it advances only on success.
//
// Misses are filled either by the host (hipMemcpyAsync of each missed blob
// after it has read the miss list back) or, with no host round trip, by
// fill_kernel: each workgroup copies one chunk of one missed blob from the
// pinned host store (mapped into the device address space; the reads cross
// the host link) into its slot.  The pages name the link as the bottleneck
// of a miss; the zero-copy fill removes the per-layer host synchronisation.
// (A capped decode layer runs the same copy in spare workgroups of its
// bucketing launch instead of a launch of its own: fill.h.)
#include "device_util.h"
#include "fill.h"
#include "moe_internal.h"

namespace {

constexpr int kThreads = 1024;
constexpr uint64_t kNone = ~0ull;

__device__ uint64_t block_min_u64(uint64_t v, uint64_t *sh) {
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
    for (int w = 1; w < kThreads / 64; ++w) m = sh[w] < m ? sh[w] : m;
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
// could not pin their working set, [5] the clock
__global__ void __launch_bounds__(kThreads) resolve_kernel(const int32_t *__restrict__ idx, int n, int layer, int E,
                                                           int S, int resident, int clear_on_fail,
                                                           int32_t *__restrict__ slot_of, int32_t *__restrict__ id_of,
                                                           uint32_t *__restrict__ stamp,
                                                           int32_t *__restrict__ slot_of_pair,
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
  for (int p = tid; p < n; p += kThreads) {
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
      for (int p = tid; p < n; p += kThreads) slot_of_pair[p] = -1;
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
    uint64_t best = kNone;
    for (int s = tid; s < S; s += kThreads) {
      uint64_t key;
      if (id_of[s] < 0)
        key = (uint64_t)s;
      else if (stamp[s] < clock)
        key = (1ull << 56) | ((uint64_t)stamp[s] << 24) | (uint64_t)s;
      else
        key = kNone;
      if ((i == 0 || key > prev) && key < best) best = key;
    }
    best = block_min_u64(best, shred);
    if (best == kNone) {  // cannot happen on a consistent table; never write out of range
      if (clear_on_fail)
        for (int p = tid; p < n; p += kThreads) slot_of_pair[p] = -1;
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
  for (int p = tid; p < n; p += kThreads) {
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

// Zero-copy miss fill: workgroup b copies chunk b % kFillChunks of miss
// b / kFillChunks (if that miss exists) into its slot.
constexpr int kFillChunks = 64;
constexpr int kFillThreads = 256;

__global__ void __launch_bounds__(kFillThreads) fill_kernel(moe::FillArgs F) {
  moe::fill_chunk(F, blockIdx.x / kFillChunks, blockIdx.x % kFillChunks, threadIdx.x, kFillThreads);
}

}  // namespace

namespace moe {

FillArgs fill_args(const moe_ctx *c, int chunks) {
  FillArgs F;
  F.dmiss = c->dmiss;
  F.host = c->host_dev;
  F.pool = (uint8_t *)c->cfg.slot_pool;
  F.stride = c->L.stride;
  F.n_ids = (int64_t)c->cfg.n_layers * c->cfg.n_experts;
  F.n_slots = c->cfg.n_slots;
  F.chunks = chunks;
  return F;
}

hipError_t launch_resolve(moe_ctx *c, int layer, const int32_t *idx, int T, int32_t *slot_of_pair, bool fill,
                          hipStream_t s, bool launch_fill) {
  const int n = T * c->cfg.top_k;
  hipLaunchKernelGGL(resolve_kernel, dim3(1), dim3(kThreads), 0, s, idx, n, layer, c->cfg.n_experts, c->cfg.n_slots,
                     c->resident ? 1 : 0, fill ? 1 : 0, c->slot_of, c->id_of, c->stamp, slot_of_pair, c->dmiss,
                     c->dstats);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || c->resident || !fill || !launch_fill) return e;
  // at most min(pairs, experts) misses per call
  const int n_miss = n < c->cfg.n_experts ? n : c->cfg.n_experts;
  hipLaunchKernelGGL(fill_kernel, dim3(n_miss * kFillChunks), dim3(kFillThreads), 0, s, fill_args(c, kFillChunks));
  return hipGetLastError();
}

}  // namespace moe
