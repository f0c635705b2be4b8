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
#include "resolve_block.h"
#include "topk_small.h"

namespace {

constexpr int kThreads = moe::kResolveThreads;

__global__ void __launch_bounds__(kThreads) resolve_kernel(const int32_t *__restrict__ idx, int n, int layer, int E,
                                                           int S, int resident, int clear_on_fail,
                                                           int32_t *__restrict__ slot_of, int32_t *__restrict__ id_of,
                                                           uint32_t *__restrict__ stamp,
                                                           int32_t *__restrict__ slot_of_pair,
                                                           int32_t *__restrict__ dmiss, int64_t *__restrict__ stats) {
  moe::resolve_block(idx, n, layer, E, S, resident, clear_on_fail, slot_of, id_of, stamp, slot_of_pair, dmiss, stats);
}

// A capped decode layer of at most kRouteResolveMaxT tokens (moe_decode_layer
// uses it for one): the router's top-k of each token (from the partial logits
// of the router's first kernel), then the resolve of the call's pairs, in one
// workgroup -- one launch where the separate calls make two, with no handoff
// between workgroups (the top-k's idx reaches the resolve through a barrier).
constexpr int kRouteResolveMaxT = 2;

__global__ void __launch_bounds__(kThreads) route_resolve_kernel(const float *__restrict__ part, int T, int E, int KS,
                                                                 const float *__restrict__ bias, int k,
                                                                 float *__restrict__ logits, int32_t *__restrict__ idx,
                                                                 float *__restrict__ w, int layer, int S,
                                                                 int32_t *__restrict__ slot_of,
                                                                 int32_t *__restrict__ id_of,
                                                                 uint32_t *__restrict__ stamp,
                                                                 int32_t *__restrict__ slot_of_pair,
                                                                 int32_t *__restrict__ dmiss,
                                                                 int64_t *__restrict__ stats) {
  for (int t = 0; t < T; ++t) {
    moe::finish_token(part, T, t, E, KS, bias, k, logits, idx, w);
    __syncthreads();  // the top-k's LDS is reused by the next token
  }
  __threadfence_block();  // idx, written by the top-k's first k threads, read by every thread below
  __syncthreads();
  moe::resolve_block(idx, T * k, layer, E, S, 0, 1, slot_of, id_of, stamp, slot_of_pair, dmiss, stats);
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

hipError_t launch_route_resolve(moe_ctx *c, int layer, int T, const float *bias, float *logits, int32_t *idx,
                                float *w, int32_t *slot_of_pair, hipStream_t s) {
  const int E = c->cfg.n_experts, k = c->cfg.top_k;
  if (c->resident || T < 1 || T > kRouteResolveMaxT || T > c->route_small_t || E > kThreads || T * k > kThreads)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(route_resolve_kernel, dim3(1), dim3(kThreads), 0, s, c->route_part, T, E, c->route_ks, bias, k,
                     logits, idx, w, layer, c->cfg.n_slots, c->slot_of, c->id_of, c->stamp, slot_of_pair, c->dmiss,
                     c->dstats);
  return hipGetLastError();
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
