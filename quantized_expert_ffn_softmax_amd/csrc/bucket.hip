// Token -> expert bucketing: per-expert pair counts, their exclusive scan
// (offsets[E+1]) and a stable scatter of pair ids (perm), plus the list of
// work entries (<= entry_m tokens of one expert each, then the shared
// expert's tokens) that the FFN kernels walk.
#include <mutex>

#include "device_util.h"
#include "moe_internal.h"
#include "record.h"
#include "topk_small.h"

namespace {

constexpr int kBucketThreads = 1024;
constexpr int kChunk = 256;     // pairs per chunk of the multi-block path
constexpr int kSmallMax = 1024; // pairs handled by the single-workgroup path

// Work entries from per-expert counts (one thread per expert, E <= 1024):
// expert e contributes ceil(cnt/entry_m) entries, ascending e; then the
// shared expert's T tokens in ceil(T/entry_m) entries.
__device__ void build_work(const int *cnt_sh, const int *off_sh, int E, int T, int entry_m, moe::WorkEntry *work,
                           int32_t *n_work, int *sh) {
  const int e = threadIdx.x;
  const int c = e < E ? cnt_sh[e] : 0;
  const int ne = (c + entry_m - 1) / entry_m;
  int total;
  const int base = moe::block_excl_scan_1024(ne, &total, sh);
  if (e < E) {
    for (int i = 0; i < ne; ++i) {
      moe::WorkEntry w;
      w.expert = e;
      w.first = off_sh[e] + i * entry_m;
      w.m = min(entry_m, c - i * entry_m);
      w.pad = 0;
      work[base + i] = w;
    }
  }
  const int ns = (T + entry_m - 1) / entry_m;
  for (int i = threadIdx.x; i < ns; i += blockDim.x) {
    moe::WorkEntry w;
    w.expert = -1;
    w.first = i * entry_m;
    w.m = min(entry_m, T - i * entry_m);
    w.pad = 0;
    work[total + i] = w;
  }
  if (threadIdx.x == 0) {
    n_work[0] = total + ns;
    n_work[1] = total;
  }
}

// n = T*k <= 1024 pairs, E <= 1024: one workgroup does the bucketing with
// blockDim.x >= max(n, E) threads (thread i holds pair i and expert i).
//   1. each pair takes a slot in its expert by an LDS atomic (arrival order)
//   2. one scan over the experts of (entries << 16 | pairs) gives the offsets
//      and the first work entry of every expert (both totals <= 1024)
//   3. pair ids go to their expert's segment in slot order, and each pair's
//      place is its rank among the ids of its segment: perm is the stable
//      order (ascending expert, then ascending pair id), at a cost of the
//      segment's length instead of the number of pairs.
// idx may point to global memory or to LDS.  With nuniq (LDS, zeroed and
// published by a barrier before the call) the number of experts with at least
// one pair is added to it; every thread of the block must call this.
__device__ void bucket_block(const int32_t *idx, int n, int E, int T, int32_t *__restrict__ offsets,
                             int32_t *__restrict__ perm, int build, int entry_m, moe::WorkEntry *work,
                             int32_t *n_work, int *nuniq, moe::WorkEntry *work8) {
  __shared__ int cnt[1024];
  __shared__ int off[1024];
  __shared__ int ids[kSmallMax];
  __shared__ int wsum[kBucketThreads / 64];
  __shared__ int wsum8[kBucketThreads / 64];
  const int tid = threadIdx.x, nt = blockDim.x;
  const int lane = tid & 63, wave = tid >> 6, nwaves = nt >> 6;
  int ex = -1;
  if (tid < n) {
    const int v = idx[tid];
    ex = (v >= 0 && v < E) ? v : -1;  // out-of-range ids are ignored
  }
  if (tid < E) cnt[tid] = 0;
  __syncthreads();
  const int slot = ex >= 0 ? atomicAdd(&cnt[ex], 1) : 0;
  __syncthreads();
  const int c = tid < E ? cnt[tid] : 0;
  if (nuniq) {
    const uint64_t used = __ballot(c > 0);
    if (lane == 0 && used) atomicAdd(nuniq, __popcll(used));
  }
  const int ne = build ? (c + entry_m - 1) / entry_m : 0;
  const int packed = (ne << 16) | c;
  const int incl = moe::wave_incl_scan(packed);
  if (lane == 63) wsum[wave] = incl;
  // the second list's entries per expert (8 pairs each), scanned alongside
  const int ne8 = work8 ? (c + moe::kEntryTokens8 - 1) / moe::kEntryTokens8 : 0;
  const int incl8 = moe::wave_incl_scan(ne8);
  if (lane == 63) wsum8[wave] = incl8;
  __syncthreads();
  int before = 0, total = 0, before8 = 0, total8 = 0;
  for (int w = 0; w < nwaves; ++w) {
    const int v = wsum[w], v8 = wsum8[w];
    before += w < wave ? v : 0;
    total += v;
    before8 += w < wave ? v8 : 0;
    total8 += v8;
  }
  const int excl = before + incl - packed;
  const int oe = excl & 0xffff, total_pairs = total & 0xffff;
  if (tid < E) {
    off[tid] = oe;
    offsets[tid] = oe;
  }
  if (tid == 0) offsets[E] = total_pairs;
  if (build) {
    const int eb = excl >> 16, total_ents = total >> 16;
    for (int i = 0; i < ne; ++i) {
      moe::WorkEntry w;
      w.expert = tid;
      w.first = oe + i * entry_m;
      w.m = min(entry_m, c - i * entry_m);
      w.pad = 0;
      work[eb + i] = w;
    }
    // then the shared expert's T tokens
    const int ns = (T + entry_m - 1) / entry_m;
    for (int i = tid; i < ns; i += nt) {
      moe::WorkEntry w;
      w.expert = -1;
      w.first = i * entry_m;
      w.m = min(entry_m, T - i * entry_m);
      w.pad = 0;
      work[total_ents + i] = w;
    }
    if (tid == 0) {
      n_work[0] = total_ents + ns;
      n_work[1] = total_ents;
    }
    if (work8) {
      constexpr int m8 = moe::kEntryTokens8;
      const int eb8 = before8 + incl8 - ne8;
      for (int i = 0; i < ne8; ++i) {
        moe::WorkEntry w;
        w.expert = tid;
        w.first = oe + i * m8;
        w.m = min(m8, c - i * m8);
        w.pad = 0;
        work8[eb8 + i] = w;
      }
      const int ns8 = (T + m8 - 1) / m8;
      for (int i = tid; i < ns8; i += nt) {
        moe::WorkEntry w;
        w.expert = -1;
        w.first = i * m8;
        w.m = min(m8, T - i * m8);
        w.pad = 0;
        work8[total8 + i] = w;
      }
      if (tid == 0) {
        n_work[2] = total8 + ns8;
        n_work[3] = total8;
      }
    }
  }
  __syncthreads();
  if (ex >= 0) ids[off[ex] + slot] = tid;
  __syncthreads();
  if (ex >= 0) {
    const int base = off[ex], len = cnt[ex];
    int r = 0;
    for (int j = 0; j < len; ++j) r += ids[base + j] < tid;
    perm[base + r] = tid;
  }
}

// Workgroup 0 buckets (bucket_block); the next xrec_blocks workgroups build
// the record of x (decode path); any further ones fill a capped cache's
// misses, fill.chunks workgroups per miss of the resolve's list (the bucketing
// does not depend on the resolve, so the two need no order beyond the resolve
// launch before this one).  With stats (a resident cache, whose slots are the
// identities), workgroup 0 also records what the resolve kernel records for a
// resident call: the number of distinct experts touched as this call's
// lookups and hits, and one call -- so the lookup needs no launch of its own.
__global__ void __launch_bounds__(kBucketThreads) bucket_small(const int32_t *__restrict__ idx, int n, int E, int T,
                                                       int32_t *__restrict__ offsets, int32_t *__restrict__ perm,
                                                       int build, int entry_m, moe::WorkEntry *work,
                                                       int32_t *n_work, const float *__restrict__ x, int d, int nsb,
                                                       uint16_t *__restrict__ xrec, int xrec_h, int xrec_blocks,
                                                       int32_t *__restrict__ dmiss, int64_t *__restrict__ stats,
                                                       moe::WorkEntry *work8, moe::FillArgs fill) {
  if (blockIdx.x > 0) {
    const int b = blockIdx.x - 1;
    if (b < xrec_blocks) {
      moe::build_xrec_range(x, T, d, nsb, xrec, xrec_h, b * blockDim.x + threadIdx.x, xrec_blocks * blockDim.x);
    } else if (fill.chunks > 0) {
      const int fb = b - xrec_blocks;
      moe::fill_chunk(fill, fb / fill.chunks, fb % fill.chunks, threadIdx.x, blockDim.x);
    }
    return;
  }
  __shared__ int nuniq_sh;
  if (threadIdx.x == 0) nuniq_sh = 0;  // published by bucket_block's first barrier
  bucket_block(idx, n, E, T, offsets, perm, build, entry_m, work, n_work, stats ? &nuniq_sh : nullptr, work8);
  if (stats && threadIdx.x == 0) {
    const int nu = nuniq_sh;
    dmiss[0] = nu;
    dmiss[1] = 0;
    dmiss[2] = 0;
    atomicAdd(reinterpret_cast<unsigned long long *>(stats + 0), (unsigned long long)nu);
    atomicAdd(reinterpret_cast<unsigned long long *>(stats + 1), (unsigned long long)nu);
    atomicAdd(reinterpret_cast<unsigned long long *>(stats + 3), 1ull);
  }
}

// A resident decode layer of one or two tokens (moe_decode_layer uses it for
// one: two top-ks one after another cost more than the launch they save):
// workgroup 0 finishes the router's top-k of each token from its partial
// logits (topk_small.h, as the router's own finishing kernel does with one
// workgroup per token), then
// buckets the pairs it has just written and records the lookup, as
// bucket_small does with stats; the other workgroups build the x record,
// which does not depend on the routing.  One launch where the separate steps
// make two.
__global__ void __launch_bounds__(kBucketThreads) route_bucket_small(
    const float *__restrict__ part, int KS, const float *__restrict__ bias, int k, float *__restrict__ logits,
    int32_t *__restrict__ idx, float *__restrict__ w, int E, int T, int32_t *__restrict__ offsets,
    int32_t *__restrict__ perm, int entry_m, moe::WorkEntry *work, int32_t *n_work, const float *__restrict__ x, int d,
    int nsb, uint16_t *__restrict__ xrec, int xrec_h, int xrec_blocks, int32_t *__restrict__ dmiss,
    int64_t *__restrict__ stats, moe::WorkEntry *work8) {
  if (blockIdx.x > 0) {
    moe::build_xrec_range(x, T, d, nsb, xrec, xrec_h, (blockIdx.x - 1) * blockDim.x + threadIdx.x,
                          xrec_blocks * blockDim.x);
    return;
  }
  for (int t = 0; t < T; ++t) {
    moe::finish_token(part, T, t, E, KS, bias, k, logits, idx, w);
    __syncthreads();  // the top-k's LDS is reused by the next token
  }
  __threadfence_block();  // idx, written by the top-k's first k threads, read by every thread below
  __shared__ int nuniq_sh;
  if (threadIdx.x == 0) nuniq_sh = 0;
  __syncthreads();
  bucket_block(idx, T * k, E, T, offsets, perm, 1, entry_m, work, n_work, &nuniq_sh, work8);
  if (threadIdx.x == 0) {
    const int nu = nuniq_sh;
    dmiss[0] = nu;
    dmiss[1] = 0;
    dmiss[2] = 0;
    atomicAdd(reinterpret_cast<unsigned long long *>(stats + 0), (unsigned long long)nu);
    atomicAdd(reinterpret_cast<unsigned long long *>(stats + 1), (unsigned long long)nu);
    atomicAdd(reinterpret_cast<unsigned long long *>(stats + 3), 1ull);
  }
}

// Multi-block path, phase 1: per-chunk histograms chunk_cnt[chunk][E].
__global__ void __launch_bounds__(kChunk) bucket_hist(const int32_t *__restrict__ idx, int n, int E,
                                                      int32_t *__restrict__ chunk_cnt) {
  __shared__ int cnt[1024];
  for (int e = threadIdx.x; e < E; e += kChunk) cnt[e] = 0;
  __syncthreads();
  const int p = blockIdx.x * kChunk + threadIdx.x;
  if (p < n) {
    const int e = idx[p];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kChunk) chunk_cnt[(size_t)blockIdx.x * E + e] = cnt[e];
}

// Phase 2: one workgroup turns chunk counts into chunk bases (within the
// expert), writes offsets and builds the work list.
__global__ void __launch_bounds__(kBucketThreads) bucket_scan(int32_t *__restrict__ chunk_cnt, int nchunks, int E, int T,
                                                      int32_t *__restrict__ offsets, int build, int entry_m,
                                                      moe::WorkEntry *work, int32_t *n_work, moe::WorkEntry *work8) {
  __shared__ int cnt[1024];
  __shared__ int off[1025];
  __shared__ int sh[17];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    // 32 chunk counts in flight per batch (one dependent read per chunk was
    // bound by memory latency: 480 chunks took ~120 us)
    constexpr int kBatch = 32;
    for (int ch0 = 0; ch0 < nchunks; ch0 += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) v[i] = ch0 + i < nchunks ? chunk_cnt[(size_t)(ch0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        if (ch0 + i < nchunks) chunk_cnt[(size_t)(ch0 + i) * E + e] = run;
        run += v[i];
      }
    }
    cnt[e] = run;
  }
  int total;
  const int excl = moe::block_excl_scan_1024(e < E ? run : 0, &total, sh);
  if (e < E) off[e] = excl;
  if (e == 0) off[E] = total;
  __syncthreads();
  if (e < E) offsets[e] = off[e];
  if (e == 0) offsets[E] = off[E];  // thread E does not exist when E == 1024
  if (build) build_work(cnt, off, E, T, entry_m, work, n_work, sh);
  if (build && work8) build_work(cnt, off, E, T, moe::kEntryTokens8, work8, n_work + 2, sh);
}

// Phase 3: stable scatter; rank inside the chunk by counting earlier equal ids.
__global__ void __launch_bounds__(kChunk) bucket_scatter(const int32_t *__restrict__ idx, int n, int E,
                                                         const int32_t *__restrict__ chunk_base,
                                                         const int32_t *__restrict__ offsets,
                                                         int32_t *__restrict__ perm) {
  __shared__ int ex[kChunk];
  const int p = blockIdx.x * kChunk + threadIdx.x;
  int v = p < n ? idx[p] : -1;
  ex[threadIdx.x] = (v >= 0 && v < E) ? v : -1;
  __syncthreads();
  if (p < n && ex[threadIdx.x] >= 0) {
    const int e = ex[threadIdx.x];
    int r = 0;
    for (int q = 0; q < (int)threadIdx.x; ++q) r += ex[q] == e;
    perm[offsets[e] + chunk_base[(size_t)blockIdx.x * E + e] + r] = p;
  }
}

}  // namespace

namespace moe {

hipError_t launch_bucket_ex(const moe_ctx *c, const int32_t *idx, int T, int32_t *offsets, int32_t *perm, bool build,
                            int entry_m, const float *x, uint16_t *xrec, int xrec_h, hipStream_t s,
                            moe::WorkEntry *work8) {
  const int E = c->cfg.n_experts, n = T * c->cfg.top_k;
  if (n <= kSmallMax) {
    // one thread per pair and per expert; with x, 1 + enough workgroups to
    // build its record, one value per thread (so all its loads are in flight
    // at once: at 8 per thread the record took ~6 us of dependent loads)
    const int nt = ((n > E ? n : E) + 63) / 64 * 64;
    const int xb = x ? (T * c->L.gate.nsb * moe::kSteps * 8 + nt - 1) / nt : 0;
    hipLaunchKernelGGL(bucket_small, dim3(1 + xb), dim3(nt), 0, s, idx, n, E, T, offsets, perm,
                       build ? 1 : 0, entry_m, c->work, c->n_work, x, c->cfg.d_model, c->L.gate.nsb, xrec, xrec_h, xb,
                       (int32_t *)nullptr, (int64_t *)nullptr, work8, moe::FillArgs{});
    return hipGetLastError();
  }
  const int nch = (n + kChunk - 1) / kChunk;
  hipLaunchKernelGGL(bucket_hist, dim3(nch), dim3(kChunk), 0, s, idx, n, E, c->chunk_ws);
  hipLaunchKernelGGL(bucket_scan, dim3(1), dim3(kBucketThreads), 0, s, c->chunk_ws, nch, E, T, offsets, build ? 1 : 0,
                     entry_m, c->work, c->n_work, work8);
  hipLaunchKernelGGL(bucket_scatter, dim3(nch), dim3(kChunk), 0, s, idx, n, E, c->chunk_ws, offsets, perm);
  return hipGetLastError();
}

hipError_t launch_bucket(const moe_ctx *c, const int32_t *idx, int T, int32_t *offsets, int32_t *perm, bool build,
                         hipStream_t s) {
  return launch_bucket_ex(c, idx, T, offsets, perm, build, 16, nullptr, nullptr, 0, s, nullptr);
}

hipError_t launch_bucket_lookup(const moe_ctx *c, const int32_t *idx, int T, int entry_m, const float *x,
                                uint16_t *xrec, int xrec_h, hipStream_t s) {
  const int E = c->cfg.n_experts, n = T * c->cfg.top_k;
  if (n > kSmallMax || E > 1024 || !c->resident) return hipErrorInvalidValue;
  const int nt = ((n > E ? n : E) + 63) / 64 * 64;
  const int xb = (T * c->L.gate.nsb * moe::kSteps * 8 + nt - 1) / nt;
  hipLaunchKernelGGL(bucket_small, dim3(1 + xb), dim3(nt), 0, s, idx, n, E, T, c->offsets_ws, c->perm_ws, 1, entry_m,
                     c->work, c->n_work, x, c->cfg.d_model, c->L.gate.nsb, xrec, xrec_h, xb, c->dmiss, c->dstats,
                     c->work8, moe::FillArgs{});
  return hipGetLastError();
}

hipError_t launch_route_bucket_lookup(const moe_ctx *c, int T, const float *bias, float *logits, int32_t *idx, float *w,
                                     int entry_m, const float *x, uint16_t *xrec, int xrec_h, hipStream_t s) {
  const int E = c->cfg.n_experts, k = c->cfg.top_k, n = T * k;
  if (!c->resident || T < 1 || T > 2 || T > c->route_small_t || n > kSmallMax || E > 1024) return hipErrorInvalidValue;
  // the top-k needs a thread per expert, the bucketing one per pair and per expert
  const int nt = ((n > E ? n : E) + 63) / 64 * 64;
  const int xb = (T * c->L.gate.nsb * moe::kSteps * 8 + nt - 1) / nt;
  hipLaunchKernelGGL(route_bucket_small, dim3(1 + xb), dim3(nt), 0, s, c->route_part, c->route_ks, bias, k, logits,
                     idx, w, E, T, c->offsets_ws, c->perm_ws, entry_m, c->work, c->n_work, x, c->cfg.d_model,
                     c->L.gate.nsb, xrec, xrec_h, xb, c->dmiss, c->dstats, c->work8);
  return hipGetLastError();
}

hipError_t launch_bucket_fill(const moe_ctx *c, const int32_t *idx, int T, int entry_m, const float *x,
                              uint16_t *xrec, int xrec_h, hipStream_t s) {
  const int E = c->cfg.n_experts, n = T * c->cfg.top_k;
  if (n > kSmallMax || E > 1024 || c->resident || !c->host_dev) return hipErrorInvalidValue;
  const int nt = ((n > E ? n : E) + 63) / 64 * 64;
  const int xb = x ? (T * c->L.gate.nsb * moe::kSteps * 8 + nt - 1) / nt : 0;
  // as many threads per blob as the fill kernel's 64 x 256; at most
  // min(pairs, experts) misses per call
  const int chunks = (16384 + nt - 1) / nt, n_miss = n < E ? n : E;
  hipLaunchKernelGGL(bucket_small, dim3(1 + xb + n_miss * chunks), dim3(nt), 0, s, idx, n, E, T, c->offsets_ws,
                     c->perm_ws, 1, entry_m, c->work, c->n_work, x, c->cfg.d_model, c->L.gate.nsb, xrec, xrec_h, xb,
                     (int32_t *)nullptr, (int64_t *)nullptr, c->work8, fill_args(c, chunks));
  return hipGetLastError();
}

}  // namespace moe

// ---------------------------------------------------------------------------
// Allocation-free bucketing.  Past 1,024 pairs the bucketing keeps per-chunk
// expert counts in a scratch buffer; this entry point takes it from a
// file-scope device array instead of a context's workspace, so it needs no
// context and calls no allocator.  Every chunk row the kernels read is
// written first in the same call (the histogram writes all E counts of each
// chunk), so nothing has to be cleared between calls.  One array per GPU,
// shared by every call on that GPU: calls that overlap on one GPU race.
// ---------------------------------------------------------------------------
namespace {
constexpr int kNoAllocMaxPairs = 131072;  // 512 chunks of 256 pairs
constexpr int kNoAllocMaxExperts = 1024;
constexpr int kMaxDevices = 64;
}  // namespace

static __device__ __align__(256) int32_t scratch[(kNoAllocMaxPairs / kChunk) * kNoAllocMaxExperts];  // 2 MiB

// The array's device address, looked up once per device with that device
// current; host code uses only this address, never the symbol itself.
static std::mutex g_scratch_mu;
static int32_t *g_scratch_addr[kMaxDevices];

static hipError_t scratch_addr(int32_t **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = static_cast<int32_t *>(p);
  }
  *out = g_scratch_addr[dev];
  return hipSuccess;
}

extern "C" moe_status moe_bucket_noalloc(const int32_t *idx, int32_t T, int32_t top_k, int32_t n_experts,
                                         int32_t *offsets, int32_t *perm, void *stream) {
  MOE_CHECK(idx && offsets && perm, MOE_ERR_INVALID, "moe_bucket_noalloc: null idx, offsets or perm");
  MOE_CHECK(T >= 1 && top_k >= 1 && top_k <= 32, MOE_ERR_INVALID, "moe_bucket_noalloc: need T >= 1 and 1 <= top_k <= 32");
  MOE_CHECK(n_experts >= 1 && n_experts <= kNoAllocMaxExperts, MOE_ERR_INVALID,
            "moe_bucket_noalloc: n_experts must be 1..1024");
  MOE_CHECK((int64_t)T * top_k <= kNoAllocMaxPairs, MOE_ERR_INVALID,
            "moe_bucket_noalloc: at most 131,072 pairs (T * top_k): the static scratch holds 512 chunks x 1,024 "
            "expert counts (2 MiB)");
  const int n = T * top_k, E = n_experts;
  hipStream_t s = (hipStream_t)stream;
  if (n <= kSmallMax) {  // one workgroup, no scratch
    const int nt = ((n > E ? n : E) + 63) / 64 * 64;
    hipLaunchKernelGGL(bucket_small, dim3(1), dim3(nt), 0, s, idx, n, E, T, offsets, perm, 0, 1,
                       (moe::WorkEntry *)nullptr, (int32_t *)nullptr, (const float *)nullptr, 0, 0,
                       (uint16_t *)nullptr, 0, 0, (int32_t *)nullptr, (int64_t *)nullptr, (moe::WorkEntry *)nullptr,
                       moe::FillArgs{});
    MOE_HIP(hipGetLastError());
    return MOE_OK;
  }
  int32_t *chunk = nullptr;
  MOE_HIP(scratch_addr(&chunk));
  const int nch = (n + kChunk - 1) / kChunk;
  hipLaunchKernelGGL(bucket_hist, dim3(nch), dim3(kChunk), 0, s, idx, n, E, chunk);
  hipLaunchKernelGGL(bucket_scan, dim3(1), dim3(kBucketThreads), 0, s, chunk, nch, E, T, offsets, 0, 1,
                     (moe::WorkEntry *)nullptr, (int32_t *)nullptr, (moe::WorkEntry *)nullptr);
  hipLaunchKernelGGL(bucket_scatter, dim3(nch), dim3(kChunk), 0, s, idx, n, E, (const int32_t *)chunk,
                     (const int32_t *)offsets, perm);
  MOE_HIP(hipGetLastError());
  return MOE_OK;
}
