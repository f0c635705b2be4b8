// Token -> expert bucketing: per-expert pair counts, their exclusive scan
// (offsets[E+1]) and a stable scatter of pair ids (perm), plus the list of
// work entries (<= entry_m tokens of one expert each, then the shared
// expert's tokens) that the FFN kernels walk.
#include "device_util.h"
#include "moe_internal.h"
#include "record.h"

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

// n = T*k <= 1024 pairs: one workgroup does everything.
__global__ void __launch_bounds__(kBucketThreads) bucket_small(const int32_t *__restrict__ idx, int n, int E, int T,
                                                       int32_t *__restrict__ offsets, int32_t *__restrict__ perm,
                                                       int build, int entry_m, moe::WorkEntry *work,
                                                       int32_t *n_work, const float *__restrict__ x, int d, int nsb,
                                                       uint16_t *__restrict__ xrec, int xrec_h) {
  __shared__ int ex[kSmallMax];
  __shared__ int cnt[1024];
  __shared__ int off[1025];
  __shared__ int sh[17];
  const int tid = threadIdx.x;
  if (blockIdx.x > 0) {
    // decode path: the other workgroups of this launch build the activation
    // record of x (independent of the bucketing done by workgroup 0)
    moe::build_xrec_range(x, T, d, nsb, xrec, xrec_h, (blockIdx.x - 1) * kBucketThreads + tid,
                          (gridDim.x - 1) * kBucketThreads);
    return;
  }
  cnt[tid] = 0;
  __syncthreads();
  if (tid < n) {
    const int e = idx[tid];
    ex[tid] = (e >= 0 && e < E) ? e : -1;  // out-of-range ids are ignored
    if (ex[tid] >= 0) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  int total;
  const int excl = moe::block_excl_scan_1024(tid < E ? cnt[tid] : 0, &total, sh);
  if (tid < E) off[tid] = excl;
  if (tid == 0) off[E] = total;
  __syncthreads();
  if (tid <= E) offsets[tid] = off[tid];
  if (tid < n && ex[tid] >= 0) {
    const int e = ex[tid];
    // stable rank among the pairs of expert e; 16 LDS reads in flight at once
    int r = 0;
    for (int q0 = 0; q0 < tid; q0 += 16) {
      int v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = ex[min(q0 + i, kSmallMax - 1)];
#pragma unroll
      for (int i = 0; i < 16; ++i) r += (q0 + i < tid) && v[i] == e;
    }
    perm[off[e] + r] = tid;
  }
  if (build) build_work(cnt, off, E, T, entry_m, work, n_work, sh);
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
                                                      moe::WorkEntry *work, int32_t *n_work) {
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
  if (e <= E) offsets[e] = off[e];
  if (build) build_work(cnt, off, E, T, entry_m, work, n_work, sh);
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
                            int entry_m, const float *x, uint16_t *xrec, int xrec_h, hipStream_t s) {
  const int E = c->cfg.n_experts, n = T * c->cfg.top_k;
  if (n <= kSmallMax) {
    // with x: 1 + enough workgroups to build its record, one value per
    // thread (so all its loads are in flight at once: at 8 per thread the
    // record took ~6 us of dependent loads)
    int blocks = 1;
    if (x) {
      const int vals = T * c->L.gate.nsb * moe::kSteps * 8;
      blocks += (vals + kBucketThreads - 1) / kBucketThreads;
    }
    hipLaunchKernelGGL(bucket_small, dim3(blocks), dim3(kBucketThreads), 0, s, idx, n, E, T, offsets, perm,
                       build ? 1 : 0, entry_m, c->work, c->n_work, x, c->cfg.d_model, c->L.gate.nsb, xrec, xrec_h);
    return hipGetLastError();
  }
  const int nch = (n + kChunk - 1) / kChunk;
  hipLaunchKernelGGL(bucket_hist, dim3(nch), dim3(kChunk), 0, s, idx, n, E, c->chunk_ws);
  hipLaunchKernelGGL(bucket_scan, dim3(1), dim3(kBucketThreads), 0, s, c->chunk_ws, nch, E, T, offsets, build ? 1 : 0,
                     entry_m, c->work, c->n_work);
  hipLaunchKernelGGL(bucket_scatter, dim3(nch), dim3(kChunk), 0, s, idx, n, E, c->chunk_ws, offsets, perm);
  return hipGetLastError();
}

hipError_t launch_bucket(const moe_ctx *c, const int32_t *idx, int T, int32_t *offsets, int32_t *perm, bool build,
                         hipStream_t s) {
  return launch_bucket_ex(c, idx, T, offsets, perm, build, 16, nullptr, nullptr, 0, s);
}

}  // namespace moe
