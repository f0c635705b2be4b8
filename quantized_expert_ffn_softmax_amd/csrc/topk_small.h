// The router's top-k for decode-size batches, as a workgroup-wide device
// function: the router's own finishing kernel runs it with one workgroup per
// token, and a capped cache's decode layer runs it, token after token, in the
// workgroup that then resolves the cache.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_util.h"

namespace moe {

// One token: logits = sum of the KS slices (in order) + bias, then the top-k
// by rank, where an expert's rank is the number of experts
// ordered before it by (logit desc, index asc).  The order is that of one
// 64-bit key, (logit mapped to an order-preserving uint32) << 32 | ~index, so
// each comparison is one v_cmp_gt_u64.  Two passes: each wave ranks its 64
// experts among themselves; an expert of global rank < k has wave rank < k,
// so only those candidates (k per wave) are ranked against each other, and
// for a candidate in the global top-k that rank is its global rank (every
// expert ordered before it is a candidate too).  Weights: softmax of the k
// chosen logits.  Token t by the whole workgroup (blockDim.x >= E threads, a
// multiple of 64, at most 1,024; waves past E add no candidate).
__device__ inline void finish_token(const float *__restrict__ part, int T, int t, int E, int KS,
                                    const float *__restrict__ bias, int k, float *__restrict__ logits,
                                    int32_t *__restrict__ idx, float *__restrict__ w) {
  __shared__ __attribute__((aligned(16))) uint64_t lk[1024];
  __shared__ __attribute__((aligned(16))) uint64_t ck[16 * 32];
  __shared__ float top_v[32];
  __shared__ int top_e[32];
  const int e = threadIdx.x, wave = e >> 6;
  float v = -INFINITY;
  if (e < E) {
    // the bias and the KS partial sums, requested together (8 slices at a
    // time, slices past KS clamped and not added), added in slice order
    const float bv = bias ? bias[e] : 0.f;
    v = 0.f;
    for (int q0 = 0; q0 < KS; q0 += 8) {
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = part[((size_t)min(q0 + i, KS - 1) * T + t) * E + e];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (q0 + i < KS) v += p[i];
    }
    v += bv;
    logits[(size_t)t * E + e] = v;
  }
  const uint64_t key = e < E ? order_key(v, e) : 0ull;  // lanes past E order after everything
  lk[e] = key;
  const int nc = (blockDim.x / 64) * k;  // candidate slots, k per wave
  for (int i = e; i < nc; i += blockDim.x) ck[i] = 0ull;  // empty candidate: orders before nothing
  __syncthreads();
  // pass 1: rank inside the wave, two keys per LDS read
  int r1 = 0;
  const ulonglong2 *wk = reinterpret_cast<const ulonglong2 *>(lk + wave * 64);
#pragma unroll 8
  for (int o = 0; o < 32; ++o) {
    const ulonglong2 q = wk[o];
    r1 += (q.x > key) + (q.y > key);
  }
  if (e < E && r1 < k) ck[wave * k + r1] = key;
  __syncthreads();
  // pass 2: the candidates, one per thread of the first waves, ranked among
  // themselves; the k best give their expert and logit
  if (e < nc) {
    const uint64_t ce = ck[e];
    if (ce != 0ull) {
      int r = 0;
      const ulonglong2 *c2 = reinterpret_cast<const ulonglong2 *>(ck);
      for (int i = 0; i < nc / 2; ++i) {  // two candidates per LDS read
        const ulonglong2 q = c2[i];
        r += (q.x > ce) + (q.y > ce);
      }
      if (nc & 1) r += ck[nc - 1] > ce;
      if (r < k) {
        top_v[r] = moe::key_logit(ce);
        top_e[r] = moe::key_expert(ce);
      }
    }
  }
  __syncthreads();
  // softmax of the k chosen logits
  if (e < k) {
    const float m = top_v[0];
    float sum = 0.f;
    for (int j = 0; j < k; ++j) sum += expf(top_v[j] - m);
    idx[(size_t)t * k + e] = top_e[e];
    w[(size_t)t * k + e] = expf(top_v[e] - m) / sum;
  }
}

}  // namespace moe
