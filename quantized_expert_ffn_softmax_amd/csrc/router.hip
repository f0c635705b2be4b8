// Router: logits = x W_r^T + b in fp32, then per token the top-k by
// (logit desc, index asc) and weights renormalised over the k chosen.
//
// The pages fix the shape (10 of 512 experts per token plus one shared
// expert: "一张 RTX 4090 跑千亿模型，Strata 实测 155 tok/s", section
// 如何做到：三层存储); the scoring function is the softmax reading.
#include "moe_internal.h"

namespace {

constexpr int kWave = 64;

// --- logits, few tokens: each wave owns 4 expert rows and streams them once;
// x is re-read from L2 per wave.  T <= 16.
constexpr int kEpw = 4;        // experts per wave
constexpr int kMaxTSmall = 16;

__global__ void __launch_bounds__(256) router_logits_small(const float *__restrict__ x, int T, int d,
                                                           const float *__restrict__ wr,
                                                           const float *__restrict__ bias, int E,
                                                           float *__restrict__ logits) {
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int e0 = wave * kEpw;
  if (e0 >= E) return;
  float acc[kEpw][kMaxTSmall];
#pragma unroll
  for (int a = 0; a < kEpw; ++a)
#pragma unroll
    for (int t = 0; t < kMaxTSmall; ++t) acc[a][t] = 0.f;
  for (int c = lane * 4; c < d; c += kWave * 4) {
    float4 wv[kEpw];
#pragma unroll
    for (int a = 0; a < kEpw; ++a) {
      const int e = e0 + a < E ? e0 + a : E - 1;
      wv[a] = *reinterpret_cast<const float4 *>(wr + (size_t)e * d + c);
    }
#pragma unroll
    for (int t = 0; t < kMaxTSmall; ++t) {
      if (t < T) {
        const float4 xv = *reinterpret_cast<const float4 *>(x + (size_t)t * d + c);
#pragma unroll
        for (int a = 0; a < kEpw; ++a) {
          acc[a][t] = fmaf(wv[a].x, xv.x, acc[a][t]);
          acc[a][t] = fmaf(wv[a].y, xv.y, acc[a][t]);
          acc[a][t] = fmaf(wv[a].z, xv.z, acc[a][t]);
          acc[a][t] = fmaf(wv[a].w, xv.w, acc[a][t]);
        }
      }
    }
  }
#pragma unroll
  for (int a = 0; a < kEpw; ++a) {
#pragma unroll
    for (int t = 0; t < kMaxTSmall; ++t) {
      float v = acc[a][t];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
      acc[a][t] = v;
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int a = 0; a < kEpw; ++a) {
      const int e = e0 + a;
      if (e < E) {
        const float b = bias ? bias[e] : 0.f;
#pragma unroll
        for (int t = 0; t < kMaxTSmall; ++t)
          if (t < T) logits[(size_t)t * E + e] = acc[a][t] + b;
      }
    }
  }
}

// --- logits, many tokens: LDS-tiled fp32 GEMM, 64x64 output tile, each thread 4x4.
constexpr int kTm = 64, kTn = 64, kTk = 16;

__global__ void __launch_bounds__(256) router_logits_gemm(const float *__restrict__ x, int T, int d,
                                                          const float *__restrict__ wr,
                                                          const float *__restrict__ bias, int E,
                                                          float *__restrict__ logits) {
  __shared__ float xs[kTk][kTm + 4];
  __shared__ float ws[kTk][kTn + 4];
  const int tid = threadIdx.x;
  const int m0 = blockIdx.y * kTm, n0 = blockIdx.x * kTn;
  const int tm = (tid / 16) * 4, tn = (tid % 16) * 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < d; k0 += kTk) {
    // 64 rows x 16 cols of x and of W: 1024 floats each, 4 per thread
    for (int i = tid; i < kTm * kTk / 4; i += 256) {
      const int r = i / (kTk / 4), cc = (i % (kTk / 4)) * 4;
      const int gm = m0 + r, gn = n0 + r;
      float4 xv = gm < T ? *reinterpret_cast<const float4 *>(x + (size_t)gm * d + k0 + cc) : make_float4(0, 0, 0, 0);
      float4 wv = gn < E ? *reinterpret_cast<const float4 *>(wr + (size_t)gn * d + k0 + cc) : make_float4(0, 0, 0, 0);
      xs[cc + 0][r] = xv.x; xs[cc + 1][r] = xv.y; xs[cc + 2][r] = xv.z; xs[cc + 3][r] = xv.w;
      ws[cc + 0][r] = wv.x; ws[cc + 1][r] = wv.y; ws[cc + 2][r] = wv.z; ws[cc + 3][r] = wv.w;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kTk; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = xs[kk][tm + i]; b[i] = ws[kk][tn + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int gm = m0 + tm + i;
    if (gm >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gn = n0 + tn + j;
      if (gn < E) logits[(size_t)gm * E + gn] = acc[i][j] + (bias ? bias[gn] : 0.f);
    }
  }
}

// --- top-k and weights: one wave per token.  Lane l holds experts l, l+64, ...
constexpr int kMaxPerLane = 16;  // E <= 1024

__device__ inline bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

__global__ void __launch_bounds__(256) router_topk(const float *__restrict__ logits, int T, int E, int k,
                                                   int32_t *__restrict__ idx, float *__restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  if (t >= T) return;
  const float *row = logits + (size_t)t * E;
  float v[kMaxPerLane];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = lane + i * kWave;
    v[i] = e < E ? row[e] : -INFINITY;
    if (e >= E) taken |= 1u << i;
  }
  float top_v = 0.f;
  float my_v = 0.f;
  int my_i = -1;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + i * kWave;
      if (!(taken >> i & 1u) && better(v[i], e, bv, bi)) { bv = v[i]; bi = e; }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off, kWave);
      const int oi = __shfl_xor(bi, off, kWave);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (j == 0) top_v = bv;
    if (lane == j) { my_v = bv; my_i = bi; }
  }
  // weights: softmax of the k chosen logits (max = the first one)
  const float ex = lane < k ? expf(my_v - top_v) : 0.f;
  float sum = ex;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, kWave);
  if (lane < k) {
    idx[(size_t)t * k + lane] = my_i;
    w[(size_t)t * k + lane] = ex / sum;
  }
}

}  // namespace

namespace moe {

hipError_t launch_router(const moe_ctx *c, const float *x, int T, const float *wr, const float *bias, float *logits,
                         int32_t *idx, float *w, hipStream_t s) {
  const int E = c->cfg.n_experts, d = c->cfg.d_model, k = c->cfg.top_k;
  if (T <= kMaxTSmall) {
    const int waves = (E + kEpw - 1) / kEpw;
    hipLaunchKernelGGL(router_logits_small, dim3((waves + 3) / 4), dim3(256), 0, s, x, T, d, wr, bias, E, logits);
  } else {
    hipLaunchKernelGGL(router_logits_gemm, dim3((E + kTn - 1) / kTn, (T + kTm - 1) / kTm), dim3(256), 0, s, x, T, d,
                       wr, bias, E, logits);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(router_topk, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, idx, w);
  return hipGetLastError();
}

}  // namespace moe
