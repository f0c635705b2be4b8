// Router: logits = x W_r^T + b in fp32, then per token the top-k by
// (logit desc, index asc) and weights renormalised over the k chosen.
//
// The pages fix the shape (10 of 512 experts per token plus one shared
// expert: "一张 RTX 4090 跑千亿模型，Strata 实测 155 tok/s", section
// 如何做到：三层存储); the scoring function is the softmax reading.
#include "moe_internal.h"

namespace {

constexpr int kWave = 64;

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

// top-k of one token's row by one wave
__device__ void topk_row(const float *__restrict__ row, int E, int k, int32_t *__restrict__ idx_row,
                         float *__restrict__ w_row) {
  const int lane = threadIdx.x & 63;
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
    idx_row[lane] = my_i;
    w_row[lane] = ex / sum;
  }
}

__global__ void __launch_bounds__(256) router_topk(const float *__restrict__ logits, int T, int E, int k,
                                                   int32_t *__restrict__ idx, float *__restrict__ w) {
  const int t = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  if (t >= T) return;
  topk_row(logits + (size_t)t * E, E, k, idx + (size_t)t * k, w + (size_t)t * k);
}

// --- decode-size batches (T <= 64): logits on fp32 MFMA.  Workgroup
// (tg, eg, ks) covers tokens 16 tg .. 16 tg + 15, experts 16 eg .. 16 eg + 15
// and the ks-th of KS slices of the columns; each of its waves takes every
// kRouteWaves-th chunk of 16 columns of that slice.  v_mfma_f32_16x16x4_f32
// with lane (m, g): A = W[16 eg + m][col], B = x[token 16 tg + m][col],
// col = chunk + 4 g + i for the i-th of the 4 MFMAs of a chunk; D: lane holds
// experts 4 g + i, token 16 tg + m.
// Wave partials are added in wave order into part[ks][t][e]; a second,
// single-workgroup kernel adds the KS slices in order, adds the bias and runs
// the top-k (the kernel boundary is the cross-workgroup handoff: an in-kernel
// one needs device-scope fences that write back and invalidate L2).
typedef float f4v __attribute__((ext_vector_type(4)));
constexpr int kRouteWaves = 8;

__global__ void __launch_bounds__(64 * kRouteWaves) router_logits_mfma(const float *__restrict__ x, int T, int d,
                                                                     const float *__restrict__ wr, int E, int KS,
                                                                     float *__restrict__ part) {
  __shared__ float red[kRouteWaves][64][4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = lane & 15, g = lane >> 4;
  const int n_eg = (E + 15) / 16;
  const int tg = blockIdx.x / (n_eg * KS), eg = (blockIdx.x / KS) % n_eg, ks = blockIdx.x % KS;
  const int e = 16 * eg + m, tok = 16 * tg + m;
  const int nchunk = d / 16;
  const int c0 = (int)((long)nchunk * ks / KS), c1 = (int)((long)nchunk * (ks + 1) / KS);
  f4v acc = {0.f, 0.f, 0.f, 0.f};
  const float *wrow = wr + (size_t)(e < E ? e : 0) * d;
  const float *xrow = x + (size_t)(tok < T ? tok : 0) * d;
  for (int ch = c0 + wave; ch < c1; ch += kRouteWaves) {
    const int col = ch * 16 + 4 * g;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
    if (e < E) a = *reinterpret_cast<const float4 *>(wrow + col);
    if (tok < T) b = *reinterpret_cast<const float4 *>(xrow + col);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, acc, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][lane][i] = acc[i];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = red[0][lane][i];
      for (int ww = 1; ww < kRouteWaves; ++ww) v += red[ww][lane][i];
      const int ee = 16 * eg + 4 * g + i, t = tok;
      if (ee < E && t < T) part[((size_t)ks * T + t) * E + ee] = v;
    }
  }
}

// One workgroup per token: logits = sum of the KS slices (in order) + bias,
// then the top-k by rank, where an expert's rank is the number of experts
// ordered before it by (logit desc, index asc).  The order is that of one
// 64-bit key, (logit mapped to an order-preserving uint32) << 32 | ~index, so
// each comparison is one v_cmp_gt_u64.  Two passes: each wave ranks its 64
// experts among themselves; an expert of global rank < k has wave rank < k,
// so only those candidates (k per wave) are ranked against each other, and
// for a candidate in the global top-k that rank is its global rank (every
// expert ordered before it is a candidate too).  Weights: softmax of the k
// chosen logits.
__device__ inline uint64_t order_key(float v, int e) {
  const uint32_t b = v == 0.f ? 0u : __float_as_uint(v);  // -0 and +0 are equal logits
  const uint32_t mono = (b & 0x80000000u) ? ~b : (b | 0x80000000u);  // larger float -> larger uint
  return ((uint64_t)mono << 32) | (uint32_t)~(uint32_t)e;               // equal logits: lower index larger
}

__global__ void __launch_bounds__(1024) router_finish_small(const float *__restrict__ part, int T, int E, int KS,
                                                            const float *__restrict__ bias, int k,
                                                            float *__restrict__ logits, int32_t *__restrict__ idx,
                                                            float *__restrict__ w) {
  __shared__ uint64_t lk[1024];
  __shared__ uint64_t ck[16 * 32];
  __shared__ float top[32];
  const int t = blockIdx.x, e = threadIdx.x, wave = e >> 6;
  float v = -INFINITY;
  if (e < E) {
    // the KS partial sums, requested 8 at a time and added in slice order
    v = 0.f;
    for (int q0 = 0; q0 < KS; q0 += 8) {
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = q0 + i < KS ? part[((size_t)(q0 + i) * T + t) * E + e] : 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) v += p[i];
    }
    v += bias ? bias[e] : 0.f;
    logits[(size_t)t * E + e] = v;
  }
  const uint64_t key = e < E ? order_key(v, e) : 0ull;  // lanes past E order after everything
  lk[e] = key;
  const int nw = blockDim.x / 64;
  for (int i = e; i < nw * k; i += blockDim.x) ck[i] = 0ull;  // empty candidate: orders before nothing
  __syncthreads();
  // pass 1: rank inside the wave
  int r1 = 0;
#pragma unroll 16
  for (int o = 0; o < 64; ++o) r1 += lk[wave * 64 + o] > key;
  if (e < E && r1 < k) ck[wave * k + r1] = key;
  __syncthreads();
  // pass 2: rank among the candidates
  int r = k;
  if (e < E && r1 < k) {
    r = 0;
    for (int i = 0; i < nw * k; ++i) r += ck[i] > key;
    if (r < k) top[r] = v;
  }
  __syncthreads();
  if (r < k) {
    const float m = top[0];
    float sum = 0.f;
    for (int j = 0; j < k; ++j) sum += expf(top[j] - m);
    idx[(size_t)t * k + r] = e;
    w[(size_t)t * k + r] = expf(v - m) / sum;
  }
}

}  // namespace

namespace moe {

hipError_t launch_router(const moe_ctx *c, const float *x, int T, const float *wr, const float *bias, float *logits,
                         int32_t *idx, float *w, hipStream_t s) {
  const int E = c->cfg.n_experts, d = c->cfg.d_model, k = c->cfg.top_k;
  if (T <= c->route_small_t) {
    const int KS = c->route_ks;
    const int n_tg = (T + 15) / 16;
    hipLaunchKernelGGL(router_logits_mfma, dim3(n_tg * ((E + 15) / 16) * KS), dim3(64 * kRouteWaves), 0, s, x, T, d,
                       wr, E, KS, c->route_part);
    hipLaunchKernelGGL(router_finish_small, dim3(T), dim3((E + 63) / 64 * 64), 0, s, c->route_part, T, E, KS, bias,
                       k, logits, idx, w);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(router_logits_gemm, dim3((E + kTn - 1) / kTn, (T + kTm - 1) / kTm), dim3(256), 0, s, x, T, d, wr,
                     bias, E, logits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(router_topk, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, idx, w);
  return hipGetLastError();
}

}  // namespace moe
