// Router: logits = x W_r^T + b in fp32, then per token the top-k by
// (logit desc, index asc) and weights renormalised over the k chosen.
//
// The pages fix the shape (10 of 512 experts per token plus one shared
// expert: "一张 RTX 4090 跑千亿模型，Strata 实测 155 tok/s", section
// 如何做到：三层存储); the scoring function is the softmax reading.
#include "device_util.h"
#include "moe_internal.h"
#include "topk_small.h"

namespace {

constexpr int kWave = 64;

// --- logits, many tokens: fp16 MFMA on split operands.  Each fp32 operand
// v is carried as hi = fp16(v) and lo = fp16(v - hi) (v = hi + lo to ~2^-22
// relative), and a 32-column K step of a 16 x 16 block takes three
// v_mfma_f32_16x16x32_f16: W_hi x_hi + W_hi x_lo + W_lo x_hi (the dropped
// W_lo x_lo is ~2^-22 of a product), every product exact in the fp32
// accumulation.  fp16 MFMA runs 16x the fp32 MFMA rate on this part.
// A workgroup computes 128 experts x 128 tokens; wave (we, wt) of its 2 x 2
// waves takes experts 64 we .. and tokens 64 wt .. as 4 x 4 blocks of 16 x 16.
// K runs in stages of 32 columns through LDS (double-buffered; the next
// stage is loaded into registers during the MFMAs).  An LDS row of a stage
// holds 32 hi halves then 32 lo halves (144-byte pitch).
// MFMA operands: A = W[expert 16 b + m][k], B = x[token 16 c + m][k], lane
// (m, g) supplying k = 8 g .. 8 g + 7; D: lane (m, g) holds experts
// 16 b + 4 g + i, token 16 c + m.
constexpr int kGm = 128, kGk = 32, kGpb = 144;  // tile (both sides), K stage, LDS row pitch in bytes
constexpr int kGv = kGm * kGk / 4 / 256;        // float4 loads per thread per matrix and stage

typedef float f4g __attribute__((ext_vector_type(4)));
typedef _Float16 h8g __attribute__((ext_vector_type(8)));
typedef _Float16 h4g __attribute__((ext_vector_type(4)));

__device__ inline void stage_load(const float *__restrict__ src, int rows, int r0, int d, int k0, int tid,
                                  float4 (&v)[kGv]) {
#pragma unroll
  for (int i = 0; i < kGv; ++i) {
    const int q = tid + 256 * i;  // float4 index: row q / 8, columns 4 (q % 8) ..
    const int gr = r0 + (q >> 3);
    v[i] = gr < rows ? *reinterpret_cast<const float4 *>(src + (size_t)gr * d + k0 + 4 * (q & 7))
                     : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

__device__ inline void stage_store(const float4 (&v)[kGv], int tid, uint8_t *__restrict__ lds) {
#pragma unroll
  for (int i = 0; i < kGv; ++i) {
    const int q = tid + 256 * i;
    const float f[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    h4g hi, lo;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      hi[j] = (_Float16)f[j];
      lo[j] = (_Float16)(f[j] - (float)hi[j]);
    }
    uint8_t *o = lds + (q >> 3) * kGpb + 8 * (q & 7);
    *reinterpret_cast<h4g *>(o) = hi;
    *reinterpret_cast<h4g *>(o + 64) = lo;
  }
}

__global__ void __launch_bounds__(256) router_logits_gemm(const float *__restrict__ x, int T, int d,
                                                          const float *__restrict__ wr,
                                                          const float *__restrict__ bias, int E,
                                                          float *__restrict__ logits) {
  __shared__ __attribute__((aligned(16))) uint8_t lw[2][kGm * kGpb];
  __shared__ __attribute__((aligned(16))) uint8_t lx[2][kGm * kGpb];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, g = lane >> 4;
  const int we = wave >> 1, wt = wave & 1;
  const int e0 = blockIdx.x * kGm, t0 = blockIdx.y * kGm;
  f4g acc[4][4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[b][c] = (f4g){0.f, 0.f, 0.f, 0.f};
  const int nst = d / kGk;
  float4 vw[kGv], vx[kGv];
  stage_load(wr, E, e0, d, 0, tid, vw);
  stage_load(x, T, t0, d, 0, tid, vx);
  stage_store(vw, tid, lw[0]);
  stage_store(vx, tid, lx[0]);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int cur = st & 1;
    const bool more = st + 1 < nst;
    if (more) {
      stage_load(wr, E, e0, d, (st + 1) * kGk, tid, vw);
      stage_load(x, T, t0, d, (st + 1) * kGk, tid, vx);
    }
    h8g ah[4], al[4], bh[4], bl[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint8_t *pa = lw[cur] + (64 * we + 16 * b + m) * kGpb + 16 * g;
      const uint8_t *pb = lx[cur] + (64 * wt + 16 * b + m) * kGpb + 16 * g;
      ah[b] = *reinterpret_cast<const h8g *>(pa);
      al[b] = *reinterpret_cast<const h8g *>(pa + 64);
      bh[b] = *reinterpret_cast<const h8g *>(pb);
      bl[b] = *reinterpret_cast<const h8g *>(pb + 64);
    }
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        acc[b][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[b], bh[c], acc[b][c], 0, 0, 0);
        acc[b][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[b], bl[c], acc[b][c], 0, 0, 0);
        acc[b][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[b], bh[c], acc[b][c], 0, 0, 0);
      }
    if (more) {
      // the other buffer was last read in stage st - 1, before the barrier that ended it
      stage_store(vw, tid, lw[cur ^ 1]);
      stage_store(vx, tid, lx[cur ^ 1]);
    }
    __syncthreads();
  }
  // D: lane (m, g) of block (b, c) holds experts e0 + 64 we + 16 b + 4 g + i, token t0 + 64 wt + 16 c + m
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int t = t0 + 64 * wt + 16 * c + m;
    if (t >= T) continue;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = e0 + 64 * we + 16 * b + 4 * g + i;
        if (e < E) logits[(size_t)t * E + e] = acc[b][c][i] + (bias ? bias[e] : 0.f);
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
  // two chunks per step, both requested before the first MFMA (a wave
  // usually has exactly two: one memory round trip instead of two)
  for (int ch = c0 + wave; ch < c1; ch += 2 * kRouteWaves) {
    const int ch2 = ch + kRouteWaves;
    const bool has2 = ch2 < c1;  // wave-uniform
    const int col = ch * 16 + 4 * g, col2 = (has2 ? ch2 : ch) * 16 + 4 * g;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a, a2 = a, b2 = a;
    if (e < E) {
      a = *reinterpret_cast<const float4 *>(wrow + col);
      a2 = *reinterpret_cast<const float4 *>(wrow + col2);
    }
    if (tok < T) {
      b = *reinterpret_cast<const float4 *>(xrow + col);
      b2 = *reinterpret_cast<const float4 *>(xrow + col2);
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, acc, 0, 0, 0);
    if (has2) {
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a2.x, b2.x, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a2.y, b2.y, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a2.z, b2.z, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a2.w, b2.w, acc, 0, 0, 0);
    }
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

// One workgroup per token (topk_small.h).
__global__ void __launch_bounds__(1024) router_finish_small(const float *__restrict__ part, int T, int E, int KS,
                                                            const float *__restrict__ bias, int k,
                                                            float *__restrict__ logits, int32_t *__restrict__ idx,
                                                            float *__restrict__ w) {
  moe::finish_token(part, T, blockIdx.x, E, KS, bias, k, logits, idx, w);
}

}  // namespace

namespace moe {

hipError_t launch_router_partials(const moe_ctx *c, const float *x, int T, const float *wr, hipStream_t s) {
  const int E = c->cfg.n_experts, d = c->cfg.d_model;
  if (T > c->route_small_t) return hipErrorInvalidValue;
  const int KS = c->route_ks;
  const int n_tg = (T + 15) / 16;
  hipLaunchKernelGGL(router_logits_mfma, dim3(n_tg * ((E + 15) / 16) * KS), dim3(64 * kRouteWaves), 0, s, x, T, d, wr,
                     E, KS, c->route_part);
  return hipGetLastError();
}

hipError_t launch_router(const moe_ctx *c, const float *x, int T, const float *wr, const float *bias, float *logits,
                         int32_t *idx, float *w, hipStream_t s) {
  const int E = c->cfg.n_experts, d = c->cfg.d_model, k = c->cfg.top_k;
  if (T <= c->route_small_t) {
    hipError_t e = launch_router_partials(c, x, T, wr, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(router_finish_small, dim3(T), dim3((E + 63) / 64 * 64), 0, s, c->route_part, T, E,
                       c->route_ks, bias, k, logits, idx, w);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(router_logits_gemm, dim3((E + kGm - 1) / kGm, (T + kGm - 1) / kGm), dim3(256), 0, s, x, T, d, wr,
                     bias, E, logits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(router_topk, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, idx, w);
  return hipGetLastError();
}

}  // namespace moe
