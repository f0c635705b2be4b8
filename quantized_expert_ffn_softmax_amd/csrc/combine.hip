// Weighted combine of the k routed expert outputs plus the shared expert,
// and the normalisation helper that chains stacked layers.
//
// The shared expert is added ungated after the routed terms ("另加 1 个共享
// 专家" -- one shared expert on top of the 10 routed ones: "一张 RTX 4090
// 跑千亿模型，Strata 实测 155 tok/s", section 如何做到：三层存储).
#include "device_util.h"
#include "moe_internal.h"

namespace {

// out[t][c..c+3] = sum_j w[t][j] * y_pairs[t*k+j][c..c+3] + y_shared[t][c..c+3]
// The k rows are requested 8 at a time before any is used (k <= 32), and the
// sum runs in ascending j with the shared row added last.
__global__ void __launch_bounds__(64) combine_kernel(const float *__restrict__ y_pairs, const float *__restrict__ w,
                                                      const float *__restrict__ y_shared, int T, int k, int d,
                                                      float *__restrict__ out) {
  const int d4 = d / 4;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * d4) return;
  const int t = i / d4, c4 = i % d4;
  const float4 *yp = reinterpret_cast<const float4 *>(y_pairs + (size_t)t * k * d) + c4;
  const float4 s = reinterpret_cast<const float4 *>(y_shared + (size_t)t * d)[c4];
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j0 = 0; j0 < k; j0 += 8) {
    float4 y[8];
    float wj[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool ok = j0 + j < k;
      y[j] = ok ? yp[(size_t)(j0 + j) * d4] : make_float4(0.f, 0.f, 0.f, 0.f);
      wj[j] = ok ? w[(size_t)t * k + j0 + j] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      acc.x = fmaf(wj[j], y[j].x, acc.x);
      acc.y = fmaf(wj[j], y[j].y, acc.y);
      acc.z = fmaf(wj[j], y[j].z, acc.z);
      acc.w = fmaf(wj[j], y[j].w, acc.w);
    }
  }
  acc.x += s.x;
  acc.y += s.y;
  acc.z += s.z;
  acc.w += s.w;
  reinterpret_cast<float4 *>(out + (size_t)t * d)[c4] = acc;
}

// x_next[t] = c / sqrt(mean(c^2) + 1e-6) with c = out[t] - mean(out[t]); one
// workgroup of 512 threads per token, thread i holding float4 columns
// i + 512 j (d <= 8192: j < 4), the row held in registers between the two
// reductions.  chain_norm_kernel and combine_norm_kernel share this mapping
// and the reduction order, so they give the same bits.
constexpr int kNormThreads = 512;
constexpr int kNormCols = 4;  // float4 columns per thread at d = 8192

__device__ inline float block_sum_512(float v, float *part) {
  v = moe::wave_sum(v);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  float tot = part[0];
#pragma unroll
  for (int i = 1; i < kNormThreads / 64; ++i) tot += part[i];
  __syncthreads();
  return tot;
}

__device__ inline void normalise_row(float4 (&v)[kNormCols], int d, float *part, float *__restrict__ x_next) {
  const int d4 = d / 4;
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kNormCols; ++i) s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
  const float mean = block_sum_512(s, part) / (float)d;
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kNormCols; ++i) {
    if (threadIdx.x + kNormThreads * i < d4) {
      v[i].x -= mean;
      v[i].y -= mean;
      v[i].z -= mean;
      v[i].w -= mean;
      ss = fmaf(v[i].x, v[i].x, fmaf(v[i].y, v[i].y, fmaf(v[i].z, v[i].z, fmaf(v[i].w, v[i].w, ss))));
    }
  }
  const float inv = 1.0f / sqrtf(block_sum_512(ss, part) / (float)d + 1e-6f);
  float4 *o = reinterpret_cast<float4 *>(x_next);
#pragma unroll
  for (int i = 0; i < kNormCols; ++i) {
    const int c = threadIdx.x + kNormThreads * i;
    if (c < d4) o[c] = make_float4(v[i].x * inv, v[i].y * inv, v[i].z * inv, v[i].w * inv);
  }
}

__global__ void __launch_bounds__(kNormThreads) chain_norm_kernel(const float *__restrict__ out, int d,
                                                                  float *__restrict__ x_next) {
  __shared__ float part[kNormThreads / 64];
  const int t = blockIdx.x, d4 = d / 4;
  const float4 *row = reinterpret_cast<const float4 *>(out + (size_t)t * d);
  float4 v[kNormCols];
#pragma unroll
  for (int i = 0; i < kNormCols; ++i) {
    const int c = threadIdx.x + kNormThreads * i;
    v[i] = c < d4 ? row[c] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  normalise_row(v, d, part, x_next + (size_t)t * d);
}

// combine_kernel then chain_norm_kernel in one workgroup per token, with the
// same arithmetic as the two: each of the thread's columns is combined as
// combine_kernel does it (ascending j by fma from 0, the shared row added
// last) and written to out, then the row is normalised as chain_norm_kernel
// does it -- so out and x_next are bit for bit those of the two calls.  A
// column's pair rows (16 at a time) and its shared row are requested before
// the first fma: at d_model 2048 and k <= 16 one memory round trip per token.
__global__ void __launch_bounds__(kNormThreads) combine_norm_kernel(const float *__restrict__ y_pairs,
                                                                    const float *__restrict__ w,
                                                                    const float *__restrict__ y_shared, int k, int d,
                                                                    float *__restrict__ out,
                                                                    float *__restrict__ x_next) {
  __shared__ float part[kNormThreads / 64];
  const int t = blockIdx.x, d4 = d / 4;
  const float4 *yp = reinterpret_cast<const float4 *>(y_pairs + (size_t)t * k * d);
  const float4 *ys = reinterpret_cast<const float4 *>(y_shared + (size_t)t * d);
  float4 v[kNormCols];
#pragma unroll
  for (int i = 0; i < kNormCols; ++i) {
    v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    const int c = threadIdx.x + kNormThreads * i;
    if (c >= d4) continue;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f), sh = acc;
    for (int j0 = 0; j0 < k; j0 += 16) {
      float4 y[16];
      float wj[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int jj = min(j0 + j, k - 1);  // rows past k are loaded clamped and not used
        wj[j] = w[(size_t)t * k + jj];
        y[j] = yp[(size_t)jj * d4 + c];
      }
      if (j0 == 0) sh = ys[c];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (j0 + j >= k) continue;
        acc.x = fmaf(wj[j], y[j].x, acc.x);
        acc.y = fmaf(wj[j], y[j].y, acc.y);
        acc.z = fmaf(wj[j], y[j].z, acc.z);
        acc.w = fmaf(wj[j], y[j].w, acc.w);
      }
    }
    acc.x += sh.x;
    acc.y += sh.y;
    acc.z += sh.z;
    acc.w += sh.w;
    reinterpret_cast<float4 *>(out + (size_t)t * d)[c] = acc;
    v[i] = acc;
  }
  normalise_row(v, d, part, x_next + (size_t)t * d);
}

}  // namespace

namespace moe {

hipError_t launch_combine_norm(const float *y_pairs, const float *w, const float *y_shared, int T, int k, int d,
                               float *out, float *x_next, hipStream_t s) {
  hipLaunchKernelGGL(combine_norm_kernel, dim3(T), dim3(kNormThreads), 0, s, y_pairs, w, y_shared, k, d, out, x_next);
  return hipGetLastError();
}


hipError_t launch_combine(const float *y_pairs, const float *w, const float *y_shared, int T, int k, int d, float *out,
                          hipStream_t s) {
  // one wave per workgroup: few tokens still spread their rows over many CUs
  const int n = T * (d / 4);
  hipLaunchKernelGGL(combine_kernel, dim3((n + 63) / 64), dim3(64), 0, s, y_pairs, w, y_shared, T, k, d, out);
  return hipGetLastError();
}

hipError_t launch_chain_norm(const float *out, int T, int d, float *x_next, hipStream_t s) {
  hipLaunchKernelGGL(chain_norm_kernel, dim3(T), dim3(kNormThreads), 0, s, out, d, x_next);
  return hipGetLastError();
}

}  // namespace moe
