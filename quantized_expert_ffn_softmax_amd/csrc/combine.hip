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
// workgroup per token, two passes over the row (it stays in L2).
__device__ inline float block_sum_256(float v, float *part) {
  v = moe::wave_sum(v);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  const float tot = part[0] + part[1] + part[2] + part[3];
  __syncthreads();
  return tot;
}

// The row is read once into registers (d <= 8192: at most 8 float4 per
// thread), then reduced twice and written.
__global__ void __launch_bounds__(256) chain_norm_kernel(const float *__restrict__ out, int d,
                                                         float *__restrict__ x_next) {
  __shared__ float part[4];
  const int t = blockIdx.x;
  const int d4 = d / 4;
  const float4 *row = reinterpret_cast<const float4 *>(out + (size_t)t * d);
  float4 v[8];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = threadIdx.x + 256 * i;
    v[i] = c < d4 ? row[c] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
  const float mean = block_sum_256(s, part) / (float)d;
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (threadIdx.x + 256 * i < d4) {
      v[i].x -= mean;
      v[i].y -= mean;
      v[i].z -= mean;
      v[i].w -= mean;
      ss = fmaf(v[i].x, v[i].x, fmaf(v[i].y, v[i].y, fmaf(v[i].z, v[i].z, fmaf(v[i].w, v[i].w, ss))));
    }
  }
  const float inv = 1.0f / sqrtf(block_sum_256(ss, part) / (float)d + 1e-6f);
  float4 *o = reinterpret_cast<float4 *>(x_next + (size_t)t * d);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = threadIdx.x + 256 * i;
    if (c < d4) o[c] = make_float4(v[i].x * inv, v[i].y * inv, v[i].z * inv, v[i].w * inv);
  }
}

// combine_kernel then chain_norm_kernel in one workgroup per token, with the
// same arithmetic as the two: each thread combines the 8 float4 columns that
// chain_norm_kernel gives it (ascending j by fma, the shared row added last,
// as in combine_kernel), writes them to out, keeps them in registers and
// normalises them with chain_norm_kernel's reductions -- so out and x_next
// are bit for bit those of the two separate calls.
__global__ void __launch_bounds__(256) combine_norm_kernel(const float *__restrict__ y_pairs,
                                                           const float *__restrict__ w,
                                                           const float *__restrict__ y_shared, int k, int d,
                                                           float *__restrict__ out, float *__restrict__ x_next) {
  __shared__ float part[4];
  const int t = blockIdx.x, d4 = d / 4;
  const float4 *yp = reinterpret_cast<const float4 *>(y_pairs + (size_t)t * k * d);
  const float4 *ys = reinterpret_cast<const float4 *>(y_shared + (size_t)t * d);
  float4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  // two columns at a time, all their pair rows (16 at a time) requested
  // before the first fma: one memory round trip per 16 experts
#pragma unroll
  for (int i0 = 0; i0 < 8; i0 += 2) {
    if (threadIdx.x + 256 * i0 >= d4) continue;
    float4 acc[2], sh[2];
    acc[0] = acc[1] = make_float4(0.f, 0.f, 0.f, 0.f);
    auto chunk = [&](int j0) {
      float4 y[2][16];
      float wj[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int jj = min(j0 + j, k - 1);  // rows past k are loaded clamped and not used
        wj[j] = w[(size_t)t * k + jj];
#pragma unroll
        for (int h = 0; h < 2; ++h) y[h][j] = yp[(size_t)jj * d4 + min((int)threadIdx.x + 256 * (i0 + h), d4 - 1)];
      }
      if (j0 == 0) {
        // the shared rows, requested behind the pair rows (columns clamped,
        // unused past d4)
#pragma unroll
        for (int h = 0; h < 2; ++h) sh[h] = ys[min((int)threadIdx.x + 256 * (i0 + h), d4 - 1)];
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (j0 + j >= k) continue;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          acc[h].x = fmaf(wj[j], y[h][j].x, acc[h].x);
          acc[h].y = fmaf(wj[j], y[h][j].y, acc[h].y);
          acc[h].z = fmaf(wj[j], y[h][j].z, acc[h].z);
          acc[h].w = fmaf(wj[j], y[h][j].w, acc[h].w);
        }
      }
    };
    if (k <= 16) {
      chunk(0);  // straight-line: no loop header for the compiler to wait at
    } else {
      for (int j0 = 0; j0 < k; j0 += 16) chunk(j0);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = threadIdx.x + 256 * (i0 + h);
      if (c >= d4) continue;
      acc[h].x += sh[h].x;
      acc[h].y += sh[h].y;
      acc[h].z += sh[h].z;
      acc[h].w += sh[h].w;
      reinterpret_cast<float4 *>(out + (size_t)t * d)[c] = acc[h];
      v[i0 + h] = acc[h];
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
  const float mean = block_sum_256(s, part) / (float)d;
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (threadIdx.x + 256 * i < d4) {
      v[i].x -= mean;
      v[i].y -= mean;
      v[i].z -= mean;
      v[i].w -= mean;
      ss = fmaf(v[i].x, v[i].x, fmaf(v[i].y, v[i].y, fmaf(v[i].z, v[i].z, fmaf(v[i].w, v[i].w, ss))));
    }
  }
  const float inv = 1.0f / sqrtf(block_sum_256(ss, part) / (float)d + 1e-6f);
  float4 *o = reinterpret_cast<float4 *>(x_next + (size_t)t * d);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = threadIdx.x + 256 * i;
    if (c < d4) o[c] = make_float4(v[i].x * inv, v[i].y * inv, v[i].z * inv, v[i].w * inv);
  }
}

}  // namespace

namespace moe {

hipError_t launch_combine_norm(const float *y_pairs, const float *w, const float *y_shared, int T, int k, int d,
                               float *out, float *x_next, hipStream_t s) {
  hipLaunchKernelGGL(combine_norm_kernel, dim3(T), dim3(256), 0, s, y_pairs, w, y_shared, k, d, out, x_next);
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
  hipLaunchKernelGGL(chain_norm_kernel, dim3(T), dim3(256), 0, s, out, d, x_next);
  return hipGetLastError();
}

}  // namespace moe
