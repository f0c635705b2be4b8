// Weighted combine of the k routed expert outputs plus the shared expert,
// and the normalisation helper that chains stacked layers.
//
// The shared expert is added ungated after the routed terms ("另加 1 个共享
// 专家" -- one shared expert on top of the 10 routed ones: "一张 RTX 4090
// 跑千亿模型，Strata 实测 155 tok/s", section 如何做到：三层存储).
#include "moe_internal.h"

namespace {

// out[t][c..c+3] = sum_j w[t][j] * y_pairs[t*k+j][c..c+3] + y_shared[t][c..c+3]
__global__ void __launch_bounds__(256) combine_kernel(const float *__restrict__ y_pairs, const float *__restrict__ w,
                                                      const float *__restrict__ y_shared, int T, int k, int d,
                                                      float *__restrict__ out) {
  const int d4 = d / 4;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * d4) return;
  const int t = i / d4, c4 = i % d4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const float wj = w[(size_t)t * k + j];
    const float4 y = reinterpret_cast<const float4 *>(y_pairs + ((size_t)t * k + j) * d)[c4];
    acc.x = fmaf(wj, y.x, acc.x);
    acc.y = fmaf(wj, y.y, acc.y);
    acc.z = fmaf(wj, y.z, acc.z);
    acc.w = fmaf(wj, y.w, acc.w);
  }
  const float4 s = reinterpret_cast<const float4 *>(y_shared + (size_t)t * d)[c4];
  acc.x += s.x;
  acc.y += s.y;
  acc.z += s.z;
  acc.w += s.w;
  reinterpret_cast<float4 *>(out + (size_t)t * d)[c4] = acc;
}

// x_next[t] = c / sqrt(mean(c^2) + 1e-6) with c = out[t] - mean(out[t]); one
// workgroup per token, two passes over the row (it stays in L2).
__device__ inline float block_sum_256(float v, float *part) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  const float tot = part[0] + part[1] + part[2] + part[3];
  __syncthreads();
  return tot;
}

__global__ void __launch_bounds__(256) chain_norm_kernel(const float *__restrict__ out, int d,
                                                         float *__restrict__ x_next) {
  __shared__ float part[4];
  const int t = blockIdx.x;
  const float *row = out + (size_t)t * d;
  float s = 0.f;
  for (int c = threadIdx.x; c < d; c += blockDim.x) s += row[c];
  const float mean = block_sum_256(s, part) / (float)d;
  float ss = 0.f;
  for (int c = threadIdx.x; c < d; c += blockDim.x) {
    const float v = row[c] - mean;
    ss = fmaf(v, v, ss);
  }
  const float inv = 1.0f / sqrtf(block_sum_256(ss, part) / (float)d + 1e-6f);
  for (int c = threadIdx.x; c < d; c += blockDim.x) x_next[(size_t)t * d + c] = (row[c] - mean) * inv;
}

}  // namespace

namespace moe {

hipError_t launch_combine(const float *y_pairs, const float *w, const float *y_shared, int T, int k, int d, float *out,
                          hipStream_t s) {
  const int n = T * (d / 4);
  hipLaunchKernelGGL(combine_kernel, dim3((n + 255) / 256), dim3(256), 0, s, y_pairs, w, y_shared, T, k, d, out);
  return hipGetLastError();
}

hipError_t launch_chain_norm(const float *out, int T, int d, float *x_next, hipStream_t s) {
  hipLaunchKernelGGL(chain_norm_kernel, dim3(T), dim3(256), 0, s, out, d, x_next);
  return hipGetLastError();
}

}  // namespace moe
