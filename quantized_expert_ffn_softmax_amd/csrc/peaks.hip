// Achievable-peak probes of the device the layer runs on: a streaming HBM
// read and a loop of dense fp16 MFMAs.  The layer's
// roofline fractions are quoted against the data-sheet peaks and against
// these measured ones (the pages give no hardware figure for this part).
#include "moe_internal.h"

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;  // 16-byte loads in flight per thread

// Every byte of [buf, buf + n16 * 16) is loaded once with 16-byte loads
// (grid-stride in groups of kReadUnroll per thread, all requested before any
// is used).  The XOR of the data is stored only if it equals a value no data
// produces in practice, so the loads stay live and nothing is written.
__global__ void __launch_bounds__(kReadThreads) hbm_read_kernel(const uint4 *__restrict__ buf, uint64_t n16,
                                                                uint32_t *__restrict__ sink) {
  const uint64_t nth = (uint64_t)gridDim.x * kReadThreads;
  uint64_t i = (uint64_t)blockIdx.x * kReadThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kReadUnroll - 1) * nth < n16; i += kReadUnroll * nth) {
    uint4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = buf[i + u * nth];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += nth) {
    const uint4 v = buf[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

typedef float f16v __attribute__((ext_vector_type(16)));

// Each wave runs `iters` rounds of 4 independent v_mfma_f32_32x32x16_f16 on
// register operands (32,768 flops each; four chains are more than its
// latency needs).  The operands are made opaque every round so that no result
// is loop-invariant; the sums are stored only under a condition no run meets,
// which keeps them live.  (This shape compiles to a loop of the four MFMAs
// alone; eight 16x16x32 chains were compiled with accumulator copies between
// the MFMAs, which measured the copies instead.)
__global__ void __launch_bounds__(256) mfma_loop_kernel(int iters, float *__restrict__ sink) {
  h8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)(0.001f * (threadIdx.x + i));
    b[i] = (_Float16)(0.002f * (i - (int)threadIdx.x % 7));
  }
  f16v c0, c1, c2, c3;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    c0[i] = 0.f;
    c1[i] = 1.f;
    c2[i] = 2.f;
    c3[i] = 3.f;
  }
  for (int it = 0; it < iters; ++it) {
    asm volatile("" : "+v"(a));
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c3, 0, 0, 0);
  }
  const float s = c0[0] + c1[5] + c2[10] + c3[15];
  if (s == -12345.678f) sink[blockIdx.x] = s;
}

}  // namespace

extern "C" moe_status moe_peak_hbm_read(const void *buf, uint64_t bytes, uint32_t *sink, int32_t n_blocks,
                                        void *stream) {
  MOE_CHECK(buf && sink && n_blocks >= 1 && n_blocks <= (1 << 20), MOE_ERR_INVALID,
            "moe_peak_hbm_read: null buffer or sink, or n_blocks outside 1..2^20");
  MOE_CHECK(((uintptr_t)buf % 16) == 0 && bytes % 16 == 0, MOE_ERR_ALIGN,
            "moe_peak_hbm_read: buffer and size must be multiples of 16 bytes");
  hipLaunchKernelGGL(hbm_read_kernel, dim3((unsigned)n_blocks), dim3(kReadThreads), 0, (hipStream_t)stream,
                     (const uint4 *)buf, (uint64_t)(bytes / 16), sink);
  MOE_HIP(hipGetLastError());
  return MOE_OK;
}

extern "C" moe_status moe_peak_mfma_f16(int32_t iters, int32_t n_blocks, float *sink, void *stream) {
  MOE_CHECK(sink && iters >= 1 && n_blocks >= 1 && n_blocks <= (1 << 20), MOE_ERR_INVALID,
            "moe_peak_mfma_f16: null sink, iters < 1 or n_blocks outside 1..2^20");
  hipLaunchKernelGGL(mfma_loop_kernel, dim3((unsigned)n_blocks), dim3(256), 0, (hipStream_t)stream, iters, sink);
  MOE_HIP(hipGetLastError());
  return MOE_OK;
}
