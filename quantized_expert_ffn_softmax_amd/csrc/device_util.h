// Small device helpers shared by the single-workgroup kernels.
#pragma once
#include <hip/hip_runtime.h>

namespace moe {

// Exclusive scan of one int per thread over a 1024-thread block; *total gets
// the block sum.  Every thread of the block must call it.
__device__ inline int block_excl_scan_1024(int v, int *total, int *sh /* >= 17 ints */) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) sh[wave] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < 16; ++w) {
      const int t = sh[w];
      sh[w] = run;
      run += t;
    }
    sh[16] = run;
  }
  __syncthreads();
  const int res = sh[wave] + incl - v;
  *total = sh[16];
  __syncthreads();
  return res;
}

}  // namespace moe
