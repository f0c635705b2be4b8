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
  if (wave == 0) {
    // the 16 wave sums scanned by the first 16 lanes of wave 0 (shuffles,
    // not a serial chain of LDS reads)
    const int t = lane < 16 ? sh[lane] : 0;
    int run = t;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int o = __shfl_up(run, off, 64);
      if (lane >= off) run += o;
    }
    if (lane < 16) sh[lane] = run - t;
    if (lane == 15) sh[16] = run;
  }
  __syncthreads();
  const int res = sh[wave] + incl - v;
  *total = sh[16];
  __syncthreads();
  return res;
}

}  // namespace moe
