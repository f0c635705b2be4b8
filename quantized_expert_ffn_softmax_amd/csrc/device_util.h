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

// Inclusive scan of one int per lane over a wave64, in DPP moves (no LDS
// round trips): shifts by 1, 2, 4 and 8 inside each 16-lane row, then the
// row totals carried across rows by the row_bcast:15 and row_bcast:31
// broadcasts.  Lanes a move does not reach keep the 0 passed as `old`.
// Every lane of the wave must be active (a DPP move reads inactive lanes'
// stale registers): call it outside divergent branches.
__device__ inline int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1 and 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2 and 3
  return v;
}

template <int CTRL, int ROWS>
__device__ inline float dpp_move(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWS, 0xf, false));
}

// Sum of one float per lane over a wave64, in the same DPP moves as
// wave_incl_scan (a fixed tree order); the total is returned to every lane.
// Every lane of the wave must be active, as for wave_incl_scan.
__device__ inline float wave_sum(float v) {
  v += dpp_move<0x111, 0xf>(v);  // row_shr:1
  v += dpp_move<0x112, 0xf>(v);  // row_shr:2
  v += dpp_move<0x114, 0xf>(v);  // row_shr:4
  v += dpp_move<0x118, 0xf>(v);  // row_shr:8
  v += dpp_move<0x142, 0xa>(v);  // row_bcast:15
  v += dpp_move<0x143, 0xc>(v);  // row_bcast:31
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Top-k order of router logits as one 64-bit key: (the logit mapped to an
// order-preserving uint32) << 32 | ~expert, so a larger key is a larger logit,
// and equal logits order the lower expert index first; -0 and +0 are equal.
// Every expert of a row has a distinct key; 0 orders after every real key.
__device__ inline uint64_t order_key(float v, int e) {
  const uint32_t b = v == 0.f ? 0u : __float_as_uint(v);
  const uint32_t mono = (b & 0x80000000u) ? ~b : (b | 0x80000000u);  // larger float -> larger uint
  return ((uint64_t)mono << 32) | (uint32_t)~(uint32_t)e;
}
__device__ inline float key_logit(uint64_t key) {
  const uint32_t mono = (uint32_t)(key >> 32);
  return __uint_as_float((mono & 0x80000000u) ? (mono & 0x7fffffffu) : ~mono);
}
__device__ inline int key_expert(uint64_t key) { return (int)~(uint32_t)key; }

}  // namespace moe
