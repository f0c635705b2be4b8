// Activation records of the decode path: values in MFMA step order, each
// split into two fp16 halves (hi, lo = value - hi) so that a pair of fp16
// MFMAs reproduces the fp32 value to about 2^-22.
//
// For one token and one matrix with nsb 160-column superblocks the record
// holds, for each superblock S and step t (0..19), 8 hi halves then 8 lo
// halves; the 8 halves are the columns of code pairs p = 4t..4t+3, pair p
// being columns (c, c+5) with c = 160 S + 10 (p / 5) + p % 5 -- the two codes
// that share the low and high half of one packed word.
//
// Code slot j = p % 5 of a pair is extracted in place, without shifting the
// word down: slots 0..2 from the word itself, slots 3..4 from word >> 9, so
// the weight reaches the MFMA multiplied by f = 2^(3 (j mod 3)) (1, 8 or 64).
// The record stores the activation divided by the same f, an exact rescale
// by a power of two, so every product keeps its value.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_internal.h"

namespace moe {

__host__ __device__ constexpr int pair_col(int p) { return 10 * (p / 5) + p % 5; }
// 1 / f for pair p (see above)
__host__ __device__ constexpr float pair_inv_f(int p) {
  return (p % 5) % 3 == 0 ? 1.0f : ((p % 5) % 3 == 1 ? 0.125f : 0.015625f);
}

// position (in halves) of column c inside one token's record (its lo half
// sits 8 further) and the factor 1/f the value is stored with
__device__ inline int rec_pos(int c, float &inv_f) {
  const int S = c / kSbCols;
  const int lc = c - S * kSbCols;
  const int w = lc / 10, j = lc - 10 * w;
  const int p = 5 * w + (j % 5);
  inv_f = pair_inv_f(p);
  return S * kSteps * 16 + (p >> 2) * 16 + 2 * (p & 3) + j / 5;
}

// record of x [T][d] (fp32), work split over `nth` threads with index `tid`
__device__ inline void build_xrec_range(const float *__restrict__ x, int T, int d, int nsb, uint16_t *__restrict__ xrec,
                                        int xrec_h, int tid, int nth) {
  const int per_tok = nsb * kSteps * 8;  // (S, t, 8 value slots)
  for (int i = tid; i < T * per_tok; i += nth) {
    const int tk = i / per_tok;
    const int r = i - tk * per_tok;
    const int S = r / (kSteps * 8);
    const int r2 = r - S * kSteps * 8;
    const int t = r2 >> 3, slot = r2 & 7;
    const int p = 4 * t + (slot >> 1);
    const int col = S * kSbCols + pair_col(p) + 5 * (slot & 1);
    const float v = col < d ? x[(size_t)tk * d + col] * pair_inv_f(p) : 0.f;
    const _Float16 hi = (_Float16)v;
    const _Float16 lo = (_Float16)(v - (float)hi);
    uint16_t *o = xrec + (size_t)tk * xrec_h + S * kSteps * 16 + t * 16;
    o[slot] = __builtin_bit_cast(uint16_t, hi);
    o[8 + slot] = __builtin_bit_cast(uint16_t, lo);
  }
}

}  // namespace moe
