// In-register dequantisation of the packed 3-bit weights, shared by the
// decode and prefill expert FFN kernels.
//
// A code pair (c, c+5) shares the low and high 15-bit halves of one packed
// word.  Slot j = p % 5 of pair p is extracted in place: slots 0..2 from the
// word itself, slots 3..4 from word >> 9, so the two codes sit at bits 3j'
// and 16 + 3j' (j' = j mod 3).  One v_and_or_b32 drops them into the
// mantissas of fp16 1024 + f q (f = 2^(3 j') = 1, 8 or 64); one v_pk_add
// takes 1024 + 4 f off, exactly, leaving f (q - 4); one v_pk_mul applies the
// pair's block scales, rounding once: f fp16((q - 4) s), f a power of two.
// The activations of that K slot are stored divided by f (record.h), so
// every product keeps its value.  Valid for block scales with
// 2^-14 <= |s| <= 255.875 (or s = 0): f (q - 4) s then stays a normal,
// finite fp16 for f up to 64 and |q - 4| <= 4.
//
// MFMA fragments (v_mfma_f32_16x16x32_f16): lane l = 16 g + r holds row r of
// a 16-row weight tile and K group g; over a 160-column superblock (16 words,
// 5 scale blocks) lane group g holds word quad g (words 4g .. 4g+3, its 20
// code pairs) and at MFMA step t (0..4) supplies pairs 4t .. 4t+3 of it.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "record.h"

namespace moe {

typedef _Float16 dq_h8 __attribute__((ext_vector_type(8)));
typedef _Float16 dq_h2 __attribute__((ext_vector_type(2)));

struct Consts {
  uint32_t mask[3];  // 0x00070007 << 3 j', kept in VGPRs so v_and_or_b32 can be used
  uint32_t magic;    // 0x64006400: fp16 1024 in both halves
};

__device__ inline Consts make_consts() {
  Consts k;
  k.mask[0] = 0x00070007u;
  k.mask[1] = 0x00380038u;
  k.mask[2] = 0x01c001c0u;
  k.magic = 0x64006400u;
  // opaque to the optimiser: stay in registers instead of becoming literals
  asm volatile("" : "+v"(k.mask[0]), "+v"(k.mask[1]), "+v"(k.mask[2]), "+s"(k.magic));
  return k;
}

template <int j>
__device__ inline dq_h2 deq_pair(uint32_t src, const Consts &K, dq_h2 sc) {
  constexpr int jj = j % 3;
  const uint32_t u = (src & K.mask[jj]) | K.magic;
  const dq_h2 v = __builtin_bit_cast(dq_h2, u);
  constexpr float off = 1024.0f + 4.0f * (jj == 0 ? 1.0f : (jj == 1 ? 8.0f : 64.0f));
  const dq_h2 o = {(_Float16)off, (_Float16)off};
  return (v - o) * sc;
}

// The scale pair a code pair needs depends on where its two columns fall: a
// quad starts at column 40 g = 8 g of scale block b = 5 S + g, so a pair's
// columns lie in blocks (b, b), (b, b+1) or (b+1, b+1), and which depends on
// g.  Per superblock a lane holds P = (s_b, s_b+1) and six byte-permuted
// copies of it, one per pattern of classes over the four lane groups that
// occurs (pairs whose class is the same for every g read P through op_sel).
//
// class of local pair q of quad g: 0 = both columns in block b, 1 = low in b
// and high in b + 1, 2 = both in b + 1
constexpr int pair_cls(int g, int q) {
  const int lo = 40 * g + pair_col(q);
  return (lo / 32 - g) + ((lo + 5) / 32 - g);
}
// pattern id of pair q: 0 = class 0 for every g, 7 = class 2 for every g,
// 1..6 = the mixed patterns.  In q order they are q 0-2: 0000, 3-4: 0001,
// 5: 0002, 6-9: 0012, 10-13: 0122, 14: 0222, 15-16: 1222, 17-19: 2222.
constexpr int pat_of(int q) {
  return q < 3 ? 0 : q < 5 ? 1 : q < 6 ? 2 : q < 10 ? 3 : q < 14 ? 4 : q < 15 ? 5 : q < 17 ? 6 : 7;
}
constexpr int pat_rep(int p) {  // a pair with pattern p
  return p == 0 ? 0 : p == 1 ? 3 : p == 2 ? 5 : p == 3 ? 6 : p == 4 ? 10 : p == 5 ? 14 : p == 6 ? 15 : 17;
}
constexpr bool pat_table_ok() {
  for (int q = 0; q < 20; ++q)
    for (int g = 0; g < 4; ++g) {
      if (pair_cls(g, q) != pair_cls(g, pat_rep(pat_of(q)))) return false;
      if (pat_of(q) == 0 && pair_cls(g, q) != 0) return false;
      if (pat_of(q) == 7 && pair_cls(g, q) != 2) return false;
    }
  return true;
}
static_assert(pat_table_ok(), "pattern table matches the scale classes");
// v_perm_b32 selector giving (s_lo, s_hi) of a class from P = s_b | s_b+1 << 16
constexpr uint32_t cls_sel(int c) {
  const uint32_t lo = c == 2 ? 2u : 0u, hi = c == 0 ? 0u : 2u;
  return lo | (lo + 1) << 8 | hi << 16 | (hi + 1) << 24;
}

// the six mixed-pattern selectors of lane group g
__device__ inline void pattern_selectors(int g, uint32_t (&sel)[6]) {
#pragma unroll
  for (int p = 1; p <= 6; ++p) {
    const int q = pat_rep(p);
    const uint32_t s0 = cls_sel(pair_cls(0, q)), s1 = cls_sel(pair_cls(1, q)), s2 = cls_sel(pair_cls(2, q)),
                   s3 = cls_sel(pair_cls(3, q));
    sel[p - 1] = g == 0 ? s0 : g == 1 ? s1 : g == 2 ? s2 : s3;
  }
}

template <int q>
__device__ inline dq_h2 pair_scale(uint32_t P, const uint32_t (&Pm)[6]) {
  constexpr int pat = pat_of(q);
  const dq_h2 S = __builtin_bit_cast(dq_h2, P);
  if constexpr (pat == 0) {
    return (dq_h2){S[0], S[0]};
  } else if constexpr (pat == 7) {
    return (dq_h2){S[1], S[1]};
  } else {
    return __builtin_bit_cast(dq_h2, Pm[pat - 1]);
  }
}

template <int q>
__device__ inline dq_h2 deq_q(const uint32_t (&w)[4], const Consts &K, uint32_t P, const uint32_t (&Pm)[6]) {
  constexpr int j = q % 5;
  return deq_pair<j>(j < 3 ? w[q / 5] : (w[q / 5] >> 9), K, pair_scale<q>(P, Pm));
}

// The same with the mixed-pattern scales computed where they are used (one
// v_perm_b32 per pattern and step, shared by the pairs of that step), for
// kernels that cannot keep the six copies in registers.
template <int q>
__device__ inline dq_h2 deq_q_sel(const uint32_t (&w)[4], const Consts &K, uint32_t P, const uint32_t (&sel)[6]) {
  constexpr int j = q % 5, pat = pat_of(q);
  const dq_h2 S = __builtin_bit_cast(dq_h2, P);
  dq_h2 sc;
  if constexpr (pat == 0)
    sc = (dq_h2){S[0], S[0]};
  else if constexpr (pat == 7)
    sc = (dq_h2){S[1], S[1]};
  else
    sc = __builtin_bit_cast(dq_h2, __builtin_amdgcn_perm(P, P, sel[pat - 1]));
  return deq_pair<j>(j < 3 ? w[q / 5] : (w[q / 5] >> 9), K, sc);
}

template <int t>
__device__ inline dq_h8 quad_a_sel(const uint32_t (&w)[4], const Consts &K, uint32_t P, const uint32_t (&sel)[6]) {
  const dq_h2 a0 = deq_q_sel<4 * t + 0>(w, K, P, sel);
  const dq_h2 a1 = deq_q_sel<4 * t + 1>(w, K, P, sel);
  const dq_h2 a2 = deq_q_sel<4 * t + 2>(w, K, P, sel);
  const dq_h2 a3 = deq_q_sel<4 * t + 3>(w, K, P, sel);
  return (dq_h8){a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
}

// the MFMA fragment of step t: pairs 4t .. 4t+3 of the lane's word quad
template <int t>
__device__ inline dq_h8 quad_a(const uint32_t (&w)[4], const Consts &K, uint32_t P, const uint32_t (&Pm)[6]) {
  const dq_h2 a0 = deq_q<4 * t + 0>(w, K, P, Pm);
  const dq_h2 a1 = deq_q<4 * t + 1>(w, K, P, Pm);
  const dq_h2 a2 = deq_q<4 * t + 2>(w, K, P, Pm);
  const dq_h2 a3 = deq_q<4 * t + 3>(w, K, P, Pm);
  return (dq_h8){a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
}

}  // namespace moe
