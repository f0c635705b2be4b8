// The parts of the prefill kernels' schedule that are plain integer
// arithmetic, kept apart so that they can be checked on the host: the copy
// waits of the K loop, where each column of the h record lives, and which
// thread of a gate/up workgroup stores which part of it.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "record.h"

namespace moe {
namespace pf {

// K loop: the x (or h) tile of step s + kXD is copied at step s into a ring
// of kXRing step tiles (two 16-byte copies per thread); at step 0 of
// superblock S each wave copies superblock S + 1's weights (4 word-quad
// copies and 4 scale copies).
constexpr int kXD = 3;
constexpr int kXRing = 4;
constexpr int kXCopies = 2;
constexpr int kWCopies = 8;

// Copies issued after a step's tile copies by the time that step waits for
// them (s_waitcnt vmcnt counts the loads still in flight, and they complete
// in order): the tiles of the kXD - 1 later steps and kWCopies weight copies
// for every superblock start among the kXD steps since.  In superblock 0
// (`first`) the prologue's order applies -- tiles 0 .. kXD-1, then superblock
// 0's weights -- and step 0 waits for all of it.
constexpr int vm_after(int t, bool first) {
  if (first) {
    if (t == 0) return 0;
    int n = 0;
    // prologue: tiles t+1 .. kXD-1, superblock 0's weights
    if (t < kXD) n += kXCopies * (kXD - 1 - t) + kWCopies;
    // steps 0 .. t-1 of superblock 0 (for t <= kXD), or t-kXD .. t-1
    const int u0 = t < kXD ? 0 : t - kXD;
    for (int u = u0; u < t; ++u) n += kXCopies + (u == 0 ? kWCopies : 0);
    return n - (t < kXD ? 0 : kXCopies);  // the issuing step's own copies come first
  }
  int n = kXCopies * (kXD - 1);
  for (int u = t - kXD; u < t; ++u) n += ((u % 5 + 5) % 5 == 0) ? kWCopies : 0;
  return n;
}

// A record row holds, per 32-K step, 128 bytes: [hi | lo][lane group g][8
// halves]; the 8 halves of (step t of superblock S, group g) -- a "piece" --
// are pairs 20 g + 4 t + i (i = 0..3), columns c and c + 5 as halves 2 i + e.
constexpr int kRecRowB = 128;

// byte of column c's hi half inside one record row (its lo half sits 64
// bytes further); `inv_f` gets the 1 / f the value is stored with
__host__ __device__ inline int rec_byte(int c, float &inv_f) {
  const int S = c / kSbCols, lc = c - S * kSbCols;
  const int w = lc / 10, j = lc - 10 * w;
  const int p = 5 * w + j % 5, e = j / 5;  // pair of the superblock, half
  const int g = p / 20, t = (p % 20) / 4, i = p % 4;
  const int jj = (j % 5) % 3;
  inv_f = jj == 0 ? 1.0f : (jj == 1 ? 0.125f : 0.015625f);
  return (S * 5 + t) * kRecRowB + g * 16 + (2 * i + e) * 2;
}

// which of the 8 halves (bit 2 i + e) of piece (S, t, g) hold a column in
// [c0, c1)
__host__ __device__ inline uint32_t piece_own(int S, int t, int g, int c0, int c1) {
  uint32_t own = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = S * kSbCols + pair_col(20 * g + 4 * t + i);
    own |= (c >= c0 && c < c1 ? 1u : 0u) << (2 * i);
    own |= (c + 5 >= c0 && c + 5 < c1 ? 1u : 0u) << (2 * i + 1);
  }
  return own;
}

// the record lines L0 .. L0 + nl - 1 that an item's columns [c0, c1) fall in
__host__ __device__ inline int item_L0(int c0) { return 5 * (c0 / kSbCols); }
__host__ __device__ inline int item_nl(int c0, int c1) { return 5 * ((c1 - 1) / kSbCols) + 5 - item_L0(c0); }

// Gate/up write-out, whole pieces: the thread with piece index wi (of the
// item's 8 nl pieces per token, line L0 + wi / 8, piece wi % 8) stores the
// piece whole when the item owns all 8 halves.  Returns the ownership mask
// (0 past the item's pieces).
__host__ __device__ inline uint32_t full_piece_own(int wi, int c0, int c1) {
  const int L0 = item_L0(c0), nl = item_nl(c0, c1);
  if (wi >= 8 * nl) return 0;
  const int L = L0 + (wi >> 3), S = L / 5, t = L - 5 * S;
  return piece_own(S, t, wi & 3, c0, c1);
}

// Gate/up write-out, shared pieces: they lie in the quad (40 columns) of a
// row-block boundary that is not quad-aligned (c0, or c1: the next block or
// the padding past d_ff), 5 lines x (hi, lo) = 10 candidate pieces each.
// Role pq (0..159) stores half jh = pq % 8 of candidate pp = pq / 8 when the
// item owns that half but not the whole piece.
struct BoundaryRole {
  bool mine;
  int line;   // record line
  int piece;  // piece inside the line (4 hl + g)
  int half;   // half inside the piece
};

__host__ __device__ inline BoundaryRole boundary_role(int pq, int c0, int c1) {
  BoundaryRole r;
  const int pp = pq >> 3;
  r.half = pq & 7;
  const int bcol = pp < 10 ? c0 : c1, tt = (pp % 10) >> 1, hl = pp & 1;
  const int Sb = bcol / kSbCols, gb = (bcol % kSbCols) / 40;
  r.line = 5 * Sb + tt;
  r.piece = 4 * hl + gb;
  r.mine = false;
  if (bcol % 40 != 0) {
    const uint32_t own = piece_own(Sb, tt, gb, c0, c1);
    r.mine = own != 0xffu && (own >> r.half & 1u);
  }
  return r;
}

}  // namespace pf
}  // namespace moe
