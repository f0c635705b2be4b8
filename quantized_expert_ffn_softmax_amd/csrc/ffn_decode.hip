// Decode path of the expert FFN: few tokens per expert, bound by streaming
// the experts' packed 3-bit weights from HBM.
//
// The pages' engine reads each touched expert once per step and shares that
// read between the tokens that picked it (speculative verify batches several
// tokens: "单卡5090跑125B 大模型 ...", section 2.3).  Here one wave handles up
// to 8 tokens of one expert against 16 weight rows with
// v_mfma_f32_16x16x32_f16:
//   A (16 rows x 32 K)  = dequantised weights fp16((q - 4) * s), built in
//                         registers from the packed words;
//   B (32 K x 16 cols)  = activations split into two fp16 halves: column n < 8
//                         holds token n's hi half, column n + 8 its lo half;
//                         adding the two output columns keeps fp32 accuracy
//                         with one MFMA per A tile.
// The layout repeats every 160 columns (16 words, 5 scale blocks): lane group
// g = lane / 16 takes superblock 4R + g, so every lane runs the same
// instruction stream; the 80 code pairs (c, c+5) of a superblock are 20 MFMA
// steps of 4 pairs.  Weights are read once; activations come from L2.
#include <algorithm>
#include <utility>

#include "moe_internal.h"
#include "dequant.h"
#include "lds_copy.h"
#include "record.h"

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));

// pair p (0..79) of a superblock: word p/5, slot p%5 (low half) and p%5+5
// (high half); columns 10 (p/5) + p%5 and +5.
using moe::pair_col;

struct DecodeParams {
  const moe::WorkEntry *work;   // entries of <= 4 tokens
  const moe::WorkEntry *work8;  // entries of <= 8 tokens
  const int32_t *n_work;        // [0]: entries of work, [2]: entries of work8
  const int32_t *perm;
  const int32_t *slot_of_pair;
  const uint8_t *slot_pool;
  const uint8_t *shared_pool;
  uint32_t stride;
  int layer, E, k, T;
  int n_slots;
  int max_work, max_work8;  // bounds on n_work[0] and n_work[2] (workspace sizes)
  moe::MatLayout gate, up, down;
  const uint16_t *xrec;    // [T + 1][xrec_h], last row zero
  int xrec_h;
  uint16_t *hrec;          // [T*k + T + 1][hrec_h], last row zero
  int hrec_h;
  const uint16_t *xrec_zero, *hrec_zero;  // the all-zero rows
  float *y_pairs, *y_shared;
  int d_model, d_ff;
};

__device__ inline const uint8_t *entry_blob(const DecodeParams &P, const moe::WorkEntry &we) {
  if (we.expert < 0) return P.shared_pool + (size_t)P.layer * P.stride;
  const int slot = P.slot_of_pair ? P.slot_of_pair[P.perm[we.first]] : P.layer * P.E + we.expert;
  if (slot < 0 || slot >= P.n_slots) return nullptr;  // never read outside the pool
  return P.slot_pool + (size_t)slot * P.stride;
}

using moe::Consts;
using moe::make_consts;

__device__ inline f4 mfma(h8 a, h8 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }

using moe::rec_pos;

// a work entry is used only if it indexes inside this call's pairs / tokens
__device__ inline bool entry_ok(const DecodeParams &P, const moe::WorkEntry &we, int cols) {
  if (we.m < 1 || we.m > cols || we.first < 0) return false;
  return we.expert >= 0 ? (we.expert < P.E && we.first + we.m <= P.T * P.k) : (we.first + we.m <= P.T);
}

// the token and the record row (pair, or T*k + token for the shared expert)
// behind entry column n
__device__ inline bool entry_token(const DecodeParams &P, const moe::WorkEntry &we, int n, int &tok, int &row) {
  if (we.expert >= 0) {
    const int pair = P.perm[we.first + n];
    if (pair < 0 || pair >= P.T * P.k) return false;
    tok = pair / P.k;
    row = pair;
  } else {
    tok = we.first + n;
    row = P.T * P.k + tok;
  }
  return true;
}

// ---------------------------------------------------------------------------
// Work decomposition.  A unit is one entry (<= 4 tokens of one expert) times
// kWaves consecutive 16-row tiles; a workgroup of kWaves waves takes a unit,
// each wave one tile over the whole K range, so no partial sums cross waves.
//
// Memory-level parallelism decides this kernel's speed: HBM latency under
// load is several microseconds, comparable to a unit's whole computation.
// So a unit issues everything it will read at once:
//   * the entry's activation record (all superblocks, its <= 4 columns) and
//     the scale arrays of the unit's 64 rows go to LDS by direct
//     global-to-LDS copies, first;
//   * then each wave loads every 16-byte word quad of its 16 rows into
//     registers (NSB superblocks x NMAT matrices of 16 bytes per lane).
// One barrier (after the copies have landed; the word loads stay in flight)
// publishes the LDS data; from there each wave walks its superblocks in
// order, waiting only for the word loads of the superblock at hand.
//
// Lane mapping inside a superblock: lane group g = lane / 16 holds word quad
// g (words 4g .. 4g+3, columns 40g .. 40g+39) of its row, and a superblock
// is 5 MFMA steps: at step t the lane group supplies pairs 4t .. 4t+3 of its
// quad, i.e. pairs 20g + 4t .. of the superblock, whose activations are
// record step 5g + t.  B columns n < 4 hold token n's hi halves, n + 4 its lo
// halves; columns 8..15 repeat 0..7 (their outputs are not used).  The
// dequantisation and its per-pair scale classes are in dequant.h.
// ---------------------------------------------------------------------------

constexpr int kWaves = 4;
constexpr int kXcds = 8;      // accelerator dies of MI355X, each with its own L2
constexpr int kSplitMaxTokens = 32;  // gate/up splits K over the waves up to this batch
// An entry of COLS tokens (4 or 8) fills MFMA B columns n (token n's hi
// half) and n + COLS (its lo half); at COLS = 4 columns 8..15 repeat 0..7 and
// their outputs are dropped.  In LDS a record step of the entry is 2 COLS
// slots of 16 bytes (hi then lo, token-minor): SB bytes.
template <int COLS>
struct Cols {
  static constexpr int SB = 2 * COLS * 16;        // bytes per record step
  static constexpr int kSbBytes = moe::kSteps * SB;  // one superblock: 2,560 B at COLS = 4
};

struct Unit {
  const uint8_t *blob;  // the expert's blob (a readable stand-in when the entry is unusable)
  int tile0;            // first 16-row tile of the unit
  int m;                // entry columns in use (0 for an unusable entry)
  int routed;
  int has_tok, tok, rrow;  // this lane's entry column (lane % 4)
};

template <int NMAT>
struct Mats {
  moe::MatLayout m[NMAT];
  const uint16_t *rec, *zero;  // activation record and its all-zero row
  int rec_h;
};

template <int NMAT>
__device__ inline Mats<NMAT> mats_of(const DecodeParams &P) {
  Mats<NMAT> Mt;
  if constexpr (NMAT == 2) {
    Mt.m[0] = P.gate;
    Mt.m[1] = P.up;
    Mt.rec = P.xrec;
    Mt.zero = P.xrec_zero;
    Mt.rec_h = P.xrec_h;
  } else {
    Mt.m[0] = P.down;
    Mt.rec = P.hrec;
    Mt.zero = P.hrec_zero;
    Mt.rec_h = P.hrec_h;
  }
  return Mt;
}

template <int COLS>
__device__ inline void unit_setup(const DecodeParams &P, int u, int tpu, int tiles, int col, Unit &U) {
  const moe::WorkEntry we = (COLS == 8 ? P.work8 : P.work)[u / tpu];
  U.tile0 = (u % tpu) * tiles;
  U.routed = we.expert >= 0;
  const uint8_t *blob = entry_ok(P, we, COLS) ? entry_blob(P, we) : nullptr;
  U.m = blob ? we.m : 0;
  U.blob = blob ? blob : P.shared_pool + (size_t)P.layer * P.stride;
  U.tok = 0;
  U.rrow = 0;
  U.has_tok = col < U.m && entry_token(P, we, col, U.tok, U.rrow);
}

using moe::lds_addr;
using moe::lds_copy16;

__device__ inline h8 lds_h8(const uint8_t *p) { return *reinterpret_cast<const h8 *>(p); }

// LDS row pitch of a unit's scale rows: the row's bytes, rounded up to an odd
// number of 16-byte granules when they are a multiple of 16 (2 nblk = 128 at
// d_model 2048 would put the 16 rows a wave reads on the same banks); other
// widths keep the plain row (48 bytes at d_ff 768: already an odd count)
__host__ __device__ constexpr int sc_pitch(int nblk) {
  return (2 * nblk) % 16 == 0 ? ((2 * nblk / 16) | 1) * 16 : 2 * nblk;
}

// number of 16-byte-per-lane copies one thread issues for the unit's LDS data
template <int NSB, int NMAT, int COLS>
struct CopyCounts {
  static constexpr int act = (NSB * moe::kSteps * 2 * COLS + 64 * kWaves - 1) / (64 * kWaves);
  // scales: <= 64 rows x sc_pitch(nblk) per matrix, nblk <= 5 NSB
  static constexpr int sc = (64 * sc_pitch(5 * NSB + 8) + 16 * 64 * kWaves - 1) / (16 * 64 * kWaves);
};

// activation slot p = (superblock * 20 + step) * 2 COLS + half * COLS + col
// holds the 8 halves of that record step for entry column col
template <int NSB, int NMAT, int COLS>
__device__ inline void copy_unit_lds(const Mats<NMAT> &Mt, const Unit &U, int tid, uint32_t row_off, int unit_rows,
                                     int sc_mat_bytes, uint8_t *lact, uint8_t *lsc) {
  const uint8_t *rec = reinterpret_cast<const uint8_t *>(Mt.rec);
  const int half = (tid / COLS) & 1, w = tid >> 6;
  const uint32_t a0 = lds_addr(lact) + 1024u * w;
#pragma unroll
  for (int i = 0; i < CopyCounts<NSB, NMAT, COLS>::act; ++i) {
    const int p = tid + 64 * kWaves * i;
    const int ms = p / (2 * COLS);
    // columns past the entry's tokens are not copied: an MFMA output column
    // depends only on its own B column and the epilogue writes only the
    // entry's tokens, so those slots may hold anything
    if (U.has_tok && p < NSB * moe::kSteps * 2 * COLS)
      lds_copy16(rec + row_off + (ms * 16 + half * 8) * 2, a0 + 4096u * i);
  }
  // scales: LDS row pitch sc_pitch(nblk) (see there); granule k of a matrix's
  // region holds 16 bytes of row k / (pitch / 16) -- the copy picks each
  // lane's source, so padding a row costs only the extra granule
  const uint32_t s0 = lds_addr(lsc) + 1024u * w;
  const int rb = Mt.m[0].nblk * 2, pitch = sc_pitch(Mt.m[0].nblk), gpr = pitch / 16;
#pragma unroll
  for (int mat = 0; mat < NMAT; ++mat) {
    const uint8_t *src = U.blob + Mt.m[mat].scale_off + (uint32_t)U.tile0 * 16 * rb;
#pragma unroll
    for (int i = 0; i < CopyCounts<NSB, NMAT, COLS>::sc; ++i) {
      const int k = tid + 64 * kWaves * i;
      if (pitch == rb) {  // rows copied as they lie (any row size)
        if (16 * k < unit_rows * rb) lds_copy16(src + 16 * k, s0 + (uint32_t)(mat * sc_mat_bytes) + 4096u * i);
      } else if (k < unit_rows * gpr) {
        const int row = k / gpr, c = min(k - row * gpr, rb / 16 - 1);  // the pad granule repeats the last
        lds_copy16(src + row * rb + 16 * c, s0 + (uint32_t)(mat * sc_mat_bytes) + 4096u * i);
      }
    }
  }
}

using moe::quad_a;

struct MatSb {
  uint32_t w[4];
  uint32_t P;
  uint32_t Pm[6];
};

// scales (s_b, s_b+1) of this lane's row from the LDS copy, b = 5 S + g
// clamped to the row (only the last superblock can reach past it)
template <bool CLAMP>
__device__ inline MatSb mat_sb(const uint4 &wq, const uint8_t *srow, int b, int nblk, const uint32_t (&sel)[6]) {
  MatSb M;
  M.w[0] = wq.x;
  M.w[1] = wq.y;
  M.w[2] = wq.z;
  M.w[3] = wq.w;
  const int b0 = CLAMP ? min(b, nblk - 1) : b, b1 = CLAMP ? min(b + 1, nblk - 1) : b + 1;
  const uint32_t lo = *reinterpret_cast<const uint16_t *>(srow + 2 * b0);
  const uint32_t hi = *reinterpret_cast<const uint16_t *>(srow + 2 * b1);
  M.P = lo | (hi << 16);
#pragma unroll
  for (int i = 0; i < 6; ++i) M.Pm[i] = __builtin_amdgcn_perm(M.P, M.P, sel[i]);
  return M;
}

template <int NMAT, int t, int COLS>
__device__ inline void sb_step(const MatSb (&M)[NMAT], const Consts &K, const uint8_t *xb, f4 &acc0, f4 &acc1) {
  const h8 x = lds_h8(xb + t * Cols<COLS>::SB);
  if constexpr (NMAT == 2) {
    acc0 = mfma(quad_a<t>(M[0].w, K, M[0].P, M[0].Pm), x, acc0);
    acc1 = mfma(quad_a<t>(M[1].w, K, M[1].P, M[1].Pm), x, acc1);
  } else if constexpr (t % 2 == 0) {
    acc0 = mfma(quad_a<t>(M[0].w, K, M[0].P, M[0].Pm), x, acc0);
  } else {
    acc1 = mfma(quad_a<t>(M[0].w, K, M[0].P, M[0].Pm), x, acc1);
  }
}

// gate/up: h = silu(g) u into the h record; down: y
template <int NMAT, int COLS>
__device__ inline void unit_epilogue(const DecodeParams &P, const Unit &U, int w, int lane, f4 acc0, f4 acc1) {
  const int r16 = lane & 15, g = lane >> 4;
  const int rows = NMAT == 2 ? P.d_ff : P.d_model;
  const int rt = U.tile0 + w;
  // D layout: lane holds rows 4g + i of the tile for MFMA column r16; token
  // n's value is column n (hi) + column n + COLS (lo)
  if constexpr (NMAT == 1) acc0 += acc1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc0[i] += __shfl_xor(acc0[i], COLS, 64);
    if constexpr (NMAT == 2) acc1[i] += __shfl_xor(acc1[i], COLS, 64);
  }
  if (!(U.has_tok && r16 < COLS && rt * 16 < rows)) return;
  if constexpr (NMAT == 2) {
    uint16_t *hr = P.hrec + (size_t)U.rrow * P.hrec_h;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float gv = acc0[i], uv = acc1[i];
      float inv_f;
      const int pos = rec_pos(rt * 16 + 4 * g + i, inv_f);
      const float h = gv / (1.0f + __expf(-gv)) * uv * inv_f;
      const _Float16 hi = (_Float16)h;
      const _Float16 lo = (_Float16)(h - (float)hi);
      hr[pos] = __builtin_bit_cast(uint16_t, hi);
      hr[pos + 8] = __builtin_bit_cast(uint16_t, lo);
    }
  } else {
    float *y = U.routed ? P.y_pairs + (size_t)U.rrow * P.d_model : P.y_shared + (size_t)U.tok * P.d_model;
    *reinterpret_cast<float4 *>(y + rt * 16 + 4 * g) = make_float4(acc0[0], acc0[1], acc0[2], acc0[3]);
  }
}

// gate/up of a K-split unit: the wave's two rows i0, i0 + 1 of its four (the
// two halves of K finalise two rows each), the same arithmetic per row as above
template <int COLS>
__device__ inline void gateup_rows(const DecodeParams &P, const Unit &U, int w, int lane, int i0, float g0, float g1,
                                   float u0, float u1) {
  const int r16 = lane & 15, g = lane >> 4;
  const int rt = U.tile0 + w;
  g0 += __shfl_xor(g0, COLS, 64);
  g1 += __shfl_xor(g1, COLS, 64);
  u0 += __shfl_xor(u0, COLS, 64);
  u1 += __shfl_xor(u1, COLS, 64);
  if (!(U.has_tok && r16 < COLS && rt * 16 < P.d_ff)) return;
  uint16_t *hr = P.hrec + (size_t)U.rrow * P.hrec_h;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float gv = j ? g1 : g0, uv = j ? u1 : u0;
    float inv_f;
    const int pos = rec_pos(rt * 16 + 4 * g + i0 + j, inv_f);
    const float h = gv / (1.0f + __expf(-gv)) * uv * inv_f;
    const _Float16 hi = (_Float16)h;
    const _Float16 lo = (_Float16)(h - (float)hi);
    hr[pos] = __builtin_bit_cast(uint16_t, hi);
    hr[pos + 8] = __builtin_bit_cast(uint16_t, lo);
  }
}

// the same for one row i of the four (the quarters of K finalise one row each)
template <int COLS>
__device__ inline void gateup_row(const DecodeParams &P, const Unit &U, int w, int lane, int i, float gv, float uv) {
  const int r16 = lane & 15, g = lane >> 4;
  const int rt = U.tile0 + w;
  gv += __shfl_xor(gv, COLS, 64);
  uv += __shfl_xor(uv, COLS, 64);
  if (!(U.has_tok && r16 < COLS && rt * 16 < P.d_ff)) return;
  uint16_t *hr = P.hrec + (size_t)U.rrow * P.hrec_h;
  float inv_f;
  const int pos = rec_pos(rt * 16 + 4 * g + i, inv_f);
  const float h = gv / (1.0f + __expf(-gv)) * uv * inv_f;
  const _Float16 hi = (_Float16)h;
  const _Float16 lo = (_Float16)(h - (float)hi);
  hr[pos] = __builtin_bit_cast(uint16_t, hi);
  hr[pos + 8] = __builtin_bit_cast(uint16_t, lo);
}

// word quads of superblocks issued up front; the rest is requested as the
// registers of superblock S - depth free up (gate/up keeps 9 superblocks of
// two matrices in flight within the register budget of 3 waves per SIMD)
template <int NSB, int NMAT>
constexpr int words_depth() {
  // a half range (K split, <= 7 superblocks) keeps 3: its kernel carries the split's extra registers
  return NMAT == 2 ? (NSB <= 7 ? (NSB < 3 ? NSB : 3) : 4) : NSB;
}

// A wave walks NSB superblocks of its range (the whole row, or one half of it
// when K is split): superblock S of the range is superblock sb0 + S of the
// row; only the first `nvalid` exist (the last one of a second half may not).
template <int NSB, int NMAT>
struct WordSrc {
  const uint8_t *blob;
  uint32_t off[NMAT];  // this lane's quad of the range's first superblock in each matrix
  int nvalid;
};

template <int NSB, int NMAT, int S>
__device__ inline void load_words(const WordSrc<NSB, NMAT> &Src, uint4 (&W)[NSB][NMAT]) {
  // only a range's last superblock can lie past the row (a shorter range)
  const uint32_t so = S + 1 < NSB ? (uint32_t)S * 64 : (uint32_t)min(S, Src.nvalid - 1) * 64;
#pragma unroll
  for (int mat = 0; mat < NMAT; ++mat) W[S][mat] = *reinterpret_cast<const uint4 *>(Src.blob + (Src.off[mat] + so));
}

template <int NSB, int NMAT, int... Ss>
__device__ inline void load_first(std::integer_sequence<int, Ss...>, const WordSrc<NSB, NMAT> &Src,
                                  uint4 (&W)[NSB][NMAT]) {
  (load_words<NSB, NMAT, Ss>(Src, W), ...);
}

template <int NSB, int NMAT, int S>
__device__ inline void refill(uint4 (&W)[NSB][NMAT], const WordSrc<NSB, NMAT> &Src) {
  constexpr int D = words_depth<NSB, NMAT>();
  if constexpr (S + D < NSB) {
    load_words<NSB, NMAT, S + D>(Src, W);
    asm volatile("" ::: "memory");  // keep the request here, a full D superblocks ahead of its use
  }
}

// superblocks S and S + 1 together, their steps interleaved (twice the
// independent dequantise-and-MFMA chains per wave); a last odd superblock
// alone.  With SHORT (quarters of K, ranges one superblock shorter than NSB
// after the first) the last pair may hold one superblock only: a uniform
// branch, and every scale block index is clamped to the row.
template <int NSB, int NMAT, int COLS, bool SHORT, int S>
__device__ inline void compute_pair(uint4 (&W)[NSB][NMAT], const WordSrc<NSB, NMAT> &Src,
                                    const uint8_t *(&srow)[NMAT], int g, int nblk, const uint32_t (&sel)[6],
                                    const Consts &K, const uint8_t *xb, f4 &acc0, f4 &acc1, f4 &acc2, f4 &acc3) {
  // g carries the range's first scale block: block 5 S + g of the range
  if constexpr (S + 1 >= NSB) {
    if (S >= Src.nvalid) return;  // a range one superblock shorter (uniform)
  }
  MatSb M[NMAT];
#pragma unroll
  for (int mat = 0; mat < NMAT; ++mat)
    M[mat] = mat_sb<(S + 2 >= NSB || SHORT)>(W[S][mat], srow[mat], 5 * S + g, nblk, sel);
  refill<NSB, NMAT, S>(W, Src);
  const uint8_t *xs = xb + S * Cols<COLS>::kSbBytes;
  bool two = S + 1 < NSB;
  if constexpr (SHORT && S + 2 == NSB) two = S + 1 < Src.nvalid;
  if (two) {
    MatSb M2[NMAT];
#pragma unroll
    for (int mat = 0; mat < NMAT; ++mat)
      M2[mat] = mat_sb<(S + 3 >= NSB || SHORT)>(W[(S + 1) % NSB][mat], srow[mat], 5 * (S + 1) + g, nblk, sel);
    refill<NSB, NMAT, S + 1>(W, Src);
    const uint8_t *xs2 = xs + Cols<COLS>::kSbBytes;
    sb_step<NMAT, 0, COLS>(M, K, xs, acc0, acc1);
    sb_step<NMAT, 0, COLS>(M2, K, xs2, acc2, acc3);
    sb_step<NMAT, 1, COLS>(M, K, xs, acc0, acc1);
    sb_step<NMAT, 1, COLS>(M2, K, xs2, acc2, acc3);
    sb_step<NMAT, 2, COLS>(M, K, xs, acc0, acc1);
    sb_step<NMAT, 2, COLS>(M2, K, xs2, acc2, acc3);
    sb_step<NMAT, 3, COLS>(M, K, xs, acc0, acc1);
    sb_step<NMAT, 3, COLS>(M2, K, xs2, acc2, acc3);
    sb_step<NMAT, 4, COLS>(M, K, xs, acc0, acc1);
    sb_step<NMAT, 4, COLS>(M2, K, xs2, acc2, acc3);
  } else {
    sb_step<NMAT, 0, COLS>(M, K, xs, acc0, acc1);
    sb_step<NMAT, 1, COLS>(M, K, xs, acc0, acc1);
    sb_step<NMAT, 2, COLS>(M, K, xs, acc0, acc1);
    sb_step<NMAT, 3, COLS>(M, K, xs, acc0, acc1);
    sb_step<NMAT, 4, COLS>(M, K, xs, acc0, acc1);
  }
}

template <int NSB, int NMAT, int COLS, bool SHORT, int... Ps>
__device__ inline void compute_all(std::integer_sequence<int, Ps...>, uint4 (&W)[NSB][NMAT],
                                   const WordSrc<NSB, NMAT> &Src, const uint8_t *(&srow)[NMAT], int g, int nblk,
                                   const uint32_t (&sel)[6], const Consts &K, const uint8_t *xb, f4 &acc0, f4 &acc1,
                                   f4 &acc2, f4 &acc3) {
  (compute_pair<NSB, NMAT, COLS, SHORT, 2 * Ps>(W, Src, srow, g, nblk, sel, K, xb, acc0, acc1, acc2, acc3), ...);
}

// KS = 2 (gate/up of small batches): K split in two halves over the waves of a
// workgroup -- waves 2h + l take tile l of the unit's 2 tiles and superblocks
// [h H, min((h + 1) H, NSB)) with H = ceil(NSB / 2) -- and the halves' sums
// added through LDS before the epilogue.  Twice the waves in flight and half
// the chain per wave, for batches whose units leave CUs idle.  KS = 4 (the
// smallest batches, whose quarter units all fit in the CUs at once): one tile
// per unit, wave q takes NSB / 4 superblocks, one more for the first NSB mod 4
// waves (13 = 4 + 3 + 3 + 3: only a range's last pair can be short), and
// wave 0 adds the other three quarters' sums in order.
// workgroups per CU the kernel is built for: gate/up 3; down 4 up to 6
// superblocks (the model's d_ff = 768 is 5), then what its registers allow
// on entries of 8 tokens (3 up to 9 superblocks, 2 beyond)
template <int NSB, int NMAT>
constexpr int decode_min_blocks() {
  return NMAT == 2 ? 3 : (NSB <= 6 ? 4 : (NSB <= 9 ? 3 : 2));
}

template <int NSB, int NMAT, int KS, int COLS>
__global__ void __launch_bounds__(64 * kWaves, (decode_min_blocks<NSB, NMAT>())) ffn_decode_kernel(DecodeParams P) {
  static_assert(KS == 1 || (NMAT == 2 && (KS == 4 || ((NSB + 1) / 2) % 2 == 1)),
                "K split: gate/up; halves of an odd length, or quarters");
  static_assert(COLS == 4 || COLS == 8, "entries of 4 or 8 tokens");
  static_assert(KS != 4 || (NSB % 4 <= 1 && NSB >= 8), "quarters: a first range at most one longer");
  constexpr int NS = (NSB + KS - 1) / KS;  // superblocks of a wave's range (the longest)
  constexpr bool SHORT = KS == 4;
  constexpr int kTiles = kWaves / KS;      // 16-row tiles of a unit
  constexpr int kActBytes = NSB * Cols<COLS>::kSbBytes;
  constexpr int kScMat = 16 * kTiles * sc_pitch(5 * NSB + 8);  // one matrix's scales of the unit's rows (nblk <= 5 NSB)
  constexpr int kScBytes = NMAT * kScMat;
  __shared__ __attribute__((aligned(1024))) uint8_t lact[kActBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lsc[(kScBytes + 4095) / 4096 * 4096];
  __shared__ f4 red[KS == 1 ? 1 : (KS == 2 ? 2 * kTiles * 64 : 4 * 64 * 2)];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int ltile = KS == 1 ? w : w % kTiles;                                    // tile of the unit
  const int half = KS == 1 ? 0 : __builtin_amdgcn_readfirstlane(w / kTiles);  // range (uniform per wave)
  // the wave's range: superblocks [sb0, sb0 + nvalid) of the row
  const int sb0 = KS == 4 ? half * (NSB / 4) + min(half, NSB % 4) : half * NS;
  const int nvalid = KS == 4 ? NSB / 4 + (half < NSB % 4 ? 1 : 0) : min(NS, NSB - sb0);
  const Mats<NMAT> Mt = mats_of<NMAT>(P);
  const int ntile = Mt.m[0].rows / 16;
  const int tpu = (ntile + kTiles - 1) / kTiles;
  const int nblk = Mt.m[0].nblk;
  const int n_units = (COLS == 8 ? min(P.n_work[2], P.max_work8) : min(P.n_work[0], P.max_work)) * tpu;
  // Workgroup b runs on XCD b % 8 (round-robin dispatch).  Each XCD takes a
  // contiguous range of units, so the tiles of neighbouring entries -- the
  // entries of an expert with more than 4 tokens, or of the shared expert --
  // stream through one L2 and the second read of a blob hits it.
  const int per = (n_units + kXcds - 1) / kXcds;
  const int xcd = blockIdx.x % kXcds, u_step = gridDim.x / kXcds;
  const int u_end = min((xcd + 1) * per, n_units);
  const Consts K = make_consts();
  uint32_t sel[6];
  moe::pattern_selectors(g, sel);
  // B operand of lane (j, g) at step t of superblock S: record step
  // ms = 20 S + 5 g + t, slot ms * 2 COLS + (j mod 2 COLS), i.e. byte
  // (20 S + t) * SB + 5 SB g + 16 (j mod 2 COLS); the wave's range starts at
  // superblock sb0
  constexpr int SB = Cols<COLS>::SB;
  const uint8_t *xb = lact + 5 * SB * g + 16 * (r16 & (2 * COLS - 1)) + sb0 * moe::kSteps * SB;
  bool first = true;
  for (int u = xcd * per + blockIdx.x / kXcds; u < u_end; u += u_step) {
    if (!first) __syncthreads();  // every wave is done with the previous unit's LDS data
    first = false;
    Unit U;
    unit_setup<COLS>(P, u, tpu, kTiles, tid & (COLS - 1), U);
    const uint32_t row_off = (uint32_t)(NMAT == 2 ? U.tok : U.rrow) * (uint32_t)Mt.rec_h * 2u;
    copy_unit_lds<NSB, NMAT, COLS>(Mt, U, tid, row_off, 16 * kTiles, kScMat, lact, lsc);
    // the word quads of this wave's rows, as many superblocks as fit
    const int row = min((U.tile0 + ltile) * 16 + r16, Mt.m[0].rows - 1);
    WordSrc<NS, NMAT> Src;
    Src.blob = U.blob;
    Src.nvalid = nvalid;
#pragma unroll
    for (int mat = 0; mat < NMAT; ++mat)
      Src.off[mat] = Mt.m[mat].code_off + (uint32_t)row * Mt.m[mat].wpr * 4 + g * 16 + sb0 * 64;
    constexpr int D = words_depth<NS, NMAT>();
    uint4 W[NS][NMAT];
    load_first<NS, NMAT>(std::make_integer_sequence<int, D>{}, Src, W);
    // the copies were issued before the word loads: waiting until only the
    // word loads may be outstanding lands them; then publish
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(D * NMAT) : "memory");
    __syncthreads();
    const uint8_t *srow[NMAT];
#pragma unroll
    for (int mat = 0; mat < NMAT; ++mat)
      srow[mat] = lsc + mat * kScMat + (ltile * 16 + r16) * sc_pitch(nblk);
    f4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f}, acc2 = acc0, acc3 = acc0;
    compute_all<NS, NMAT, COLS, SHORT>(std::make_integer_sequence<int, (NS + 1) / 2>{}, W, Src, srow, 5 * sb0 + g, nblk,
                                sel, K, xb, acc0, acc1, acc2, acc3);
    acc0 += acc2;
    acc1 += acc3;
    if constexpr (KS == 2) {
      // each half finalises two of the lane's four rows (2 h, 2 h + 1) and
      // writes its partial sums of the other two through LDS; a row is the
      // sum of the two halves' partials (one addition: the same value in
      // either order)
      const f4 mine = half == 0 ? f4{acc0[2], acc0[3], acc1[2], acc1[3]} : f4{acc0[0], acc0[1], acc1[0], acc1[1]};
      red[(half * kTiles + ltile) * 64 + lane] = mine;
      __syncthreads();
      const f4 r = red[((1 - half) * kTiles + ltile) * 64 + lane];
      if (half == 0)
        gateup_rows<COLS>(P, U, ltile, lane, 0, acc0[0] + r[0], acc0[1] + r[1], acc1[0] + r[2], acc1[1] + r[3]);
      else
        gateup_rows<COLS>(P, U, ltile, lane, 2, acc0[2] + r[0], acc0[3] + r[1], acc1[2] + r[2], acc1[3] + r[3]);
      continue;
    } else if constexpr (KS == 4) {
      // every quarter's sums -> LDS; quarter q finalises row q of the lane's
      // four, adding the quarters in order (q0 + q1 + q2 + q3)
      red[(half * 64 + lane) * 2 + 0] = acc0;
      red[(half * 64 + lane) * 2 + 1] = acc1;
      __syncthreads();
      const int q = half;  // uniform
      float gv = red[lane * 2 + 0][q], uv = red[lane * 2 + 1][q];
#pragma unroll
      for (int p = 1; p < 4; ++p) {
        gv += red[(p * 64 + lane) * 2 + 0][q];
        uv += red[(p * 64 + lane) * 2 + 1][q];
      }
      gateup_row<COLS>(P, U, ltile, lane, q, gv, uv);
      continue;
    }
    unit_epilogue<NMAT, COLS>(P, U, ltile, lane, acc0, acc1);
  }
}

// x [T][d] fp32 -> record of hi/lo fp16 halves in MFMA step order (used when
// the bucketing ran on the multi-block path and did not build it)
__global__ void __launch_bounds__(256) build_xrec_kernel(const float *__restrict__ x, int T, int d, int nsb,
                                                         uint16_t *__restrict__ xrec, int xrec_h) {
  moe::build_xrec_range(x, T, d, nsb, xrec, xrec_h, blockIdx.x * blockDim.x + threadIdx.x, gridDim.x * blockDim.x);
}

inline int max_entries(int T, int k, int E, int entry_m) {
  const int pairs = T * k;
  const int a = pairs / entry_m + (pairs < E ? pairs : E);
  return (pairs < a ? pairs : a) + (T + entry_m - 1) / entry_m;
}


// Tokens per work entry of each matrix: gate/up keeps 4 (its unit holds the
// entry's whole x record in LDS: 8 tokens at 13 superblocks would leave room
// for one workgroup per CU); down takes 8 (a 5-superblock h record), so every
// MFMA column is in use and an expert with 5..8 tokens is one entry.
template <int NMAT>
constexpr int cols_of() {
  return NMAT == 2 ? moe::kEntryTokens : moe::kEntryTokens8;
}

// one unit (entry x 4 tiles) per workgroup while that fits in the workgroups
// the CUs hold at once; beyond, workgroups loop over units
template <int NSB, int NMAT, int KS = 1>
hipError_t launch_decode_nsb(const DecodeParams &P, int units, int per_cu, int n_cu, hipStream_t s) {
  const int cap = (per_cu > 0 ? per_cu : 1) * (n_cu > 0 ? n_cu : 1);
  const int grid = (std::min(units, cap) + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL((ffn_decode_kernel<NSB, NMAT, KS, cols_of<NMAT>()>), dim3(grid), dim3(64 * kWaves), 0, s, P);
  return hipGetLastError();
}

template <int NSB, int NMAT, int KS = 1>
hipError_t occupancy_nsb(int *occ) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, ffn_decode_kernel<NSB, NMAT, KS, cols_of<NMAT>()>,
                                                      64 * kWaves, 0);
}

// the kernel built for nsb superblocks: F<NSB>() for nsb = 1..13
template <template <int> class F, typename... A>
hipError_t by_nsb(int nsb, A... a) {
  switch (nsb) {
    case 1: return F<1>::run(a...);
    case 2: return F<2>::run(a...);
    case 3: return F<3>::run(a...);
    case 4: return F<4>::run(a...);
    case 5: return F<5>::run(a...);
    case 6: return F<6>::run(a...);
    case 7: return F<7>::run(a...);
    case 8: return F<8>::run(a...);
    case 9: return F<9>::run(a...);
    case 10: return F<10>::run(a...);
    case 11: return F<11>::run(a...);
    case 12: return F<12>::run(a...);
    case 13: return F<13>::run(a...);
    static_assert(moe::kDecodeMaxNsb == 13, "one case per superblock count");
    default: return hipErrorInvalidValue;
  }
}

template <int NMAT>
struct LaunchMat {
  template <int NSB>
  struct F {
    static hipError_t run(const DecodeParams *P, int units, int per_cu, int n_cu, hipStream_t s) {
      return launch_decode_nsb<NSB, NMAT>(*P, units, per_cu, n_cu, s);
    }
  };
};

template <int NMAT>
struct OccMat {
  template <int NSB>
  struct F {
    static hipError_t run(int *occ) { return occupancy_nsb<NSB, NMAT>(occ); }
  };
};

}  // namespace

namespace moe {

hipError_t decode_occupancy(moe_ctx *c) {
  c->decode_occ[0] = c->decode_occ[1] = c->decode_occ[2] = c->decode_occ[3] = 1;
  // widths the decode kernels are not built for take the prefill path only
  if (c->L.gate.nsb > kDecodeMaxNsb || c->L.down.nsb > kDecodeMaxNsb) return hipSuccess;
  hipError_t e = by_nsb<OccMat<2>::F>(c->L.gate.nsb, &c->decode_occ[0]);
  if (e == hipSuccess) e = by_nsb<OccMat<1>::F>(c->L.down.nsb, &c->decode_occ[1]);
  if (e == hipSuccess && c->L.gate.nsb == 13) e = occupancy_nsb<13, 2, 2>(&c->decode_occ[2]);
  if (e == hipSuccess && c->L.gate.nsb == 13) e = occupancy_nsb<13, 2, 4>(&c->decode_occ[3]);
  return e;
}

hipError_t launch_ffn_decode(const moe_ctx *c, int layer, const float *x, int T, const int32_t *idx,
                             const int32_t *slot_of_pair, float *y_pairs, float *y_shared, hipStream_t s) {
  const moe_config &k = c->cfg;
  const int xh = xrec_halves(c->L.gate.nsb);
  // bucketing, work list and (on the single-workgroup path) the x record in one launch
  hipError_t e =
      launch_bucket_ex(c, idx, T, c->offsets_ws, c->perm_ws, true, moe::kEntryTokens, x, c->xrec, xh, s, c->work8);
  if (e != hipSuccess) return e;
  if (T * k.top_k > 1024) {
    const int n = T * c->L.gate.nsb * kSteps * 8;
    hipLaunchKernelGGL(build_xrec_kernel, dim3((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096), dim3(256), 0, s, x,
                       T, k.d_model, c->L.gate.nsb, c->xrec, xh);
  }
  return launch_ffn_decode_kernels(c, layer, T, slot_of_pair, y_pairs, y_shared, s);
}

hipError_t launch_ffn_decode_kernels(const moe_ctx *c, int layer, int T, const int32_t *slot_of_pair, float *y_pairs,
                                     float *y_shared, hipStream_t s) {
  const moe_config &k = c->cfg;
  const int xh = xrec_halves(c->L.gate.nsb);
  hipError_t e = hipSuccess;
  DecodeParams P;
  P.work = c->work;
  P.work8 = c->work8;
  P.n_work = c->n_work;
  P.perm = c->perm_ws;
  P.slot_of_pair = slot_of_pair;
  P.slot_pool = (const uint8_t *)k.slot_pool;
  P.shared_pool = (const uint8_t *)k.shared_pool;
  P.stride = c->L.stride;
  P.layer = layer;
  P.n_slots = k.n_slots;
  P.max_work = c->max_work;
  P.max_work8 = c->max_work8;
  P.E = k.n_experts;
  P.k = k.top_k;
  P.T = T;
  P.gate = c->L.gate;
  P.up = c->L.up;
  P.down = c->L.down;
  P.xrec = c->xrec;
  P.xrec_h = xh;
  P.hrec = c->hrec;
  P.hrec_h = xrec_halves(c->L.down.nsb);
  P.xrec_zero = c->xrec + (size_t)k.max_tokens * xh;
  P.hrec_zero = c->hrec + (size_t)(c->max_pairs + k.max_tokens) * P.hrec_h;
  P.y_pairs = y_pairs;
  P.y_shared = y_shared;
  P.d_model = k.d_model;
  P.d_ff = k.d_ff;
  const int ents = max_entries(T, k.top_k, k.n_experts, cols_of<2>());
  const int ents_d = max_entries(T, k.top_k, k.n_experts, cols_of<1>());
  const int u1 = ents * ((k.d_ff / 16 + kWaves - 1) / kWaves), u2 = ents_d * ((k.d_model / 16 + kWaves - 1) / kWaves);
  // Small batches (a single request's 1 + 4 verified tokens, ~30 entries)
  // leave most CUs idle in gate/up: split its K over the waves instead.  Up
  // to 32 tokens the split is also ahead on average (half-length chains in
  // twice the waves; at 15 tokens 51.4 -> 50.2 us per call).
  // Built for the 13-superblock rows of d_model = 1,921..2,080.
  // A batch whose quarter-K units (one tile each) all fit in the workgroups
  // the CUs hold at once -- a single token's ~11 entries -- splits K in four.
  if (T <= kSplitMaxTokens && c->L.gate.nsb == 13) {
    const int u1s = ents * ((k.d_ff / 16 + kWaves / 2 - 1) / (kWaves / 2));
    const int u1q = ents * (k.d_ff / 16);
    if (u1q <= c->decode_occ[3] * c->n_cu)
      e = launch_decode_nsb<13, 2, 4>(P, u1q, c->decode_occ[3], c->n_cu, s);
    else
      e = launch_decode_nsb<13, 2, 2>(P, u1s, c->decode_occ[2], c->n_cu, s);
  } else {
    e = by_nsb<LaunchMat<2>::F>(c->L.gate.nsb, &P, u1, c->decode_occ[0], c->n_cu, s);
  }
  if (e != hipSuccess) return e;
  e = by_nsb<LaunchMat<1>::F>(c->L.down.nsb, &P, u2, c->decode_occ[1], c->n_cu, s);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace moe
