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

#include "moe_internal.h"
#include "record.h"

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));

// pair p (0..79) of a superblock: word p/5, slot p%5 (low half) and p%5+5
// (high half); columns 10 (p/5) + p%5 and +5.
using moe::pair_col;

struct DecodeParams {
  const moe::WorkEntry *work;
  const int32_t *n_work;
  const int32_t *perm;
  const int32_t *slot_of_pair;
  const uint8_t *slot_pool;
  const uint8_t *shared_pool;
  uint32_t stride;
  int layer, E, k, T;
  int n_slots;
  int max_work;  // bound on n_work[0] (workspace size)
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

// The 5 block scales of a superblock as R[b] = (s_b, s_b+1) for b < 4 and
// R[4] = (s_4, s_4).  A code pair needs (s_lo, s_hi) = (s_b, s_b) or
// (s_b, s_b+1): the first is R[b] read with its low half in both lanes
// (v_pk_mul op_sel), the second is R[b] itself.  `raw` holds the 5 scales as
// loaded (zero-extended fp16 bits).
__device__ inline void pack_scales(const uint32_t (&raw)[5], h2 (&R)[5]) {
#pragma unroll
  for (int b = 0; b < 4; ++b) R[b] = __builtin_bit_cast(h2, raw[b] | (raw[b + 1] << 16));
  R[4] = __builtin_bit_cast(h2, raw[4] | (raw[4] << 16));
}

template <int p>
__device__ inline h2 pair_scale(const h2 (&R)[5]) {
  constexpr int blo = pair_col(p) / 32, bhi = (pair_col(p) + 5) / 32;
  if constexpr (blo == bhi) {
    return (h2){R[blo][0], R[blo][0]};
  } else {
    return R[blo];
  }
}

// Two weights of one packed word, times f (see record.h): the two 3-bit codes
// of slot j sit at bits 3j' and 16 + 3j' of `src` (src = word for j < 3,
// word >> 9 for j >= 3, j' = j mod 3); one v_and_or_b32 drops them into the
// mantissas of fp16 1024 + f q; one v_pk_add takes 1024 + 4 f off (exact:
// f (q - 4)); one v_pk_mul applies the block scales (one rounding, and the
// product is f times fp16((q - 4) s) because f is a power of two).
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
__device__ inline h2 deq_pair(uint32_t src, const Consts &K, h2 sc) {
  constexpr int jj = j % 3;
  const uint32_t u = (src & K.mask[jj]) | K.magic;
  const h2 v = __builtin_bit_cast(h2, u);
  constexpr float off = 1024.0f + 4.0f * (jj == 0 ? 1.0f : (jj == 1 ? 8.0f : 64.0f));
  const h2 o = {(_Float16)off, (_Float16)off};
  return (v - o) * sc;
}

template <int p>
__device__ inline h2 deq(const uint32_t (&w)[16], const Consts &K, const h2 (&sc)[5]) {
  constexpr int j = p % 5;
  return deq_pair<j>(j < 3 ? w[p / 5] : (w[p / 5] >> 9), K, pair_scale<p>(sc));
}

template <int t>
__device__ inline h8 build_a(const uint32_t (&w)[16], const Consts &K, const h2 (&sc)[5]) {
  constexpr int p0 = 4 * t;
  const h2 a0 = deq<p0 + 0>(w, K, sc);
  const h2 a1 = deq<p0 + 1>(w, K, sc);
  const h2 a2 = deq<p0 + 2>(w, K, sc);
  const h2 a3 = deq<p0 + 3>(w, K, sc);
  return (h8){a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
}

__device__ inline f4 mfma(h8 a, h8 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }

using moe::rec_pos;

// a work entry is used only if it indexes inside this call's pairs / tokens
__device__ inline bool entry_ok(const DecodeParams &P, const moe::WorkEntry &we) {
  if (we.m < 1 || we.m > moe::kEntryTokens || we.first < 0) return false;
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
// Work decomposition.  A unit is one entry (<= 8 tokens of one expert) times
// kWaves consecutive 16-row tiles; a workgroup of kWaves waves takes a unit,
// each wave one tile over the whole K range, so no partial sums cross waves.
// K is walked in rounds of 4 superblocks: in round R lane group g = lane / 16
// owns superblock 4R + g (20 MFMA steps).  Per round:
//   * weights: wave instruction i loads superblock 4R + i of the wave's 16
//     rows, lane group g taking word quad g -- every row's 64 bytes in one
//     instruction -- and four v_permlane32/16_swap passes transpose the 4x4
//     (instruction, lane group) blocks so that lane group g holds the four
//     quads of superblock 4R + g;
//   * activations and scales, which the kWaves tiles share, are copied by the
//     whole workgroup straight into LDS (global_load_lds), activations in the
//     order [superblock][step][hi, lo][entry column] so that the 8 columns a
//     read serves sit in 8 consecutive 16-byte slots;
//   * everything for round R+1 is requested before round R is computed, into
//     the other LDS buffer and the other register set; one barrier per round.
// In gate/up, a lane group past the last superblock computes on zero words
// against zero activations and adds exactly 0; the down kernel splits its
// last round instead (below).  Words of a partial
// last superblock that lie past the row are read from the bytes that follow
// it inside the blob (the next row, or the matrix's scale array, at least 64
// bytes) and also meet zero activations; scale reads are clamped to the row.
// ---------------------------------------------------------------------------

constexpr int kWaves = 4;
constexpr int kXcds = 8;  // accelerator dies of MI355X, each with its own L2
constexpr int kXBytes = 4 * moe::kSteps * 2 * 8 * 16;  // one round's activations: 20 KB
constexpr int kXInst = kXBytes / 1024;                  // 16-byte-per-lane copies of them
constexpr int kScDwords = 10;                           // one row's scales for one round: 4 x 5 blocks, 40 bytes
constexpr int kScBytesPerMat = kScDwords * kWaves * 16 * 4;
static_assert(kXInst % kWaves == 0, "activation copies split evenly over the waves");

struct Unit {
  const uint8_t *blob;  // the expert's blob (a readable stand-in when the entry is unusable)
  int tile0;            // first 16-row tile of the unit
  int m;                // entry columns in use (0 for an unusable entry)
  int routed;
  // this lane's entry column (lane % 8)
  int has_tok, tok, rrow;
  // byte offsets inside a matrix: this lane's weight row (+ its quad) and,
  // for the scale copies, row tile0 * 16 + lane
  uint32_t w_off, s_off;
};

template <int NMAT>
struct Mats;

__device__ inline void unit_setup(const DecodeParams &P, const moe::MatLayout &M0, int u, int tpu, int lane, Unit &U) {
  const moe::WorkEntry we = P.work[u / tpu];
  const int w = threadIdx.x >> 6, r16 = lane & 15, g = lane >> 4;
  U.tile0 = (u % tpu) * kWaves;
  U.routed = we.expert >= 0;
  const uint8_t *blob = entry_ok(P, we) ? entry_blob(P, we) : nullptr;
  U.m = blob ? we.m : 0;
  U.blob = blob ? blob : P.shared_pool + (size_t)P.layer * P.stride;
  U.tok = 0;
  U.rrow = 0;
  U.has_tok = (lane & 7) < U.m && entry_token(P, we, lane & 7, U.tok, U.rrow);
  const int wrow = min((U.tile0 + w) * 16 + r16, M0.rows - 1);
  U.w_off = (uint32_t)wrow * M0.wpr * 4 + g * 16;
  const int srow = min(U.tile0 * 16 + lane, M0.rows - 1);
  U.s_off = (uint32_t)srow * M0.nblk * 2;
}

// matrices of one kernel: gate and up (NMAT 2) or down (NMAT 1)
template <int NMAT>
struct Mats {
  moe::MatLayout m[NMAT];
  const uint16_t *rec, *zero;  // activation record and its all-zero row
  int rec_h;
};

// Activation copy i of wave w moves slots p = 64 (w + 4 i) + lane, slot
// p = ((sb * 20 + t) * 2 + half) * 8 + n with n = lane % 8; since the record
// is contiguous in (superblock, step), the source is step m = 16 i + 4 w +
// lane / 16 counted from the round's first superblock.
// Scale copy q = mat * 10 + j moves dword j of the round's 40 scale bytes of
// rows tile0 * 16 + lane; LDS holds them as [mat][j][64 rows].
template <int NMAT>
__device__ inline void stage_round(const Mats<NMAT> &Mt, const Unit &U, int R, int w, int lane, uint8_t *lx,
                                   uint8_t *lsc) {
  const int nsb = Mt.m[0].nsb, nblk = Mt.m[0].nblk;
  const uint16_t *mine = Mt.rec + (size_t)(NMAT == 2 ? U.tok : U.rrow) * Mt.rec_h + ((lane >> 3) & 1) * 8 +
                         (size_t)R * 4 * moe::kSteps * 16;
  const int m0 = 4 * w + (lane >> 4);
  const int lim = U.has_tok ? moe::kSteps * (nsb - 4 * R) : 0;  // steps of the round that exist
#pragma unroll
  for (int i = 0; i < kXInst / kWaves; ++i) {
    const int m = 16 * i + m0;
    const uint16_t *src = m < lim ? mine + m * 16 : Mt.zero;
    __builtin_amdgcn_global_load_lds(src, lx + 1024 * (w + kWaves * i), 16, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < (NMAT * kScDwords + kWaves - 1) / kWaves; ++i) {
    const int q = w + kWaves * i;
    if (q < NMAT * kScDwords) {
      const int mat = q / kScDwords, j = q % kScDwords;
      // select, not index: a runtime index into Mt.m would put it in scratch memory
      const uint32_t base = mat == 0 ? Mt.m[0].scale_off : Mt.m[NMAT - 1].scale_off;
      const uint32_t off = base + min(kScDwords * 4 * R + 4 * j, 2 * nblk - 4);
      __builtin_amdgcn_global_load_lds(U.blob + off + U.s_off, lsc + 256 * q, 4, 0, 0);
    }
  }
}

template <int NMAT>
__device__ inline void load_round_words(const Mats<NMAT> &Mt, const Unit &U, int R, uint4 (&A)[NMAT][4]) {
  const int nsb = Mt.m[0].nsb;
#pragma unroll
  for (int mat = 0; mat < NMAT; ++mat)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // past the last superblock: no load (the activations there are zero)
      A[mat][i] = make_uint4(0u, 0u, 0u, 0u);
      if (4 * R + i < nsb)
        A[mat][i] = *reinterpret_cast<const uint4 *>(U.blob + Mt.m[mat].code_off + (4 * R + i) * 64 + U.w_off);
    }
}

__device__ inline void swap32(uint32_t &a, uint32_t &b) {
  const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}
__device__ inline void swap16(uint32_t &a, uint32_t &b) {
  const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}

// A[i] of lane group g = quad g of superblock i  ->  A[j] of lane group g =
// quad j of superblock g.  permlane32_swap exchanges the upper half-wave of
// its first operand with the lower half of its second; permlane16_swap the
// odd 16-lane rows of the first with the even rows of the second.
__device__ inline void transpose_quads(uint4 (&A)[4]) {
  swap32(A[0].x, A[2].x); swap32(A[0].y, A[2].y); swap32(A[0].z, A[2].z); swap32(A[0].w, A[2].w);
  swap32(A[1].x, A[3].x); swap32(A[1].y, A[3].y); swap32(A[1].z, A[3].z); swap32(A[1].w, A[3].w);
  swap16(A[0].x, A[1].x); swap16(A[0].y, A[1].y); swap16(A[0].z, A[1].z); swap16(A[0].w, A[1].w);
  swap16(A[2].x, A[3].x); swap16(A[2].y, A[3].y); swap16(A[2].z, A[3].z); swap16(A[2].w, A[3].w);
}

__device__ inline void words_of(const uint4 (&A)[4], uint32_t (&wd)[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    wd[4 * i + 0] = A[i].x;
    wd[4 * i + 1] = A[i].y;
    wd[4 * i + 2] = A[i].z;
    wd[4 * i + 3] = A[i].w;
  }
}

__device__ inline h8 lds_h8(const uint8_t *p) { return *reinterpret_cast<const h8 *>(p); }

// step t: x operand from LDS (read two steps ahead), one MFMA per matrix
template <int NMAT, int t>
__device__ inline void lstep(const uint32_t (&wa)[16], const h2 (&sa)[5], const uint32_t (&wb)[16],
                             const h2 (&sb)[5], const Consts &K, h8 (&xr)[2], const uint8_t *xb, f4 &acc0,
                             f4 &acc1) {
  const h8 x = xr[t & 1];
  if constexpr (t + 2 < moe::kSteps) xr[t & 1] = lds_h8(xb + (t + 2) * 256);
  if constexpr (NMAT == 2) {
    acc0 = mfma(build_a<t>(wa, K, sa), x, acc0);
    acc1 = mfma(build_a<t>(wb, K, sb), x, acc1);
  } else if constexpr (t % 2 == 0) {
    acc0 = mfma(build_a<t>(wa, K, sa), x, acc0);
  } else {
    acc1 = mfma(build_a<t>(wa, K, sa), x, acc1);
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <int... ts>
struct StepSeq {};
using AllSteps = StepSeq<0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16, 17, 18, 19>;

template <int NMAT, int... ts>
__device__ inline void lsteps(StepSeq<ts...>, const uint32_t (&wa)[16], const h2 (&sa)[5], const uint32_t (&wb)[16],
                              const h2 (&sb)[5], const Consts &K, h8 (&xr)[2], const uint8_t *xb, f4 &acc0,
                              f4 &acc1) {
  (lstep<NMAT, ts>(wa, sa, wb, sb, K, xr, xb, acc0, acc1), ...);
}

template <int NMAT>
__device__ inline void compute_round(const uint4 (&A)[NMAT][4], const uint8_t *lx, const uint8_t *lsc, int w,
                                     int lane, const Consts &K, f4 &acc0, f4 &acc1) {
  // per-lane offsets computed here, not held in registers across the loop
  asm volatile("" : "+v"(lane), "+v"(w));
  const int r16 = lane & 15, g = lane >> 4, tcol = lane & 7, half = (lane >> 3) & 1;
  uint32_t wa[16], wb[16];
  h2 sa[5], sb[5];
  words_of(A[0], wa);
  // block 5 g + k of the round sits in dword (5 g + k) / 2, half (5 g + k) % 2
  uint32_t raw[5];
  const uint8_t *sc = lsc + (w * 16 + r16) * 4;
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    const int b = 5 * g + k;
    raw[k] = *reinterpret_cast<const uint16_t *>(sc + (b >> 1) * 256 + (b & 1) * 2);
  }
  pack_scales(raw, sa);
  if constexpr (NMAT == 2) {
    words_of(A[1], wb);
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      const int b = 5 * g + k;
      raw[k] = *reinterpret_cast<const uint16_t *>(sc + kScBytesPerMat + (b >> 1) * 256 + (b & 1) * 2);
    }
    pack_scales(raw, sb);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) wb[i] = 0;
#pragma unroll
    for (int k = 0; k < 5; ++k) sb[k] = sa[k];
  }
  const uint8_t *xb = lx + 16 * ((g * moe::kSteps * 2 + half) * 8 + tcol);
  h8 xr[2] = {lds_h8(xb), lds_h8(xb + 256)};
  lsteps<NMAT>(AllSteps{}, wa, sa, wb, sb, K, xr, xb, acc0, acc1);
}

// ---------------------------------------------------------------------------
// Split last round.  When the last round holds r < 4 superblocks, lane groups
// past r would compute a whole round on zeros.  Instead the words are left as
// loaded (lane group g holds word quad g of superblock 4R + i in A[i]) and
// each superblock is 5 MFMA steps: lane group g takes steps 5 g .. 5 g + 4 of
// it, i.e. pairs 20 g .. 20 g + 19 (quad g), whose activations are the
// record's steps 5 g + t'.  Quad g spans blocks g and g + 1 of the
// superblock (its first column is 40 g, and 40 g / 32 = g); a pair's two
// columns are (g, g), (g, g + 1) or (g + 1, g + 1), which depends on g, so the
// scale register of each pair is picked per lane with v_cndmask.
// ---------------------------------------------------------------------------

// scale class of local pair q (0..19) of quad g: 0 = both columns in block g,
// 2 = low in g and high in g + 1, 3 = both in g + 1
constexpr int quad_cls(int g, int q) {
  const int col = 40 * g + pair_col(q);
  return (col / 32 - g) + 2 * ((col + 5) / 32 - g);
}

struct QuadScales {
  h2 s00, s01, s11;
};

__device__ inline h2 cls_reg(const QuadScales &S, int c) { return c == 0 ? S.s00 : (c == 2 ? S.s01 : S.s11); }

// the class only grows with g (the quad's offset inside its first block is
// 0, 8, 16, 24), so one select per change of class; ge[k] = (g >= k)
template <int q>
__device__ inline h2 tail_scale(const QuadScales &S, const bool (&ge)[4]) {
  constexpr int c0 = quad_cls(0, q), c1 = quad_cls(1, q), c2 = quad_cls(2, q), c3 = quad_cls(3, q);
  static_assert(c0 <= c1 && c1 <= c2 && c2 <= c3, "class grows with the lane group");
  h2 r = cls_reg(S, c0);
  if constexpr (c1 != c0) r = ge[1] ? cls_reg(S, c1) : r;
  if constexpr (c2 != c1) r = ge[2] ? cls_reg(S, c2) : r;
  if constexpr (c3 != c2) r = ge[3] ? cls_reg(S, c3) : r;
  return r;
}

// scales of blocks b and b + 1 of this lane's row (LDS [dword][row] copy)
__device__ inline QuadScales quad_scales(const uint8_t *sc, int b) {
  const uint32_t r0 = *reinterpret_cast<const uint16_t *>(sc + (b >> 1) * 256 + (b & 1) * 2);
  const uint32_t r1 = *reinterpret_cast<const uint16_t *>(sc + ((b + 1) >> 1) * 256 + ((b + 1) & 1) * 2);
  QuadScales S;
  S.s00 = __builtin_bit_cast(h2, r0 | (r0 << 16));
  S.s01 = __builtin_bit_cast(h2, r0 | (r1 << 16));
  S.s11 = __builtin_bit_cast(h2, r1 | (r1 << 16));
  return S;
}

template <int q>
__device__ inline h2 tail_deq(const uint32_t (&w)[4], const Consts &K, const QuadScales &S, const bool (&ge)[4]) {
  constexpr int j = q % 5;
  return deq_pair<j>(j < 3 ? w[q / 5] : (w[q / 5] >> 9), K, tail_scale<q>(S, ge));
}

template <int t>
__device__ inline h8 tail_a(const uint32_t (&w)[4], const Consts &K, const QuadScales &S, const bool (&ge)[4]) {
  const h2 a0 = tail_deq<4 * t + 0>(w, K, S, ge);
  const h2 a1 = tail_deq<4 * t + 1>(w, K, S, ge);
  const h2 a2 = tail_deq<4 * t + 2>(w, K, S, ge);
  const h2 a3 = tail_deq<4 * t + 3>(w, K, S, ge);
  return (h8){a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
}

template <int NMAT, int t>
__device__ inline void tail_step(const uint32_t (&wa)[4], const QuadScales &Sa, const uint32_t (&wb)[4],
                                 const QuadScales &Sb, const Consts &K, const bool (&ge)[4], const uint8_t *xb,
                                 f4 &acc0, f4 &acc1) {
  const h8 x = lds_h8(xb + t * 256);
  if constexpr (NMAT == 2) {
    acc0 = mfma(tail_a<t>(wa, K, Sa, ge), x, acc0);
    acc1 = mfma(tail_a<t>(wb, K, Sb, ge), x, acc1);
  } else if constexpr (t % 2 == 0) {
    acc0 = mfma(tail_a<t>(wa, K, Sa, ge), x, acc0);
  } else {
    acc1 = mfma(tail_a<t>(wa, K, Sa, ge), x, acc1);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// superblock i of a split round
template <int NMAT, int i>
__device__ inline void tail_superblock(const uint4 (&A)[NMAT][4], const uint8_t *lx, const uint8_t *lsc, int w,
                                       int lane, const Consts &K, const bool (&ge)[4], f4 &acc0, f4 &acc1) {
  const int r16 = lane & 15, g = lane >> 4, tcol = lane & 7, half = (lane >> 3) & 1;
  const uint8_t *sc = lsc + (w * 16 + r16) * 4;
  const uint32_t wa[4] = {A[0][i].x, A[0][i].y, A[0][i].z, A[0][i].w};
  const QuadScales Sa = quad_scales(sc, 5 * i + g);
  uint32_t wb[4] = {0u, 0u, 0u, 0u};
  QuadScales Sb = Sa;
  if constexpr (NMAT == 2) {
    wb[0] = A[NMAT - 1][i].x;
    wb[1] = A[NMAT - 1][i].y;
    wb[2] = A[NMAT - 1][i].z;
    wb[3] = A[NMAT - 1][i].w;
    Sb = quad_scales(sc + kScBytesPerMat, 5 * i + g);
  }
  const uint8_t *xb = lx + 16 * ((((i * moe::kSteps + 5 * g) * 2) + half) * 8 + tcol);
  tail_step<NMAT, 0>(wa, Sa, wb, Sb, K, ge, xb, acc0, acc1);
  tail_step<NMAT, 1>(wa, Sa, wb, Sb, K, ge, xb, acc0, acc1);
  tail_step<NMAT, 2>(wa, Sa, wb, Sb, K, ge, xb, acc0, acc1);
  tail_step<NMAT, 3>(wa, Sa, wb, Sb, K, ge, xb, acc0, acc1);
  tail_step<NMAT, 4>(wa, Sa, wb, Sb, K, ge, xb, acc0, acc1);
}

// a split round of r (1..3) superblocks
template <int NMAT>
__device__ inline void compute_tail(const uint4 (&A)[NMAT][4], int r, const uint8_t *lx, const uint8_t *lsc, int w,
                                    int lane, const Consts &K, f4 &acc0, f4 &acc1) {
  // opaque copy: keeps the tail's per-lane addresses and masks from being
  // hoisted out of the stream loop, where they would hold registers all along
  asm volatile("" : "+v"(lane), "+v"(w));
  const int g = lane >> 4;
  const bool ge[4] = {true, g >= 1, g >= 2, g >= 3};
  tail_superblock<NMAT, 0>(A, lx, lsc, w, lane, K, ge, acc0, acc1);
  if (r > 1) tail_superblock<NMAT, 1>(A, lx, lsc, w, lane, K, ge, acc0, acc1);
  if (r > 2) tail_superblock<NMAT, 2>(A, lx, lsc, w, lane, K, ge, acc0, acc1);
}

// gate/up: h = silu(g) u into the h record; down: y
template <int NMAT>
__device__ inline void unit_epilogue(const DecodeParams &P, const Unit &U, int w, int lane, f4 acc0, f4 acc1) {
  const int r16 = lane & 15, g = lane >> 4;
  const int rows = NMAT == 2 ? P.d_ff : P.d_model;
  const int rt = U.tile0 + w;
  // D layout: lane holds rows 4g + i of the tile for MFMA column r16; the
  // token's value is column r16 (hi) + column r16 + 8 (lo)
  if constexpr (NMAT == 1) acc0 += acc1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc0[i] += __shfl_xor(acc0[i], 8, 64);
    if constexpr (NMAT == 2) acc1[i] += __shfl_xor(acc1[i], 8, 64);
  }
  if (!(U.has_tok && r16 < 8 && rt * 16 < rows)) return;
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

__device__ inline void wait_loads_and_sync() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

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

// One round of the stream: request (un, Rn) into the other buffers, compute
// (u, R) from the current ones, finish the unit after its last round.
// Returns false when the stream ends.
template <int NMAT>
__device__ inline bool stream_round(const DecodeParams &P, const Mats<NMAT> &Mt, int tpu, int u_end, int u_step,
                                    int rounds, int split_r,
                                    int w, int lane, int &u, int &R, Unit &U, uint8_t *lx_cur, uint8_t *lsc_cur,
                                    uint8_t *lx_nxt, uint8_t *lsc_nxt, const uint4 (&Acur)[NMAT][4],
                                    uint4 (&Anxt)[NMAT][4], const Consts &K, f4 &acc0, f4 &acc1) {
  const bool last = R + 1 == rounds;
  const int un = last ? u + u_step : u;
  const int Rn = last ? 0 : R + 1;
  const bool more = un < u_end;
  Unit Un = U;
  if (last && more) unit_setup(P, Mt.m[0], un, tpu, lane, Un);
  if (more) {
    stage_round<NMAT>(Mt, Un, Rn, w, lane, lx_nxt, lsc_nxt);
    load_round_words<NMAT>(Mt, Un, Rn, Anxt);
  }
  if (last && split_r)
    compute_tail<NMAT>(Acur, split_r, lx_cur, lsc_cur, w, lane, K, acc0, acc1);
  else
    compute_round<NMAT>(Acur, lx_cur, lsc_cur, w, lane, K, acc0, acc1);
  if (last) {
    unit_epilogue<NMAT>(P, U, w, lane, acc0, acc1);
    acc0 = acc1 = (f4){0.f, 0.f, 0.f, 0.f};
  }
  if (!more) return false;
  wait_loads_and_sync();
  if (!(split_r && Rn + 1 == rounds))
#pragma unroll
    for (int mat = 0; mat < NMAT; ++mat) transpose_quads(Anxt[mat]);
  u = un;
  R = Rn;
  U = Un;
  return true;
}

template <int NMAT>
__global__ void __launch_bounds__(64 * kWaves, 3) ffn_decode_kernel(DecodeParams P) {
  __shared__ __attribute__((aligned(1024))) uint8_t lx[2][kXBytes];
  __shared__ __attribute__((aligned(256))) uint8_t lsc[2][NMAT * kScBytesPerMat];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const Mats<NMAT> Mt = mats_of<NMAT>(P);
  const int ntile = Mt.m[0].rows / 16;
  const int tpu = (ntile + kWaves - 1) / kWaves;
  const int rounds = (Mt.m[0].nsb + 3) / 4;
  // superblocks of a split last round (0: none).  Down only: 768 columns are
  // 5 superblocks, so a whole second round would be 3/4 idle.  Gate/up keeps
  // whole rounds (13 superblocks, the last round 1/4 used): with both paths
  // in that kernel the register allocator spills and the kernel ran slower.
  const int split_r = NMAT == 1 ? Mt.m[0].nsb % 4 : 0;
  const int n_units = min(P.n_work[0], P.max_work) * tpu;
  // Workgroup b runs on XCD b % 8 (round-robin dispatch).  Each XCD takes a
  // contiguous range of units, so the tiles of neighbouring entries -- both
  // entries of an expert with more than 8 tokens, or of the shared expert --
  // stream through one L2 and the second read of a blob hits it.
  const int per = (n_units + kXcds - 1) / kXcds;
  const int xcd = blockIdx.x % kXcds, u_step = gridDim.x / kXcds;
  const int u_end = min((xcd + 1) * per, n_units);
  int u = xcd * per + blockIdx.x / kXcds, R = 0;
  if (u >= u_end) return;
  Unit U;
  unit_setup(P, Mt.m[0], u, tpu, lane, U);
  uint4 A0[NMAT][4], A1[NMAT][4];
  stage_round<NMAT>(Mt, U, 0, w, lane, lx[0], lsc[0]);
  load_round_words<NMAT>(Mt, U, 0, A0);
  wait_loads_and_sync();
  if (!(split_r && rounds == 1))
#pragma unroll
    for (int mat = 0; mat < NMAT; ++mat) transpose_quads(A0[mat]);
  const Consts K = make_consts();
  f4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  // the two register sets and LDS buffers alternate by round
  while (stream_round<NMAT>(P, Mt, tpu, u_end, u_step, rounds, split_r, w, lane, u, R, U, lx[0], lsc[0], lx[1], lsc[1], A0,
                            A1, K, acc0, acc1) &&
         stream_round<NMAT>(P, Mt, tpu, u_end, u_step, rounds, split_r, w, lane, u, R, U, lx[1], lsc[1], lx[0], lsc[0], A1,
                            A0, K, acc0, acc1)) {
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

}  // namespace

namespace moe {

hipError_t launch_bucket_ex(const moe_ctx *c, const int32_t *idx, int T, int32_t *offsets, int32_t *perm, bool build,
                            int entry_m, const float *x, uint16_t *xrec, int xrec_h, hipStream_t s);

hipError_t launch_ffn_decode(const moe_ctx *c, int layer, const float *x, int T, const int32_t *idx,
                             const int32_t *slot_of_pair, float *y_pairs, float *y_shared, hipStream_t s) {
  const moe_config &k = c->cfg;
  const int xh = xrec_halves(c->L.gate.nsb);
  // bucketing, work list and (on the single-workgroup path) the x record in one launch
  hipError_t e = launch_bucket_ex(c, idx, T, c->offsets_ws, c->perm_ws, true, moe::kEntryTokens, x, c->xrec, xh, s);
  if (e != hipSuccess) return e;
  if (T * k.top_k > 1024) {
    const int n = T * c->L.gate.nsb * kSteps * 8;
    hipLaunchKernelGGL(build_xrec_kernel, dim3((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096), dim3(256), 0, s, x,
                       T, k.d_model, c->L.gate.nsb, c->xrec, xh);
  }
  DecodeParams P;
  P.work = c->work;
  P.n_work = c->n_work;
  P.perm = c->perm_ws;
  P.slot_of_pair = slot_of_pair;
  P.slot_pool = (const uint8_t *)k.slot_pool;
  P.shared_pool = (const uint8_t *)k.shared_pool;
  P.stride = c->L.stride;
  P.layer = layer;
  P.n_slots = k.n_slots;
  P.max_work = c->max_work;
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
  const int ents = max_entries(T, k.top_k, k.n_experts, moe::kEntryTokens);
  // one unit (entry x 4 tiles) per workgroup while that fits; beyond,
  // workgroups loop over units and overlap one unit's start with the previous
  // unit's last round
  const int cap = 768;  // three workgroups per CU; a multiple of kXcds
  auto grid = [&](int units) { return (std::min(units, cap) + kXcds - 1) / kXcds * kXcds; };
  const int u1 = ents * ((k.d_ff / 16 + kWaves - 1) / kWaves), u2 = ents * ((k.d_model / 16 + kWaves - 1) / kWaves);
  hipLaunchKernelGGL(ffn_decode_kernel<2>, dim3(grid(u1)), dim3(64 * kWaves), 0, s, P);
  hipLaunchKernelGGL(ffn_decode_kernel<1>, dim3(grid(u2)), dim3(64 * kWaves), 0, s, P);
  return hipGetLastError();
}

}  // namespace moe
