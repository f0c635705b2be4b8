// Prefill path of the expert FFN: many tokens per expert, a real dense
// contraction, so it runs as a grouped GEMM on MFMA.
//
// The pages' engine runs prefill in chunks of 12,288 tokens on one card ("一张
// RTX 4090 跑千亿模型，Strata 实测 155 tok/s", section 加个草稿层); every token
// of a chunk is routed to 10 of 512 experts, so one chunk is 122,880
// (token, expert) pairs grouped per expert, plus the shared expert's 12,288.
//
// Precision: the dequantised weights enter the MFMA rounded once to fp16
// (dequant.h), as on the decode path; the activations x and h = silu(g) u
// are carried at fp32 accuracy as two fp16 halves, hi = fp16(v) and
// lo = fp16(v - hi), each multiplied into the same fp32 accumulator.
// Rounding x and h to fp16 as well puts a real-shape layer about 2.3e-3 x
// RMS from the exact definition, and rounding h alone still reaches it on
// small layers: both are above the 2e-3 bar.
//
// Work: a workgroup of 8 waves takes one work entry (<= 128 tokens of one
// expert) against a block of weight rows -- gate/up: 256 rows of gate and the
// same 256 rows of up (the epilogue writes h for them); down: 512 rows.  Each
// wave owns 4 16-row tiles (gate/up: 2 of gate and the same 2 of up) against
// all 128 tokens: 4 x 8 16x16 output tiles, 128 fp32 accumulators per lane.
//   A (16 rows x 32 K)  = weights: each wave's word quads and scale words are
//                         copied to LDS a superblock ahead; each step reads
//                         the one or two words it needs (the scale pairs
//                         once per superblock) and dequantises the next
//                         step's fragments while its own MFMAs run;
//   B (32 K x 16 tokens) = activations (hi, then lo) from a 4-slot LDS ring
//                         of step tiles that all 8 waves share, filled 3
//                         steps ahead, one barrier per 32-K step.
// Every global load of the K loop is a direct global-to-LDS copy whose
// completion the kernel waits for itself (the counts: prefill_plan.h).  The
// gate/up epilogue stages h in LDS in record order and stores whole 16-byte
// pieces of the h record.
// v_mfma_f32_16x16x32_f16 only.
#include <algorithm>

#include "dequant.h"
#include "lds_copy.h"
#include "moe_internal.h"
#include "prefill_plan.h"

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));  // a plain vector (kept in registers)

constexpr int kPM = 128;                // tokens per work entry
constexpr int kTT = kPM / 16;           // 16-token tiles of an entry
constexpr int kPWaves = 8;              // waves per workgroup (two per SIMD)
constexpr int kPThreads = 64 * kPWaves;
constexpr int kXcds = 8;                // accelerator dies, each with its own L2

// Activation records of this path, one row per token (gate/up: x) or per
// pair row (down: h), in MFMA step order: step s = 5 S + t of superblock S
// holds, for lane group g, the 8 values of pairs 20 g + 4 t .. 20 g + 4 t + 3
// (each pair (c, c+5) as two adjacent halves, divided by the f of its code
// slot), as 128 B = [hi | lo][g][8 halves].
// In LDS a step's tile is [row n][8 granules of 16 B] with granule
// (piece ^ swz(n)) holding `piece` (= hl * 4 + g): the 16 lanes that read one
// MFMA B operand (16 rows, one piece) then touch 16 distinct bank groups.
template <int HL>
struct RecGeom {
  static constexpr int kRowB = 64 * HL;           // bytes of one row per step
  static constexpr int kGran = kRowB / 16;        // 16-byte granules per row per step
  static constexpr int kStepB = kPM * kRowB;      // one step's LDS tile
  static constexpr int kCopies = kPM * kGran / kPThreads;  // granules per thread per step
  __host__ __device__ static constexpr int swz(int n) { return (n >> 1) & 7; }
};
constexpr int kHL = 2;  // halves per value: hi and lo
using Geo = RecGeom<kHL>;
static_assert(Geo::kCopies == moe::pf::kXCopies && Geo::kGran == 8 && Geo::kRowB == moe::pf::kRecRowB,
              "copy roles, swizzle width and record row as the plan has them");
using moe::pf::rec_byte;

struct PrefillParams {
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
  const uint8_t *xrec;  // [T][xrec_b]: x record (hi and lo)
  uint8_t *hrec;        // [T*k + T][hrec_b]: h record (hi and lo)
  int xrec_b, hrec_b;   // bytes per record row
  float *y_pairs, *y_shared;
  int d_model, d_ff;
};

// A wave-uniform read of data that no kernel of this launch writes (the work
// list, the bucketing and the slot map): through the constant address space,
// so it is a scalar load rather than a vector load, whose wait would also
// wait for every copy in flight.
template <class T>
__device__ __attribute__((always_inline)) inline T ld_uniform(const T *p) {
  return *(const __attribute__((address_space(4))) T *)p;
}

__device__ __attribute__((always_inline)) inline const uint8_t *entry_blob(const PrefillParams &P, const moe::WorkEntry &we) {
  if (we.expert < 0) return P.shared_pool + (size_t)P.layer * P.stride;
  const int slot = P.slot_of_pair ? ld_uniform(P.slot_of_pair + ld_uniform(P.perm + we.first)) : P.layer * P.E + we.expert;
  if (slot < 0 || slot >= P.n_slots) return nullptr;  // never read outside the pool
  return P.slot_pool + (size_t)slot * P.stride;
}

// a work entry is used only if it indexes inside this call's pairs / tokens
__device__ __attribute__((always_inline)) inline bool entry_ok(const PrefillParams &P, const moe::WorkEntry &we) {
  if (we.m < 1 || we.m > kPM || we.first < 0) return false;
  return we.expert >= 0 ? (we.expert < P.E && we.first + we.m <= P.T * P.k) : (we.first + we.m <= P.T);
}

// a work entry's fields, one scalar load each (a struct read can be narrowed
// to three dwords, for which there is no scalar load)
__device__ __attribute__((always_inline)) inline moe::WorkEntry ld_entry(const moe::WorkEntry *p) {
  moe::WorkEntry we;
  we.expert = ld_uniform(&p->expert);
  we.first = ld_uniform(&p->first);
  we.m = ld_uniform(&p->m);
  we.pad = 0;
  return we;
}

// The first item at or after `it` (stepping by istep) whose entry has work
// and whose blob exists, with that entry and blob; i_end when none is left.
// Wave-uniform (scalar loads).
__device__ __attribute__((always_inline)) inline int fetch_item(const PrefillParams &P, int it, int istep, int i_end,
                                                                int nrt, moe::WorkEntry &we, const uint8_t *&blob) {
  for (; it < i_end; it += istep) {
    we = ld_entry(P.work + it / nrt);
    if (!entry_ok(P, we)) continue;
    blob = entry_blob(P, we);
    if (blob) break;
  }
  return it;
}

// A routed entry's pair ids into LDS `pairs` (kPM ints) by waves 0 and 1
// with direct copies (column n reads perm[first + min(n, m - 1)], inside the
// entry), which no compiler-inserted wait covers: the K loop's own waits
// (and the drain at its end) cover them.  Nothing for the shared expert.
__device__ __attribute__((always_inline)) inline void copy_pairs(const PrefillParams &P, const moe::WorkEntry &we,
                                                                 int *pairs, int w, int lane) {
  if (we.expert < 0 || w >= kPM / 64) return;  // wave-uniform
  const int n = 64 * w + lane;
  moe::lds_copy4_off(moe::uniform_base(P.perm), 4u * (uint32_t)(we.first + min(n, we.m - 1)),
                     moe::lds_addr(pairs + 64 * w));
}

// record row of entry column n (the pair id, or T*k + token for the shared
// expert), -1 for a column without a token or an out-of-range pair
__device__ __attribute__((always_inline)) inline int entry_row(const PrefillParams &P, const moe::WorkEntry &we, int n,
                                                               const int *pairs) {
  if (n >= we.m) return -1;
  if (we.expert < 0) return P.T * P.k + we.first + n;
  const int pair = pairs[n];
  return pair >= 0 && pair < P.T * P.k ? pair : -1;
}

// token of a record row from entry_row (>= 0)
__device__ __attribute__((always_inline)) inline int row_token(const PrefillParams &P, int row) {
  return row < P.T * P.k ? row / P.k : row - P.T * P.k;
}

__device__ __attribute__((always_inline)) inline f4 mfma(h8 a, h8 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }

// Where the lane's 4 weight rows live, as byte offsets into the entry's blob:
// tile a's words at code + coff[a], its scales at scale + soff[a] (coff and
// soff are the same for the whole wave)
struct WRows {
  uint64_t blob;    // the entry's blob (wave-uniform)
  uint32_t code;    // word quad g of superblock 0 of tile 0's row
  uint32_t scale;   // tile 0's row of scales
  uint32_t coff[4], soff[4];
  int nblk;
};

// K loop.  Every global load in it is a direct global-to-LDS copy that the
// kernel waits for itself (lds_copy.h), so the only memory operations the
// compiler sees are LDS reads, which it counts exactly:
//   * the x (or h) record tile of step s + kXD goes to ring slot (s + kXD) & 3
//     at step s (two 16-byte copies per thread);
//   * at step 0 of superblock S, the next superblock's word quads (one 16-byte
//     copy per tile: lane l's quad lands at 16 l) and, per tile, the three
//     dwords of each of its 16 rows that hold scale blocks 5 S' .. 5 S' + 4
//     (one 4-byte copy by 48 lanes) go to weight slot (S + 1) & 1 (8 copies
//     per wave);
//   * each step starts by waiting until its tile's copies have landed (loads
//     complete in order, so everything issued before them has too), then one
//     barrier publishes the tile to all waves.
// Weights stay in their LDS slot for the superblock: each step reads the one
// or two words of the lane's quad it needs, and the scale pairs are read once
// per superblock; fragments are dequantised a step ahead of their MFMAs.
using moe::pf::kXD;      // x tiles copied this many steps ahead
using moe::pf::kXRing;   // slots of the x ring (> kXD)
using moe::pf::kWCopies; // copies per wave per superblock: 4 quads + 4 scale sets
using moe::pf::vm_after; // the wait count of each step (prefill_plan.h)
constexpr int kQuadB = 1024;                // one tile's quads of one wave: 64 lanes x 16 B
constexpr int kScB = 256;                   // one tile's scale dwords: 16 rows x 3 (64 lane slots)
constexpr int kTileWB = kQuadB + kScB;      // one tile's weights of one superblock
constexpr int kWSlotB = kPWaves * 4 * kTileWB;  // one superblock's weights of the workgroup
static_assert(kXRing > kXD && (kXRing & (kXRing - 1)) == 0, "x ring");
static_assert(kWCopies == 2 * 4, "a quad copy and a scale copy per tile");

template <int N>
__device__ __attribute__((always_inline)) inline void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

struct XCopy {
  uint64_t base;                // the record (wave-uniform)
  uint32_t src[Geo::kCopies];   // byte offset of this thread's granules of step 0 (row, piece)
  uint32_t lds;                 // LDS byte of the wave's first granule inside a step tile
};

// the copies of step s's tile into ring slot s & 3 (s clamped: past the last
// step the last tile is copied again into a slot nobody reads); copy i of the
// wave fills granules 64 (w + 8 i) .. + 63
__device__ __attribute__((always_inline)) inline void copy_x(const XCopy &X, uint32_t ring, int s, int nsteps) {
  const int sc = min(s, nsteps - 1);
  const uint32_t slot = ring + (uint32_t)(s & (kXRing - 1)) * Geo::kStepB;
#pragma unroll
  for (int i = 0; i < Geo::kCopies; ++i)
    moe::lds_copy16_off(X.base, X.src[i] + (uint32_t)sc * Geo::kRowB, slot + X.lds + (uint32_t)(i * kPThreads * 16));
}

// superblock S's weights (S clamped) into weight slot S & 1: per tile the
// lane's quad, and the scale dwords d0 + k (k = 0..2, d0 = floor(5 S / 2),
// each clamped to the row) of row lane / 3 copied by lanes 0..47 (lane
// 3 r + k), which hold blocks 2 d0 .. 2 d0 + 5 -- every block 5 S + g and
// 5 S + g + 1 the row's lanes read
__device__ __attribute__((always_inline)) inline void copy_w(const WRows &R, uint32_t wbase, int S, int nsb, int r16,
                                                             int lane, int w) {
  const int Sc = min(S, nsb - 1);
  const uint32_t slot = wbase + (uint32_t)(S & 1) * kWSlotB + (uint32_t)w * 4 * kTileWB;
  const int crow = lane / 3, dk = min((5 * Sc) / 2 + (lane - 3 * crow), R.nblk / 2 - 1);
  // scale dword dk of row crow (rows are consecutive, crow - r16 rows from the lane's own)
  const uint32_t sco = (uint32_t)((int)R.scale + (crow - r16) * R.nblk * 2 + 4 * dk);
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const uint32_t t0 = slot + (uint32_t)a * kTileWB;
    moe::lds_copy16_off(R.blob, R.code + R.coff[a] + (uint32_t)Sc * 64, t0);
    if (lane < 48) moe::lds_copy4_off(R.blob, sco + R.soff[a], t0 + kQuadB);
  }
}

// superblock S's scale pairs from its LDS slot, one per tile: b0 = min(5 S +
// g, nblk - 1), b1 = min(b0 + 1, nblk - 1) from the row's three dwords (block
// b is half (b - 2 d0) of dword (b - 2 d0) / 2).  Step 4 of the last
// superblock reads for S = nsb, which has no blocks: the clamp can put the
// dword index up to 3 below the row's first, still inside the slot (its quad
// region), and nothing uses those values.
__device__ __attribute__((always_inline)) inline void read_p(const uint8_t *wlds, int S, int g, int r16, int nblk,
                                                             int w, uint32_t (&P)[4]) {
  const uint8_t *slot = wlds + (S & 1) * kWSlotB + w * 4 * kTileWB;
  const int d0 = (5 * S) / 2;
  const int b0 = min(5 * S + g, nblk - 1), b1 = min(b0 + 1, nblk - 1);
  const int j0 = b0 - 2 * d0, j1 = b1 - 2 * d0;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const uint8_t *t0 = slot + a * kTileWB;
    const uint32_t e0 = *reinterpret_cast<const uint32_t *>(t0 + kQuadB + 4 * (3 * r16 + (j0 >> 1)));
    const uint32_t e1 = *reinterpret_cast<const uint32_t *>(t0 + kQuadB + 4 * (3 * r16 + (j1 >> 1)));
    const uint32_t s0 = (j0 & 1) ? e0 >> 16 : e0 & 0xffffu, s1 = (j1 & 1) ? e1 >> 16 : e1 & 0xffffu;
    P[a] = s0 | (s1 << 16);
  }
}

// A fragment of step t of one tile from the lane's word quad in LDS (`quad`):
// only the words holding pairs 4t .. 4t+3 are read
template <int t>
__device__ __attribute__((always_inline)) inline h8 deq_step(const uint8_t *quad, uint32_t P, const moe::Consts &K,
                                                             const uint32_t (&sel)[6]) {
  constexpr int k0 = (4 * t) / 5, k1 = (4 * t + 3) / 5;
  uint32_t q[4] = {0u, 0u, 0u, 0u};
  q[k0] = *reinterpret_cast<const uint32_t *>(quad + 4 * k0);
  if constexpr (k1 != k0) q[k1] = *reinterpret_cast<const uint32_t *>(quad + 4 * k1);
  return moe::quad_a_sel<t>(q, K, P, sel);
}

// One K step (t of superblock S; FIRST: superblock 0): wait for the step's
// tile, publish it, issue the copies of later data, then the wave's 4 row
// tiles x the entry's token tiles, every product twice (the activations' hi
// and lo halves).  The A fragments of the step were dequantised during the
// previous one; this step's MFMAs run beside the dequantisation of the next
// step's (so VALU work fills the matrix pipe's shadow).  At step 4 the next
// superblock's scale pairs replace the registers, whose last use was step 3's
// dequantisation of step 4.  FULL (an entry of kPM tokens): no token tile
// is skipped, so the step is one branch-free block for the scheduler.
template <int t, bool FIRST, bool FULL>
__device__ __attribute__((always_inline)) inline void k_step(int S, int nsb, int nsteps, const WRows &R, int g, int r16,
                                                             int w, int lane, uint32_t (&P)[4], h8 (&A)[4], const XCopy &X,
                                                             uint32_t ring, const uint8_t *xring, uint32_t wbase,
                                                             const uint8_t *wlds, const uint32_t (&sel)[6],
                                                             const moe::Consts &K, int ntt, bool wact, int rl_hi,
                                                             int rl_lo, f4 (&acc)[4][kTT]) {
  using G = Geo;
  const int s = 5 * S + t;
  wait_vm<vm_after(t, FIRST)>();
  __syncthreads();  // step s's tile is in LDS for every wave; slot (s - 1) & 3 is no longer read
  copy_x(X, ring, s + kXD, nsteps);
  if constexpr (t == 0) copy_w(R, wbase, S + 1, nsb, r16, lane, w);
  if (!wact) return;  // wave-uniform: rows past the matrix
  const uint8_t *quads = wlds + w * 4 * kTileWB + 16 * lane;  // tile 0's quad of the lane in slot 0
  if constexpr (FIRST && t == 0) {
    // the very first step has no previous one to dequantise its fragments
    read_p(wlds, 0, g, r16, R.nblk, w, P);
#pragma unroll
    for (int a = 0; a < 4; ++a) A[a] = deq_step<0>(quads + a * kTileWB, P[a], K, sel);
  }
  // superblock S + 1's words landed with step 5 S + 4's tile (copied after them)
  if constexpr (t == 4) read_p(wlds, S + 1, g, r16, R.nblk, w, P);
  constexpr int tn = t == 4 ? 0 : t + 1;
  const uint8_t *qn = quads + ((t == 4 ? S + 1 : S) & 1) * kWSlotB;  // the next step's superblock slot
  h8 An[4];
  // B operands one read ahead of their MFMAs
  const uint8_t *tile = xring + (s & (kXRing - 1)) * G::kStepB;
  h8 cur = *reinterpret_cast<const h8 *>(tile + rl_hi);
#pragma unroll
  for (int nt = 0; nt < kTT; ++nt) {
    if (FULL || nt < ntt) {  // wave-uniform: token tiles holding tokens
      const h8 bl = *reinterpret_cast<const h8 *>(tile + nt * 16 * G::kRowB + rl_lo);
#pragma unroll
      for (int a = 0; a < 4; ++a) acc[a][nt] = mfma(A[a], cur, acc[a][nt]);
      if (nt + 1 < kTT && (FULL || nt + 1 < ntt)) cur = *reinterpret_cast<const h8 *>(tile + (nt + 1) * 16 * G::kRowB + rl_hi);
#pragma unroll
      for (int a = 0; a < 4; ++a) acc[a][nt] = mfma(A[a], bl, acc[a][nt]);
    }
    if (nt < 4) An[nt] = deq_step<tn>(qn + nt * kTileWB, P[nt], K, sel);
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) A[a] = An[a];
}

template <bool FIRST, bool FULL>
__device__ __attribute__((always_inline)) inline void k_superblock(int S, int nsb, int nsteps, const WRows &R, int g,
                                                                   int r16, int w, int lane, uint32_t (&P)[4], h8 (&A)[4],
                                                                   const XCopy &X, uint32_t ring, const uint8_t *xring,
                                                                   uint32_t wbase, const uint8_t *wlds,
                                                                   const uint32_t (&sel)[6], const moe::Consts &K,
                                                                   int ntt, bool wact, int rl_hi, int rl_lo,
                                                                   f4 (&acc)[4][kTT]) {
#define MOE_K_STEP(t) \
  k_step<t, FIRST, FULL>(S, nsb, nsteps, R, g, r16, w, lane, P, A, X, ring, xring, wbase, wlds, sel, K, ntt, wact, rl_hi, rl_lo, acc)
  MOE_K_STEP(0);
  MOE_K_STEP(1);
  MOE_K_STEP(2);
  MOE_K_STEP(3);
  MOE_K_STEP(4);
#undef MOE_K_STEP
}

// NMAT = 2: gate/up -> h record; NMAT = 1: down -> y.  One workgroup per CU
// walks its accelerator die's share of the (entry, row block) items.
// Gate/up epilogue staging: the h values of 64 tokens at a time, laid out in
// LDS as the bytes of their h records over the record lines (step tiles of
// 128 B) that the item's columns fall in -- at most 3 superblocks, 15 lines
// -- one token every nl * 128 + 16 bytes; the item then writes every 16-byte
// piece it owns whole, and 2-byte halves only in pieces it shares with the
// neighbouring row block.
constexpr int kImgTokens = 64;
constexpr int kImgMaxLines = 15;
constexpr int kSmemB = kXRing * Geo::kStepB + 2 * kWSlotB;
static_assert(kImgTokens * (kImgMaxLines * 128 + 16) <= kSmemB, "staged h fits in the K loop's LDS");

template <int NMAT>
__global__ void __launch_bounds__(kPThreads, 1) prefill_kernel(PrefillParams P) {
  using G = Geo;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kSmemB];
  uint8_t *const xring = smem;                          // K loop: x ring
  uint8_t *const wlds = smem + kXRing * G::kStepB;      // K loop: weight slots
  // pair ids of the current item's entry and of the next one's (copied in
  // during the current item, before its stores, so that no load waits for
  // those stores)
  __shared__ int pair_sh[2][kPM];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const moe::MatLayout &M0 = NMAT == 2 ? P.gate : P.down;
  const int nsb = M0.nsb, nsteps = 5 * nsb;
  const int rows_out = NMAT == 2 ? P.d_ff : P.d_model;
  constexpr int kWRows = NMAT == 2 ? 32 : 64;  // output rows per wave (gate/up: h rows)
  constexpr int kGRows = kPWaves * kWRows;
  const int nrt = (rows_out + kGRows - 1) / kGRows;
  const int n_items = min(ld_uniform(P.n_work), P.max_work) * nrt;
  // Workgroup b runs on die b % 8 (round-robin dispatch); each die takes a
  // contiguous range of items, so the row blocks of one entry and the entries
  // of one expert share that die's L2 (activations and weights re-read there).
  const int per = (n_items + kXcds - 1) / kXcds;
  const int xcd = blockIdx.x % kXcds, istep = gridDim.x / kXcds;
  const int i_end = min((xcd + 1) * per, n_items);
  const moe::Consts K = moe::make_consts();
  uint32_t sel[6];
  moe::pattern_selectors(g, sel);
  const uint32_t ring = moe::lds_addr(xring), wbase = moe::lds_addr(wlds);
  // this lane's B operand (token r16 of a 16-token tile, K group g) inside a
  // step tile: granule piece ^ swz(row), piece g (hi) or 4 + g (lo)
  const int sw = G::swz(r16);
  const int rl_hi = r16 * G::kRowB + ((g ^ sw) << 4), rl_lo = r16 * G::kRowB + (((4 + g) ^ sw) << 4);
  moe::WorkEntry we_n;
  const uint8_t *blob_n = nullptr;
  int it_n = fetch_item(P, xcd * per + blockIdx.x / kXcds, istep, i_end, nrt, we_n, blob_n);
  if (it_n < i_end) copy_pairs(P, we_n, pair_sh[0], w, lane);
  wait_vm<0>();
  int lb = 0;  // pair buffer of the current item
  while (it_n < i_end) {
    const int it = it_n;
    const moe::WorkEntry we = we_n;
    const uint8_t *const blob = blob_n;
    const int ei = it / nrt, rt = it - ei * nrt;
    const int *const pairs = pair_sh[lb];
    __syncthreads();  // the item's pair ids are published; the previous item no longer reads the LDS data
    const int m = we.m, ntt = (m + 15) >> 4;
    const int wrow0 = rt * kGRows + w * kWRows;
    const bool wact = wrow0 < rows_out;  // whole wave: d_ff, d_model are multiples of 64
    // weight rows of this lane: tiles a = 0..3 (gate/up: gate, gate, up, up);
    // a wave past the matrix reads its last rows (and computes nothing), so
    // the tiles' offsets from tile 0 are the same for every lane
    WRows R;
    {
      const moe::MatLayout &M = NMAT == 2 ? P.gate : P.down;
      const int rbase = wact ? wrow0 : rows_out - kWRows;  // rows_out >= 64 >= kWRows
      R.nblk = M.nblk;
      R.blob = moe::uniform_base(blob);
      R.code = M.code_off + (uint32_t)(rbase + r16) * M.wpr * 4 + g * 16;
      R.scale = M.scale_off + (uint32_t)(rbase + r16) * M.nblk * 2;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int ta = NMAT == 2 ? (a & 1) : a;  // 16-row tile within the wave's rows
        const uint32_t mat = NMAT == 2 && a >= 2 ? P.up.code_off - P.gate.code_off : 0u;
        const uint32_t smat = NMAT == 2 && a >= 2 ? P.up.scale_off - P.gate.scale_off : 0u;
        R.coff[a] = mat + (uint32_t)(16 * ta) * M.wpr * 4;
        R.soff[a] = smat + (uint32_t)(16 * ta) * M.nblk * 2;
      }
    }
    // activation copy roles: granule q = tid + 512 i of a step tile, row n =
    // q / 8 of the tile (its record row, row 0 for columns without a token),
    // its piece swizzled by the row; lands at LDS byte 16 q of the tile
    XCopy X;
    {
      const uint32_t stride = (uint32_t)(NMAT == 2 ? P.xrec_b : P.hrec_b);
      X.base = moe::uniform_base(NMAT == 2 ? P.xrec : P.hrec);
      X.lds = (uint32_t)(64 * w) * 16u;
#pragma unroll
      for (int i = 0; i < G::kCopies; ++i) {
        const int q = tid + kPThreads * i, n = q / G::kGran, pos = q - n * G::kGran;
        const int row = entry_row(P, we, n, pairs);
        const int rr = NMAT == 2 && row >= 0 ? row_token(P, row) : row;
        X.src[i] = (uint32_t)(rr < 0 ? 0 : rr) * stride + (uint32_t)(pos ^ G::swz(n)) * 16u;
      }
    }
    f4 acc[4][kTT];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int nt = 0; nt < kTT; ++nt) acc[a][nt] = (f4){0.f, 0.f, 0.f, 0.f};
    // prologue: the tiles of steps 0 .. kXD-1, then superblock 0's weights
#pragma unroll
    for (int s0 = 0; s0 < kXD; ++s0) copy_x(X, ring, s0, nsteps);
    copy_w(R, wbase, 0, nsb, r16, lane, w);
    uint32_t Pw[4];
    h8 A[4];
    // the next item's entry, and its pair ids copied into the other buffer,
    // as the last superblock starts: younger than the copies in flight (so
    // every counted wait only gets stronger) and landed by the end of the K
    // loop; the next item's start barrier publishes them
    auto fetch_next = [&]() {
      it_n = fetch_item(P, it + istep, istep, i_end, nrt, we_n, blob_n);
      if (it_n < i_end) copy_pairs(P, we_n, pair_sh[lb ^ 1], w, lane);
    };
    if (nsb == 1) fetch_next();
    if (ntt == kTT) {  // uniform
      k_superblock<true, true>(0, nsb, nsteps, R, g, r16, w, lane, Pw, A, X, ring, xring, wbase, wlds, sel, K, ntt, wact,
                               rl_hi, rl_lo, acc);
      for (int S = 1; S < nsb; ++S) {
        if (S == nsb - 1) fetch_next();
        k_superblock<false, true>(S, nsb, nsteps, R, g, r16, w, lane, Pw, A, X, ring, xring, wbase, wlds, sel, K, ntt,
                                  wact, rl_hi, rl_lo, acc);
      }
    } else {
      k_superblock<true, false>(0, nsb, nsteps, R, g, r16, w, lane, Pw, A, X, ring, xring, wbase, wlds, sel, K, ntt,
                                wact, rl_hi, rl_lo, acc);
      for (int S = 1; S < nsb; ++S) {
        if (S == nsb - 1) fetch_next();
        k_superblock<false, false>(S, nsb, nsteps, R, g, r16, w, lane, Pw, A, X, ring, xring, wbase, wlds, sel, K, ntt,
                                   wact, rl_hi, rl_lo, acc);
      }
    }
    // every copy of this item (the ones past the last step included, and the
    // next item's pair ids) has landed before the next item's prologue reuses
    // the slots
    wait_vm<0>();
    // D layout: lane (r16, g) holds rows 4 g + i of each row tile for token
    // r16 of each token tile
    if constexpr (NMAT == 2) {
      // the item owns h columns [c0, c1); they lie in record lines L0 .. L0 + nl - 1
      const int c0 = rt * kGRows, c1 = min(c0 + kGRows, P.d_ff);
      const int L0 = moe::pf::item_L0(c0), nl = moe::pf::item_nl(c0, c1);
      const int istride = nl * 128 + 16;
      // write-out roles: thread (tq, wi) stores piece wi (line L0 + wi / 8,
      // piece wi % 8) of the record for tokens tq, tq + 4, ... of each half,
      // so neighbouring threads store neighbouring bytes of one record; which
      // of the piece's 8 halves the item owns is the same for every token.
      // (The thread index is made opaque here so that none of this is
      // computed ahead of the item loop and kept live through the K loop.)
      int tid_e = tid;
      asm volatile("" : "+v"(tid_e));
      const int wi = tid_e & 127, tq = tid_e >> 7;
      const uint32_t own = moe::pf::full_piece_own(wi, c0, c1);
      const size_t dst_off = (size_t)L0 * 128 + (size_t)wi * 16;
      // Pieces the item owns only in part (moe::pf::boundary_role): thread
      // (tb, pq) stores one half of one of them for tokens tb, tb + 3, ...
      // (whole pieces go out as 16-byte stores above)
      const int pq = tid_e % 160, tb = tid_e / 160;  // tb == 3: idle
      const moe::pf::BoundaryRole br = moe::pf::boundary_role(pq, c0, c1);
      const bool mine = tb < 3 && br.mine;
      const int b_img = ((br.line - L0) * 8 + br.piece) * 16 + 2 * br.half;  // byte in a token's image
      const size_t b_dst = (size_t)br.line * 128 + br.piece * 16 + 2 * br.half;
      // h = silu(gate) up / f of the lane's 8 columns for all token tiles, as
      // packed (hi, lo) fp16 halves (the accumulators die here), and each
      // column's offset in the image
      uint32_t hp[8][kTT];
      int off[8];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float inv_f;
          off[4 * a + i] = rec_byte(wrow0 + 16 * a + 4 * ((tid_e & 63) >> 4) + i, inv_f) - L0 * 128;
#pragma unroll
          for (int nt = 0; nt < kTT; ++nt) {
            const float gv = acc[a][nt][i], uv = acc[a + 2][nt][i];
            const float h = gv / (1.0f + __expf(-gv)) * uv * inv_f;
            const _Float16 hh = (_Float16)h, hl = (_Float16)(h - (float)hh);
            hp[4 * a + i][nt] = (uint32_t)__builtin_bit_cast(uint16_t, hh) |
                                ((uint32_t)__builtin_bit_cast(uint16_t, hl) << 16);
          }
        }
      __syncthreads();  // every wave is done with the x ring and the weight slots
#pragma unroll
      for (int half = 0; half < kTT / 4; ++half) {
        if (16 * 4 * half >= m) break;  // uniform: no token in this half
        if (wact) {
#pragma unroll
          for (int c8 = 0; c8 < 8; ++c8)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const int nt = 4 * half + q4, n = 16 * nt + r16;
              if (nt < ntt && n < m) {
                uint8_t *o = smem + (16 * q4 + r16) * istride + off[c8];
                *reinterpret_cast<uint16_t *>(o) = (uint16_t)hp[c8][nt];
                *reinterpret_cast<uint16_t *>(o + 64) = (uint16_t)(hp[c8][nt] >> 16);
              }
            }
        }
        __syncthreads();  // the half's image is complete
        const int n_tok = min(kImgTokens, m - kImgTokens * half);
        constexpr int kTq = kPThreads / 128;  // token stride of a thread
        if (own == 0xffu) {
          // 4 tokens at a time: every LDS read before the stores
#pragma unroll
          for (int j0 = 0; j0 < kImgTokens / kTq; j0 += 4) {
            u4 v[4];
            int rw[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int nloc = tq + kTq * (j0 + j);  // < kImgTokens: the image read stays in it
              rw[j] = nloc < n_tok ? entry_row(P, we, kImgTokens * half + nloc, pairs) : -1;
              v[j] = *reinterpret_cast<const u4 *>(smem + nloc * istride + wi * 16);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (rw[j] >= 0) *reinterpret_cast<u4 *>(P.hrec + (size_t)rw[j] * P.hrec_b + dst_off) = v[j];
          }
        }
        if (mine) {
          for (int nloc = tb; nloc < n_tok; nloc += 3) {
            const int row = entry_row(P, we, kImgTokens * half + nloc, pairs);
            if (row >= 0)
              *reinterpret_cast<uint16_t *>(P.hrec + (size_t)row * P.hrec_b + b_dst) =
                  *reinterpret_cast<const uint16_t *>(smem + nloc * istride + b_img);
          }
        }
        __syncthreads();  // the image is read out before the next half or item reuses it
      }
    } else if (wact) {
#pragma unroll
      for (int nt = 0; nt < kTT; ++nt) {
        const int n = 16 * nt + r16;
        if (nt < ntt && n < m) {
          const int row = entry_row(P, we, n, pairs);
          if (row >= 0) {
            float *y = we.expert >= 0 ? P.y_pairs + (size_t)row * P.d_model
                                      : P.y_shared + (size_t)(row - P.T * P.k) * P.d_model;
#pragma unroll
            for (int a = 0; a < 4; ++a)
              *reinterpret_cast<float4 *>(y + wrow0 + 16 * a + 4 * g) =
                  make_float4(acc[a][nt][0], acc[a][nt][1], acc[a][nt][2], acc[a][nt][3]);
          }
        }
      }
    }
    lb ^= 1;
  }
}

// x [T][d] fp32 -> the gate/up x record: thread (token, step, g) writes the
// 8 hi halves and the 8 lo halves of its granule pair
__global__ void __launch_bounds__(256) build_xrec_prefill(const float *__restrict__ x, int T, int d, int nsteps,
                                                          uint8_t *__restrict__ xrec, int xrec_b) {
  const size_t n = (size_t)T * nsteps * 4;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const int gq = (int)(i & 3);
    const size_t r = i >> 2;
    const int s = (int)(r % nsteps), tok = (int)(r / nsteps);
    const int S = s / 5, t = s - 5 * S;
    h8 hi, lo;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int p = 20 * gq + 4 * t + (j >> 1), e = j & 1;
      const int c = S * moe::kSbCols + moe::pair_col(p) + 5 * e;
      const float v = c < d ? x[(size_t)tok * d + c] * moe::pair_inv_f(p) : 0.f;
      hi[j] = (_Float16)v;
      lo[j] = (_Float16)(v - (float)hi[j]);
    }
    uint8_t *o = xrec + (size_t)tok * xrec_b + (size_t)s * 128 + gq * 16;
    *reinterpret_cast<h8 *>(o) = hi;
    *reinterpret_cast<h8 *>(o + 64) = lo;
  }
}

}  // namespace

namespace moe {

hipError_t launch_ffn_prefill(const moe_ctx *c, int layer, const float *x, int T, const int32_t *idx,
                              const int32_t *slot_of_pair, float *y_pairs, float *y_shared, hipStream_t s) {
  const moe_config &k = c->cfg;
  if (k.d_ff % 64 || k.d_model % 64) return hipErrorInvalidValue;
  hipError_t e = launch_bucket_ex(c, idx, T, c->offsets_ws, c->perm_ws, true, kPM, nullptr, nullptr, 0, s, nullptr);
  if (e != hipSuccess) return e;
  // the x record shares the decode path's record buffer (the same bytes per
  // token: nsb x 5 steps x 128 B); calls on one context never overlap
  const int gsteps = 5 * c->L.gate.nsb, xrec_b = gsteps * 128;
  {
    const size_t n = (size_t)T * gsteps * 4;
    const size_t blocks = std::min<size_t>((n + 255) / 256, 16384);
    hipLaunchKernelGGL(build_xrec_prefill, dim3((unsigned)blocks), dim3(256), 0, s, x, T, k.d_model, gsteps,
                       (uint8_t *)c->xrec, xrec_b);
  }
  PrefillParams P;
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
  P.xrec = (const uint8_t *)c->xrec;
  P.hrec = (uint8_t *)c->h16;
  P.xrec_b = xrec_b;
  P.hrec_b = 5 * c->L.down.nsb * Geo::kRowB;
  P.y_pairs = y_pairs;
  P.y_shared = y_shared;
  P.d_model = k.d_model;
  P.d_ff = k.d_ff;
  // one workgroup of 8 waves per CU, each walking its die's items
  const int grid = (c->n_cu + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL(prefill_kernel<2>, dim3(grid), dim3(kPThreads), 0, s, P);
  hipLaunchKernelGGL(prefill_kernel<1>, dim3(grid), dim3(kPThreads), 0, s, P);
  return hipGetLastError();
}

}  // namespace moe
