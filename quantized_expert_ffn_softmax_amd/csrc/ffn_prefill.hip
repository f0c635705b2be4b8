// Prefill path of the expert FFN: many tokens per expert, a real dense
// contraction, so it runs as a grouped GEMM on MFMA.
//
// The pages' engine runs prefill in chunks of 12,288 tokens ("一张 RTX 4090
// 跑千亿模型，Strata 实测 155 tok/s", the PREFILL=12288 finding); every token
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
//   A (16 rows x 32 K)  = weights, dequantised per wave in registers from the
//                         packed words (no LDS round trip);
//   B (32 K x 16 tokens) = activations (hi, then lo) from a double-buffered
//                         LDS tile that all 8 waves share, one barrier per
//                         32-K step.
// Every global load is an ordinary register load the compiler tracks: word
// quads and scales one superblock ahead, activations two steps ahead of
// their LDS write.  v_mfma_f32_16x16x32_f16 only.
#include <algorithm>

#include "dequant.h"
#include "moe_internal.h"

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
static_assert(Geo::kCopies == 2 && Geo::kGran == 8, "copy roles and swizzle width");

// byte offset of column c's hi half inside one row of a record (its lo half
// sits 64 bytes further); `inv_f` gets the 1 / f the value is stored with
__host__ __device__ inline int rec_byte(int c, float &inv_f) {
  const int S = c / moe::kSbCols, lc = c - S * moe::kSbCols;
  const int w = lc / 10, j = lc - 10 * w;
  const int p = 5 * w + j % 5, e = j / 5;  // pair of the superblock, half
  const int g = p / 20, t = (p % 20) / 4, i = p % 4;
  const int jj = (j % 5) % 3;
  inv_f = jj == 0 ? 1.0f : (jj == 1 ? 0.125f : 0.015625f);
  return (S * 5 + t) * Geo::kRowB + g * 16 + (2 * i + e) * 2;
}

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

__device__ __attribute__((always_inline)) inline const uint8_t *entry_blob(const PrefillParams &P, const moe::WorkEntry &we) {
  if (we.expert < 0) return P.shared_pool + (size_t)P.layer * P.stride;
  const int slot = P.slot_of_pair ? P.slot_of_pair[P.perm[we.first]] : P.layer * P.E + we.expert;
  if (slot < 0 || slot >= P.n_slots) return nullptr;  // never read outside the pool
  return P.slot_pool + (size_t)slot * P.stride;
}

// a work entry is used only if it indexes inside this call's pairs / tokens
__device__ __attribute__((always_inline)) inline bool entry_ok(const PrefillParams &P, const moe::WorkEntry &we) {
  if (we.m < 1 || we.m > kPM || we.first < 0) return false;
  return we.expert >= 0 ? (we.expert < P.E && we.first + we.m <= P.T * P.k) : (we.first + we.m <= P.T);
}

// token and record row (pair id, or T*k + token for the shared expert) of
// entry column n
__device__ __attribute__((always_inline)) inline bool entry_token(const PrefillParams &P, const moe::WorkEntry &we, int n, int &tok, int &row) {
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

__device__ __attribute__((always_inline)) inline f4 mfma(h8 a, h8 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }

// The lane's 4 weight rows: word quad g of each and the scale pairs, for the
// current and the next superblock (indexed by superblock parity).  Each
// quad is one 16-byte load per row, requested at step 0 of the superblock
// before its use, five steps ahead.
struct WSb {
  u4 q[2][4];        // [superblock parity][tile]: words 4g .. 4g + 3
  uint32_t s[2][4];  // [superblock parity][tile]: s_b | s_b+1 << 16
};

// Where the lane's 4 weight rows live: tile a's words at code + coff[a], its
// scales at scale + soff[a] (the offsets are the same for the whole wave)
struct WRows {
  const uint8_t *code;   // word quad g of superblock 0 of tile 0's row
  const uint8_t *scale;  // tile 0's row of scales
  uint32_t coff[4], soff[4];
  int nblk;
};

// every load is unconditional (callers clamp S), so the compiler's waits count
// exactly the loads issued after the one they wait for
template <int SP>
__device__ __attribute__((always_inline)) inline void load_quads(const WRows &R, int S, WSb &o) {
#pragma unroll
  for (int a = 0; a < 4; ++a) o.q[SP][a] = *reinterpret_cast<const u4 *>(R.code + (R.coff[a] + S * 64));
}

template <int SP>
__device__ __attribute__((always_inline)) inline void load_scales(const WRows &R, int S, int g, WSb &o) {
  const int b0 = min(5 * S + g, R.nblk - 1), b1 = min(5 * S + g + 1, R.nblk - 1);
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const uint32_t lo = *reinterpret_cast<const uint16_t *>(R.scale + (R.soff[a] + 2 * b0));
    const uint32_t hi = *reinterpret_cast<const uint16_t *>(R.scale + (R.soff[a] + 2 * b1));
    o.s[SP][a] = lo | (hi << 16);
  }
}

// activation staging of one step: this thread's granules of the tile
template <int HL>
struct XStage {
  u4 v[RecGeom<HL>::kCopies];
};

template <int HL>
struct XRoles {
  const uint8_t *base;                   // the record
  uint32_t stride;                       // bytes per record row
  uint32_t row[RecGeom<HL>::kCopies];    // record row (row 0 for columns without a token)
  uint32_t piece[RecGeom<HL>::kCopies];  // byte offset of the granule inside a step
  uint32_t lds[RecGeom<HL>::kCopies];    // byte offset inside a step tile
};

template <int HL>
__device__ __attribute__((always_inline)) inline void load_x(const XRoles<HL> &X, int s, XStage<HL> &o) {
#pragma unroll
  for (int i = 0; i < RecGeom<HL>::kCopies; ++i)
    o.v[i] = *reinterpret_cast<const u4 *>(X.base + (size_t)X.row[i] * X.stride +
                                           (X.piece[i] + (uint32_t)s * RecGeom<HL>::kRowB));
}

template <int HL>
__device__ __attribute__((always_inline)) inline void store_x(const XRoles<HL> &X, const XStage<HL> &v, uint8_t *tile) {
#pragma unroll
  for (int i = 0; i < RecGeom<HL>::kCopies; ++i) *reinterpret_cast<u4 *>(tile + X.lds[i]) = v.v[i];
}

// One K step (t of superblock S, parity PAR of the step index; SP: parity
// of S): after the barrier, stage the next step's tile into the free LDS
// buffer and request the one after it, request the next superblock's word
// (and scales) that this step frees, then the wave's 4 row tiles x the
// entry's token tiles: every product twice, with the activations' hi and lo.
template <int NMAT, int t, int PAR, int SP>
__device__ __attribute__((always_inline)) inline void k_step(int S, int nsb, const WRows &R, int g, WSb &W,
                                                             uint8_t (*xs)[Geo::kStepB],
                                                             const XRoles<kHL> &XR, XStage<kHL> (&XS)[2],
                                                             const uint32_t (&sel)[6], const moe::Consts &K, int ntt,
                                                             bool wact, int rl_hi, int rl_lo, f4 (&acc)[4][kTT]) {
  using G = Geo;
  const int s = 5 * S + t, nsteps = 5 * nsb;
  __syncthreads();  // step s's tile is complete; the other buffer is no longer read
  // past the last step these restage the last tile: harmless, and no load is
  // conditional
  store_x<kHL>(XR, XS[PAR ^ 1], xs[PAR ^ 1]);
  load_x<kHL>(XR, min(s + 3, nsteps - 1), XS[PAR ^ 1]);
  // the next superblock's quads and scales, a superblock ahead of their use
  if constexpr (t == 0) {
    load_quads<SP ^ 1>(R, min(S + 1, nsb - 1), W);
    load_scales<SP ^ 1>(R, min(S + 1, nsb - 1), g, W);
  }
  h8 A[4];  // (a wave past the matrix dequantises its clamped rows and drops them)
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const uint32_t w4[4] = {W.q[SP][a].x, W.q[SP][a].y, W.q[SP][a].z, W.q[SP][a].w};
    A[a] = moe::quad_a_sel<t>(w4, K, W.s[SP][a], sel);
  }
  if (!wact) return;  // wave-uniform: rows past the matrix
  // B operands one read ahead of their MFMAs: the next half is requested
  // before the current one's four MFMAs, so LDS latency overlaps them
  const uint8_t *tile = xs[PAR];
  h8 cur = *reinterpret_cast<const h8 *>(tile + rl_hi);
#pragma unroll
  for (int nt = 0; nt < kTT; ++nt) {
    if (nt < ntt) {  // wave-uniform: token tiles holding tokens
      const h8 bl = *reinterpret_cast<const h8 *>(tile + nt * 16 * G::kRowB + rl_lo);
#pragma unroll
      for (int a = 0; a < 4; ++a) acc[a][nt] = mfma(A[a], cur, acc[a][nt]);
      if (nt + 1 < ntt) cur = *reinterpret_cast<const h8 *>(tile + (nt + 1) * 16 * G::kRowB + rl_hi);
#pragma unroll
      for (int a = 0; a < 4; ++a) acc[a][nt] = mfma(A[a], bl, acc[a][nt]);
    }
  }
}

// One superblock (5 K steps).  PAR: parity of its first step index, SP: of
// the superblock index (the two alternate together: 5 steps per superblock).
template <int NMAT, int SP>
__device__ __attribute__((always_inline)) inline void k_superblock(int S, int nsb, const WRows &R, int g, WSb &W,
                                                                   uint8_t (*xs)[Geo::kStepB],
                                                                   const XRoles<kHL> &XR, XStage<kHL> (&XS)[2],
                                                                   const uint32_t (&sel)[6], const moe::Consts &K,
                                                                   int ntt, bool wact, int rl_hi, int rl_lo,
                                                                   f4 (&acc)[4][kTT]) {
  constexpr int PAR = SP;
  k_step<NMAT, 0, PAR, SP>(S, nsb, R, g, W, xs, XR, XS, sel, K, ntt, wact, rl_hi, rl_lo, acc);
  k_step<NMAT, 1, PAR ^ 1, SP>(S, nsb, R, g, W, xs, XR, XS, sel, K, ntt, wact, rl_hi, rl_lo, acc);
  k_step<NMAT, 2, PAR, SP>(S, nsb, R, g, W, xs, XR, XS, sel, K, ntt, wact, rl_hi, rl_lo, acc);
  k_step<NMAT, 3, PAR ^ 1, SP>(S, nsb, R, g, W, xs, XR, XS, sel, K, ntt, wact, rl_hi, rl_lo, acc);
  k_step<NMAT, 4, PAR, SP>(S, nsb, R, g, W, xs, XR, XS, sel, K, ntt, wact, rl_hi, rl_lo, acc);
}

// NMAT = 2: gate/up -> h record; NMAT = 1: down -> y.  One workgroup per CU
// walks its accelerator die's share of the (entry, row block) items.
template <int NMAT>
__global__ void __launch_bounds__(kPThreads, 1) prefill_kernel(PrefillParams P) {
  using G = Geo;
  __shared__ __attribute__((aligned(16))) uint8_t xs[2][G::kStepB];
  __shared__ int row_sh[kPM], tok_sh[kPM];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const moe::MatLayout &M0 = NMAT == 2 ? P.gate : P.down;
  const int nsb = M0.nsb, nsteps = 5 * nsb;
  const int rows_out = NMAT == 2 ? P.d_ff : P.d_model;
  constexpr int kWRows = NMAT == 2 ? 32 : 64;  // output rows per wave (gate/up: h rows)
  constexpr int kGRows = kPWaves * kWRows;
  const int nrt = (rows_out + kGRows - 1) / kGRows;
  const int n_items = min(P.n_work[0], P.max_work) * nrt;
  // Workgroup b runs on die b % 8 (round-robin dispatch); each die takes a
  // contiguous range of items, so the row blocks of one entry and the entries
  // of one expert share that die's L2 (activations and weights re-read there).
  const int per = (n_items + kXcds - 1) / kXcds;
  const int xcd = blockIdx.x % kXcds, istep = gridDim.x / kXcds;
  const int i_end = min((xcd + 1) * per, n_items);
  const moe::Consts K = moe::make_consts();
  uint32_t sel[6];
  moe::pattern_selectors(g, sel);
  // this lane's B operand (token r16 of a 16-token tile, K group g) inside a
  // step tile: granule piece ^ swz(row), piece g (hi) or 4 + g (lo)
  const int sw = G::swz(r16);
  const int rl_hi = r16 * G::kRowB + ((g ^ sw) << 4), rl_lo = r16 * G::kRowB + (((4 + g) ^ sw) << 4);
  for (int it = xcd * per + blockIdx.x / kXcds; it < i_end; it += istep) {
    const int ei = it / nrt, rt = it - ei * nrt;
    const moe::WorkEntry we = P.work[ei];
    if (!entry_ok(P, we)) continue;  // uniform over the workgroup
    const uint8_t *blob = entry_blob(P, we);
    if (!blob) continue;
    __syncthreads();  // the previous item no longer reads the token lists or the tiles
    if (tid < kPM) {
      int tok = -1, row = -1;
      if (tid < we.m && !entry_token(P, we, tid, tok, row)) tok = row = -1;
      tok_sh[tid] = tok;
      row_sh[tid] = row;
    }
    __syncthreads();
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
      R.code = blob + M.code_off + (size_t)(rbase + r16) * M.wpr * 4 + g * 16;
      R.scale = blob + M.scale_off + (size_t)(rbase + r16) * M.nblk * 2;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int ta = NMAT == 2 ? (a & 1) : a;  // 16-row tile within the wave's rows
        const uint32_t mat = NMAT == 2 && a >= 2 ? P.up.code_off - P.gate.code_off : 0u;
        const uint32_t smat = NMAT == 2 && a >= 2 ? P.up.scale_off - P.gate.scale_off : 0u;
        R.coff[a] = mat + (uint32_t)(16 * ta) * M.wpr * 4;
        R.soff[a] = smat + (uint32_t)(16 * ta) * M.nblk * 2;
      }
    }
    // activation copy roles: granule q = tid + 512 i of a step tile
    XRoles<kHL> XR;
    XR.base = NMAT == 2 ? P.xrec : P.hrec;
    XR.stride = (uint32_t)(NMAT == 2 ? P.xrec_b : P.hrec_b);
#pragma unroll
    for (int i = 0; i < G::kCopies; ++i) {
      const int q = tid + kPThreads * i, n = q / G::kGran, pos = q - n * G::kGran;
      const int rr = n < m ? (NMAT == 2 ? tok_sh[n] : row_sh[n]) : -1;
      XR.row[i] = (uint32_t)(rr < 0 ? 0 : rr);
      XR.piece[i] = (uint32_t)(pos ^ G::swz(n)) * 16u;
      XR.lds[i] = (uint32_t)q * 16u;
    }
    f4 acc[4][kTT];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int nt = 0; nt < kTT; ++nt) acc[a][nt] = (f4){0.f, 0.f, 0.f, 0.f};
    // prologue: superblock 0's weights; tiles of steps 0 (to LDS), 1 and 2
    WSb W;
    load_quads<0>(R, 0, W);
    load_scales<0>(R, 0, g, W);
    XStage<kHL> XS[2];
    load_x<kHL>(XR, 0, XS[0]);
    load_x<kHL>(XR, min(1, nsteps - 1), XS[1]);
    store_x<kHL>(XR, XS[0], xs[0]);
    load_x<kHL>(XR, min(2, nsteps - 1), XS[0]);
    int S = 0;
    for (; S + 1 < nsb; S += 2) {
      k_superblock<NMAT, 0>(S, nsb, R, g, W, xs, XR, XS, sel, K, ntt, wact, rl_hi, rl_lo, acc);
      k_superblock<NMAT, 1>(S + 1, nsb, R, g, W, xs, XR, XS, sel, K, ntt, wact, rl_hi, rl_lo, acc);
    }
    if (S < nsb) k_superblock<NMAT, 0>(S, nsb, R, g, W, xs, XR, XS, sel, K, ntt, wact, rl_hi, rl_lo, acc);
    if (!wact) continue;
    // D layout: lane (r16, g) holds rows 4 g + i of each row tile for token
    // r16 of each token tile
    if constexpr (NMAT == 2) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float inv_f;
          const int off = rec_byte(wrow0 + 16 * a + 4 * g + i, inv_f);
#pragma unroll
          for (int nt = 0; nt < kTT; ++nt) {
            const int n = 16 * nt + r16;
            if (nt < ntt && n < m) {
              const int row = row_sh[n];
              if (row >= 0) {
                const float gv = acc[a][nt][i], uv = acc[a + 2][nt][i];
                const float h = gv / (1.0f + __expf(-gv)) * uv * inv_f;
                const _Float16 hh = (_Float16)h, hl = (_Float16)(h - (float)hh);
                uint8_t *o = P.hrec + (size_t)row * P.hrec_b + off;
                *reinterpret_cast<_Float16 *>(o) = hh;
                *reinterpret_cast<_Float16 *>(o + 64) = hl;
              }
            }
          }
        }
    } else {
#pragma unroll
      for (int nt = 0; nt < kTT; ++nt) {
        const int n = 16 * nt + r16;
        if (nt < ntt && n < m) {
          const int row = row_sh[n];
          if (row >= 0) {
            float *y = we.expert >= 0 ? P.y_pairs + (size_t)row * P.d_model
                                      : P.y_shared + (size_t)tok_sh[n] * P.d_model;
#pragma unroll
            for (int a = 0; a < 4; ++a)
              *reinterpret_cast<float4 *>(y + wrow0 + 16 * a + 4 * g) =
                  make_float4(acc[a][nt][0], acc[a][nt][1], acc[a][nt][2], acc[a][nt][3]);
          }
        }
      }
    }
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
