// Prefill path of the expert FFN: many tokens per expert, a real dense
// contraction, so it runs as a grouped GEMM on MFMA.
//
// The pages' engine runs prefill in chunks of 12,288 tokens ("一张 RTX 4090
// 跑千亿模型，Strata 实测 155 tok/s", the PREFILL=12288 finding); every token
// of a chunk is routed to 10 of 512 experts, so one chunk is 122,880
// (token, expert) pairs grouped per expert.
//
// Operands are fp16, as the reading for this path fixes: x, the dequantised
// weights fp16((q - 4) * s) and h = silu(g) * u are each rounded to fp16
// once; products and sums are fp32 (v_mfma_f32_16x16x32_f16).
// Work: tiles of (up to 128 tokens of one expert) x (128 weight rows); K runs
// in steps of 80 slots, dequantised into LDS.
#include <algorithm>

#include "moe_internal.h"

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Tiles: 128 tokens of one expert x 128 weight rows (gate/up: 64 rows of each
// matrix, so one tile yields h for 64 rows; down: 128 rows, the last tile of a
// d_model that is an odd multiple of 64 half used).  Every token's activations
// are read once per row tile, so the row tile sets how often they are read:
// 128 rows read them 12 (gate/up) and 16 (down) times per chunk instead of 24
// and 32 with 64-row tiles.  K runs in steps
// of 80 slots -- half a 160-column superblock, 8 packed words -- in "pair
// order": inside each superblock, slot 2p + e holds column c_p + 5 e with
// c_p = 10 (p / 5) + p % 5, i.e. the two codes that share the two halves of a
// packed word sit side by side.  The fp16 copies of x and h are stored in
// that order (zero at slots past the last column), so one v_and_or_b32 +
// v_pk_add + v_pk_mul dequantises two adjacent K slots in place, and any K
// order is the same contraction.
// Per step every thread copies 80 bytes of activations and dequantises four
// words of one weight row into LDS; the next step's global loads are in flight
// while the MFMAs of this one run.  The LDS tile is single-buffered (two
// barriers per step): at 46 KB a CU holds three workgroups.
// MFMA: v_mfma_f32_16x16x32_f16 twice and v_mfma_f32_16x16x16_f16 once per
// 16 x 16 output tile per step; each wave owns 64 tokens x 64 rows (4 x 4
// tiles); D[token][row].
// ---------------------------------------------------------------------------
constexpr int kPM = 128;       // tokens per tile (work entries hold <= kPM tokens)
constexpr int kPN = 128;       // weight rows per tile
constexpr int kPK = 80;        // K slots per step
constexpr int kPld = kPK + 8;  // LDS pitch in halves: rows 176 B apart, 8 consecutive rows on 8 bank groups

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
  const _Float16 *x16;  // [T][kp_model], pair order
  _Float16 *h16;        // [T*k + T][kp_ff], pair order
  int kp_model, kp_ff;  // padded row lengths: superblocks x 160
  float *y_pairs, *y_shared;
  int d_model, d_ff;
};

__device__ inline const uint8_t *entry_blob(const PrefillParams &P, const moe::WorkEntry &we) {
  if (we.expert < 0) return P.shared_pool + (size_t)P.layer * P.stride;
  const int slot = P.slot_of_pair ? P.slot_of_pair[P.perm[we.first]] : P.layer * P.E + we.expert;
  if (slot < 0 || slot >= P.n_slots) return nullptr;  // never read outside the pool
  return P.slot_pool + (size_t)slot * P.stride;
}

// a work entry is used only if it indexes inside this call's pairs / tokens
__device__ inline bool entry_ok(const PrefillParams &P, const moe::WorkEntry &we) {
  if (we.m < 1 || we.m > kPM || we.first < 0) return false;
  return we.expert >= 0 ? (we.expert < P.E && we.first + we.m <= P.T * P.k) : (we.first + we.m <= P.T);
}

__device__ inline bool entry_token(const PrefillParams &P, const moe::WorkEntry &we, int n, int &tok, int &row) {
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

// column -> pair-order slot, and back
__host__ __device__ inline int pair_slot(int c) {
  const int S = c / moe::kSbCols, lc = c - S * moe::kSbCols, w = lc / 10, j = lc - 10 * w;
  return S * moe::kSbCols + 2 * (5 * w + j % 5) + j / 5;
}
__host__ __device__ inline int slot_col(int s) {
  const int S = s / moe::kSbCols, r = s - S * moe::kSbCols, p = r >> 1;
  return S * moe::kSbCols + 10 * (p / 5) + p % 5 + 5 * (r & 1);
}
// 1 / f of K slot s: the weights of a pair whose codes sit at slot j = p % 5
// of their word reach the MFMA multiplied by f = 1, 8 or 64 (j mod 3), so the
// activations in that slot are stored divided by f (exact powers of two)
__host__ __device__ inline float slot_inv_f(int s) {
  const int j = ((s % moe::kSbCols) >> 1) % 5 % 3;
  return j == 0 ? 1.0f : (j == 1 ? 0.125f : 0.015625f);
}

__device__ inline f4 mfma32(h8 a, h8 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }
__device__ inline f4 mfma16(h4 a, h4 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0); }

// Weight part of one thread: B row brow, words 4u .. 4u+3 of each 8-word step
// (u is the same for a whole wave, so the pair selectors below are uniform).
struct WSrc {
  const uint8_t *codes;   // the row's words
  const uint8_t *scales;  // the row's scales
  int nblk;
};

// raw loads of step s for this thread: 4 words (40 columns starting at
// 80 hh + 40 u of the superblock, always inside 2 scale blocks) and those 2
// scale blocks
struct WRaw {
  uint4 w;
  uint32_t s0, s1;
};

__device__ inline void load_w(const WSrc &W, int s, int u, WRaw &r) {
  const int S = s >> 1, hh = s & 1;
  r.w = *reinterpret_cast<const uint4 *>(W.codes + (size_t)(S * 16 + 8 * hh + 4 * u) * 4);
  const int b0 = 5 * S + (80 * hh + 40 * u) / 32;
  r.s0 = *reinterpret_cast<const uint16_t *>(W.scales + (size_t)min(b0, W.nblk - 1) * 2);
  r.s1 = *reinterpret_cast<const uint16_t *>(W.scales + (size_t)min(b0 + 1, W.nblk - 1) * 2);
}

struct PConsts {
  uint32_t mask[3];  // 0x00070007 << 3 j', kept in VGPRs so v_and_or_b32 can be used
  uint32_t magic;    // fp16 1024 in both halves
};

// Which of the thread's two scale blocks each half of code pair (a, j) uses:
// with c0 = 80 hh + 40 u the superblock-relative column of the thread's
// first code, column c0 + lc uses the second block when lc >= thr(hh, u) =
// 32 (c0 / 32 + 1) - c0 (32, 24, 16, 8).  hh (step parity) and u (the wave's
// word quad) are compile-time below, so each pair's scales come from one
// packed register through op_sel, with no per-pair byte permute.
__host__ __device__ constexpr int scale_thr(int hh, int u) {
  return ((80 * hh + 40 * u) / 32 + 1) * 32 - (80 * hh + 40 * u);
}

// Dequantise the thread's 20 code pairs into 40 consecutive K slots (80 B).
// Per pair: one v_and_or_b32 (fp16 1024 + f q), one v_pk_add (- (1024 + 4 f),
// exact: f (q - 4)), one v_pk_mul by the pair's scales, taken from the packed
// (s0, s1) by op_sel (one rounding: f fp16((q - 4) s), f a power of two); the
// activations of the slot carry 1 / f.
template <int HH, int U>
__device__ inline void deq_w(const WRaw &r, const PConsts &K, _Float16 *dst) {
  constexpr int thr = scale_thr(HH, U);
  const h2 S = __builtin_bit_cast(h2, (r.s0 & 0xffffu) | (r.s1 << 16));
  h2 out[20];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const uint32_t word = a == 0 ? r.w.x : a == 1 ? r.w.y : a == 2 ? r.w.z : r.w.w;
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      const int jj = j % 3;
      const uint32_t src = j < 3 ? word : (word >> 9);
      const float f = jj == 0 ? 1.0f : (jj == 1 ? 8.0f : 64.0f);
      const h2 v = __builtin_bit_cast(h2, (src & K.mask[jj]) | K.magic);
      const h2 o = {(_Float16)(1024.0f + 4.0f * f), (_Float16)(1024.0f + 4.0f * f)};
      const int lc = 10 * a + j;
      const h2 sc = {lc >= thr ? S[1] : S[0], lc + 5 >= thr ? S[1] : S[0]};
      out[5 * a + j] = (v - o) * sc;
    }
  }
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const uint4 pk = make_uint4(__builtin_bit_cast(uint32_t, out[4 * i]), __builtin_bit_cast(uint32_t, out[4 * i + 1]),
                                __builtin_bit_cast(uint32_t, out[4 * i + 2]), __builtin_bit_cast(uint32_t, out[4 * i + 3]));
    *reinterpret_cast<uint4 *>(dst + 8 * i) = pk;
  }
}

// One K step: (with one buffer: wait until every wave has read the previous
// step) store the prefetched activations and dequantised weights into buffer
// B, request step s + 1, barrier, then the wave's MFMAs on buffer B.
template <int B, int NBUF, int HH>
__device__ inline void prefill_step(int s, int nsteps, bool xact, uint4 &xv0, uint4 &xv1, uint4 &xv2, uint4 &xv3,
                                    uint4 &xv4, _Float16 *xdst, WRaw &wr, const PConsts &K,
                                    _Float16 *wdst, const WSrc &W, int u, const _Float16 *xsrc, int xh,
                                    const _Float16 (*wsb)[kPld], const _Float16 (*xsb)[kPld], const int (&bro)[4],
                                    int r16, int g, int wm, int mt_active, f4 (&acc)[4][4]) {
  if constexpr (NBUF == 1) __syncthreads();  // every wave has read the previous step
  if (xact) {
    uint4 *dst = reinterpret_cast<uint4 *>(xdst);
    dst[0] = xv0;
    dst[1] = xv1;
    dst[2] = xv2;
    dst[3] = xv3;
    dst[4] = xv4;
  }
  if (u == 0)  // u is wave-uniform
    deq_w<HH, 0>(wr, K, wdst);
  else
    deq_w<HH, 1>(wr, K, wdst);
  if (s + 1 < nsteps) {
    if (xact) {
      const uint4 *src = reinterpret_cast<const uint4 *>(xsrc + (s + 1) * kPK + 40 * xh);
      xv0 = src[0];
      xv1 = src[1];
      xv2 = src[2];
      xv3 = src[3];
      xv4 = src[4];
    }
    load_w(W, s + 1, u, wr);
  }
  __syncthreads();
  h8 b32[4][2];
  h4 b16[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const _Float16 *wrow = wsb[bro[nb] + r16];
    b32[nb][0] = *reinterpret_cast<const h8 *>(wrow + 8 * g);
    b32[nb][1] = *reinterpret_cast<const h8 *>(wrow + 32 + 8 * g);
    b16[nb] = *reinterpret_cast<const h4 *>(wrow + 64 + 4 * g);
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    if (mt < mt_active) {
      const _Float16 *xrow = xsb[64 * wm + 16 * mt + r16];
      const h8 a0 = *reinterpret_cast<const h8 *>(xrow + 8 * g);
      const h8 a1 = *reinterpret_cast<const h8 *>(xrow + 32 + 8 * g);
      const h4 a2 = *reinterpret_cast<const h4 *>(xrow + 64 + 4 * g);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        acc[mt][nb] = mfma32(a0, b32[nb][0], acc[mt][nb]);
        acc[mt][nb] = mfma32(a1, b32[nb][1], acc[mt][nb]);
        acc[mt][nb] = mfma16(a2, b16[nb], acc[mt][nb]);
      }
    }
  }
}

constexpr int kNBuf = 1;  // LDS buffers of the K loop (2: double-buffered, one barrier per step)
template <int NMAT>
__global__ void __launch_bounds__(256, kNBuf == 1 ? 3 : 2) prefill_kernel(PrefillParams P) {
  __shared__ __attribute__((aligned(16))) _Float16 xs[kNBuf][kPM][kPld];
  __shared__ __attribute__((aligned(16))) _Float16 ws[kNBuf][kPN][kPld];
  __shared__ int row_sh[kPM], tok_sh[kPM];
  const int rows_out = NMAT == 2 ? P.d_ff : P.d_model;
  const int tile_rows = NMAT == 2 ? kPN / 2 : kPN;  // output rows per tile
  const int ntile = (rows_out + tile_rows - 1) / tile_rows;
  const int item = blockIdx.x;
  if (item >= min(P.n_work[0], P.max_work) * ntile) return;
  const moe::WorkEntry we = P.work[item / ntile];
  const int nt = item % ntile;
  if (!entry_ok(P, we)) return;
  const uint8_t *blob = entry_blob(P, we);
  if (!blob) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < kPM) {
    int tok = -1, row = -1;
    if (tid < we.m && !entry_token(P, we, tid, tok, row)) tok = row = -1;
    tok_sh[tid] = tok;
    row_sh[tid] = row;
  }
  __syncthreads();
  const int m = we.m;
  const int kp = NMAT == 2 ? P.kp_model : P.kp_ff;
  const int nsteps = kp / kPK;
  // activation copy role: row xr, the 40 slots starting at 40 xh
  const int xr = tid >> 1, xh = tid & 1;
  const bool xact = xr < m && row_sh[xr] >= 0;
  const _Float16 *xsrc = nullptr;
  if (xact) xsrc = NMAT == 2 ? P.x16 + (size_t)tok_sh[xr] * kp : P.h16 + (size_t)row_sh[xr] * kp;
  // weight role: B row brow, word quad u (one u per wave; readfirstlane makes
  // that visible, so the pair selectors live in scalar registers)
  const int brow = lane + 64 * (wave >> 1), u = __builtin_amdgcn_readfirstlane(wave & 1);
  WSrc W;
  {
    const moe::MatLayout &M = NMAT == 2 ? (brow < kPN / 2 ? P.gate : P.up) : P.down;
    const int wrow = NMAT == 2 ? nt * (kPN / 2) + (brow & (kPN / 2 - 1)) : min(nt * kPN + brow, rows_out - 1);
    W.codes = blob + M.code_off + (size_t)wrow * M.wpr * 4;
    W.scales = blob + M.scale_off + (size_t)wrow * M.nblk * 2;
    W.nblk = M.nblk;
  }
  PConsts K;
  K.mask[0] = 0x00070007u;
  K.mask[1] = 0x00380038u;
  K.mask[2] = 0x01c001c0u;
  K.magic = 0x64006400u;
  asm volatile("" : "+v"(K.mask[0]), "+v"(K.mask[1]), "+v"(K.mask[2]), "+s"(K.magic));
  uint4 xv0, xv1, xv2, xv3, xv4;
  WRaw wr;
  const int wm = wave & 1, wn = wave >> 1;
  // output tiles of this wave: M tiles mt (16 tokens each), N tiles nb
  f4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = (f4){0.f, 0.f, 0.f, 0.f};
  // B rows of N tile nb: gate/up -> gate rows 32 wn + 16 nb (nb < 2), up rows
  // 64 + 32 wn + 16 (nb - 2); down -> 64 wn + 16 nb
  int bro[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
    bro[nb] = NMAT == 2 ? (nb < 2 ? 32 * wn + 16 * nb : kPN / 2 + 32 * wn + 16 * (nb - 2)) : 64 * wn + 16 * nb;
  const int r16 = lane & 15, g = lane >> 4;
  const int mt_active = min(4, max(0, (m - 64 * wm + 15) / 16));  // M tiles holding tokens
  if (xact) {
    const uint4 *src = reinterpret_cast<const uint4 *>(xsrc + 40 * xh);
    xv0 = src[0];
    xv1 = src[1];
    xv2 = src[2];
    xv3 = src[3];
    xv4 = src[4];
  }
  load_w(W, 0, u, wr);
  // steps come in (even, odd) pairs: buffer and scale classes are static
  for (int s = 0; s < nsteps; s += 2) {
    constexpr int b1 = kNBuf - 1;
    prefill_step<0, kNBuf, 0>(s, nsteps, xact, xv0, xv1, xv2, xv3, xv4, xs[0][xr] + 40 * xh, wr, K,
                              ws[0][brow] + 40 * u, W, u, xsrc, xh, ws[0], xs[0], bro, r16, g, wm, mt_active, acc);
    prefill_step<b1, kNBuf, 1>(s + 1, nsteps, xact, xv0, xv1, xv2, xv3, xv4, xs[b1][xr] + 40 * xh, wr, K,
                               ws[b1][brow] + 40 * u, W, u, xsrc, xh, ws[b1], xs[b1], bro, r16, g, wm, mt_active, acc);
  }
  // D: lane holds tokens 4 g + i of the M tile for column r16 of the N tile.
  // gate/up: the lane's two h columns, their K slots in the down record and
  // the 1 / f they are stored with
  int hsl[2] = {0, 0};
  float hinv[2] = {1.0f, 1.0f};
  if constexpr (NMAT == 2) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      hsl[nb] = pair_slot(nt * (kPN / 2) + 32 * wn + 16 * nb + r16);
      hinv[nb] = slot_inv_f(hsl[nb]);
    }
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int mm = 64 * wm + 16 * mt + 4 * g + i;
      if (mm >= m) continue;
      const int hrow = row_sh[mm];
      if (hrow < 0) continue;
      if constexpr (NMAT == 2) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const float gv = acc[mt][nb][i], uv = acc[mt][nb + 2][i];
          // h is rounded to fp16 here, so the division is kept exact; stored
          // divided by the f of its K slot in the down weights
          const float h = gv / (1.0f + __expf(-gv)) * uv;
          P.h16[(size_t)hrow * P.kp_ff + hsl[nb]] = (_Float16)(h * hinv[nb]);
        }
      } else {
        float *y = we.expert >= 0 ? P.y_pairs + (size_t)hrow * P.d_model : P.y_shared + (size_t)tok_sh[mm] * P.d_model;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int col = nt * kPN + 64 * wn + 16 * nb + r16;
          if (col < P.d_model) y[col] = acc[mt][nb][i];
        }
      }
    }
}

// x [T][d] fp32 -> fp16 in pair order, rows of kp slots (zero past column d),
// each value divided by the f of its slot
__global__ void __launch_bounds__(256) to_fp16_pairs_kernel(const float *__restrict__ x, int T, int d, int kp,
                                                            _Float16 *__restrict__ y) {
  const size_t n = (size_t)T * kp;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const int t = (int)(i / kp), sl = (int)(i - (size_t)t * kp);
    const int c = slot_col(sl);
    y[i] = c < d ? (_Float16)(x[(size_t)t * d + c] * slot_inv_f(sl)) : (_Float16)0.f;
  }
}

}  // namespace

namespace moe {

hipError_t launch_bucket_ex(const moe_ctx *c, const int32_t *idx, int T, int32_t *offsets, int32_t *perm, bool build,
                            int entry_m, const float *x, uint16_t *xrec, int xrec_h, hipStream_t s);

hipError_t launch_ffn_prefill(const moe_ctx *c, int layer, const float *x, int T, const int32_t *idx,
                              const int32_t *slot_of_pair, float *y_pairs, float *y_shared, hipStream_t s) {
  const moe_config &k = c->cfg;
  if (k.d_ff % (kPN / 2) || k.d_model % (kPN / 2)) return hipErrorInvalidValue;
  hipError_t e = launch_bucket_ex(c, idx, T, c->offsets_ws, c->perm_ws, true, kPM, nullptr, nullptr, 0, s);
  if (e != hipSuccess) return e;
  const int kpm = c->L.gate.nsb * moe::kSbCols, kpf = c->L.down.nsb * moe::kSbCols;
  {
    const size_t nx = (size_t)T * kpm;
    const size_t blocks = std::min<size_t>((nx + 255) / 256, 8192);
    hipLaunchKernelGGL(to_fp16_pairs_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, T, k.d_model, kpm,
                       (_Float16 *)c->x16);
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
  P.x16 = (const _Float16 *)c->x16;
  P.h16 = (_Float16 *)c->h16;
  P.kp_model = kpm;
  P.kp_ff = kpf;
  P.y_pairs = y_pairs;
  P.y_shared = y_shared;
  P.d_model = k.d_model;
  P.d_ff = k.d_ff;
  // entries hold <= kPM tokens: at most pairs/kPM + min(E, pairs) routed ones + the shared ones
  const int pairs = T * k.top_k;
  const int ents = pairs / kPM + (pairs < k.n_experts ? pairs : k.n_experts) + (T + kPM - 1) / kPM;
  hipLaunchKernelGGL(prefill_kernel<2>, dim3(ents * (k.d_ff / (kPN / 2))), dim3(256), 0, s, P);
  hipLaunchKernelGGL(prefill_kernel<1>, dim3(ents * ((k.d_model + kPN - 1) / kPN)), dim3(256), 0, s, P);
  return hipGetLastError();
}

}  // namespace moe
