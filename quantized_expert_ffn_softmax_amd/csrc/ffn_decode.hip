// Decode path of the expert FFN: few tokens per expert, bound by streaming
// the experts' packed 3-bit weights from HBM.
//
// The pages' engine reads each touched expert once per step and shares that
// read between the tokens that picked it (speculative verify batches several
// tokens: "单卡5090跑125B 大模型 ...", section 2.3).  Here one wave handles up
// to 16 tokens of one expert against 16 weight rows with
// v_mfma_f32_16x16x32_f16:
//   A (16 rows x 32 K)  = dequantised weights fp16((q - 4) * s), built in
//                         registers from the packed words;
//   B (32 K x 16 tokens)= activations split into two fp16 halves (hi, lo),
//                         so a pair of MFMAs keeps them at fp32 accuracy.
// The layout repeats every 160 columns (16 words, 5 scale blocks): lane group
// g = lane / 16 takes superblock 4R + g, so every lane runs the same
// instruction stream; the 80 code pairs (c, c+5) of a superblock are 20 MFMA
// steps of 4 pairs.  Weights are read once; activations come from L2.
#include "moe_internal.h"
#include "record.h"

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));

// pair p (0..79) of a superblock: word p/5, slot p%5 (low half) and p%5+5
// (high half); columns 10 (p/5) + p%5 and +5.
using moe::pair_col;
__host__ __device__ constexpr int pair_scale_idx(int p) {
  // index into the 9 packed scale pairs (b, b) and (b, b+1)
  return 2 * (pair_col(p) / 32) + ((pair_col(p) + 5) / 32 - pair_col(p) / 32);
}

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

// 16 words of superblock S of one row (zero where past the row's words)
__device__ inline void load_words(const uint8_t *row_codes, int S, int wpr, bool act, uint32_t (&w)[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (act && 16 * S + 4 * i < wpr) v = *reinterpret_cast<const uint4 *>(row_codes + (size_t)(16 * S + 4 * i) * 4);
    w[4 * i + 0] = v.x;
    w[4 * i + 1] = v.y;
    w[4 * i + 2] = v.z;
    w[4 * i + 3] = v.w;
  }
}

// the 5 block scales of superblock S, packed as the 9 pairs a code pair uses
__device__ inline void load_scales(const uint8_t *row_scales, int S, int nblk, bool act, h2 (&sc)[9]) {
  _Float16 s[5];
#pragma unroll
  for (int b = 0; b < 5; ++b) {
    const int blk = 5 * S + b;
    s[b] = (act && blk < nblk) ? *reinterpret_cast<const _Float16 *>(row_scales + (size_t)blk * 2) : (_Float16)0.f;
  }
#pragma unroll
  for (int b = 0; b < 5; ++b) {
    sc[2 * b] = (h2){s[b], s[b]};
    if (b < 4) sc[2 * b + 1] = (h2){s[b], s[b + 1]};
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
__device__ inline h2 deq(const uint32_t (&w)[16], const uint32_t (&w9)[16], const Consts &K, const h2 (&sc)[9]) {
  constexpr int j = p % 5;
  return deq_pair<j>(j < 3 ? w[p / 5] : w9[p / 5], K, sc[pair_scale_idx(p)]);
}

template <int t>
__device__ inline h8 build_a(const uint32_t (&w)[16], const uint32_t (&w9)[16], const Consts &K, const h2 (&sc)[9]) {
  constexpr int p0 = 4 * t;
  const h2 a0 = deq<p0 + 0>(w, w9, K, sc);
  const h2 a1 = deq<p0 + 1>(w, w9, K, sc);
  const h2 a2 = deq<p0 + 2>(w, w9, K, sc);
  const h2 a3 = deq<p0 + 3>(w, w9, K, sc);
  return (h8){a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
}

__device__ inline f4 mfma(h8 a, h8 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }

template <int t>
__device__ inline void load_b(const uint16_t *xs, h8 &bhi, h8 &blo) {
  // columns without a token point at an all-zero row: same address for all of
  // them, so the loads coalesce and no register needs zeroing
  bhi = *reinterpret_cast<const h8 *>(xs + t * 16);
  blo = *reinterpret_cast<const h8 *>(xs + t * 16 + 8);
}

template <int t>
__device__ inline void step2(const uint32_t (&wa)[16], const uint32_t (&wa9)[16], const h2 (&sa)[9],
                             const uint32_t (&wb)[16], const uint32_t (&wb9)[16], const h2 (&sb)[9],
                             const Consts &K, const uint16_t *xs, f4 &acca, f4 &accb) {
  h8 bhi, blo;
  load_b<t>(xs, bhi, blo);
  const h8 a = build_a<t>(wa, wa9, K, sa);
  const h8 b = build_a<t>(wb, wb9, K, sb);
  acca = mfma(a, bhi, acca);
  accb = mfma(b, bhi, accb);
  acca = mfma(a, blo, acca);
  accb = mfma(b, blo, accb);
}

template <int t>
__device__ inline void step1(const uint32_t (&wa)[16], const uint32_t (&wa9)[16], const h2 (&sa)[9],
                             const Consts &K, const uint16_t *xs, f4 &acc) {
  h8 bhi, blo;
  load_b<t>(xs, bhi, blo);
  const h8 a = build_a<t>(wa, wa9, K, sa);
  acc = mfma(a, bhi, acc);
  acc = mfma(a, blo, acc);
}

__device__ inline void shift9(const uint32_t (&w)[16], uint32_t (&w9)[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) w9[i] = w[i] >> 9;
}

using moe::rec_pos;

// the record row (token of x, or pair / shared row of h) behind MFMA column n
// a work entry is used only if it indexes inside this call's pairs / tokens
__device__ inline bool entry_ok(const DecodeParams &P, const moe::WorkEntry &we) {
  if (we.m < 1 || we.m > 16 || we.first < 0) return false;
  return we.expert >= 0 ? (we.expert < P.E && we.first + we.m <= P.T * P.k) : (we.first + we.m <= P.T);
}

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

// One work item = one entry (<= 16 tokens of one expert) x 16 weight rows.
// The K range is split over the WAVES waves of the workgroup: lane group g of
// wave w takes superblocks S = 4w + g, 4w + g + 4*WAVES, ...; the partial
// sums are added in LDS in wave order (deterministic).  MFMA columns without
// a token issue no activation loads.

template <int WAVES>
__device__ inline void reduce_waves(float (*red)[64][8], int wave, int lane, f4 &a, f4 &b, int nv) {
  if (WAVES == 1) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    red[wave][lane][i] = a[i];
    if (nv > 1) red[wave][lane][4 + i] = b[i];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 1; w < WAVES; ++w)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] += red[w][lane][i];
        if (nv > 1) b[i] += red[w][lane][4 + i];
      }
  }
}

// gate and up for 16 rows of d_ff, then h = silu(g) * u into the h record
template <int WAVES>
__global__ void __launch_bounds__(64 * WAVES) ffn_gateup_kernel(DecodeParams P) {
  __shared__ float red[WAVES][64][8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int ntile = P.d_ff / 16;
  const int n_items = min(P.n_work[0], P.max_work) * ntile;
  const int nsb = P.gate.nsb;
  const int rounds = (nsb + 4 * WAVES - 1) / (4 * WAVES);
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const moe::WorkEntry we = P.work[item / ntile];
    const int rt = item % ntile;
    if (!entry_ok(P, we)) continue;
    const uint8_t *blob = entry_blob(P, we);
    if (!blob) continue;
    int tok = 0, hrow = 0;
    const bool has_tok = r16 < we.m && entry_token(P, we, r16, tok, hrow);
    const int row = rt * 16 + r16;
    const uint8_t *gcode = blob + P.gate.code_off + (size_t)row * P.gate.wpr * 4;
    const uint8_t *ucode = blob + P.up.code_off + (size_t)row * P.up.wpr * 4;
    const uint8_t *gsc = blob + P.gate.scale_off + (size_t)row * P.gate.nblk * 2;
    const uint8_t *usc = blob + P.up.scale_off + (size_t)row * P.up.nblk * 2;
    f4 accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
    const Consts K = make_consts();
    for (int R = 0; R < rounds; ++R) {
      const int S = 4 * WAVES * R + 4 * wave + g;
      const bool act = S < nsb;
      uint32_t gw[16], uw[16];
      h2 gs[9], us[9];
      load_words(gcode, S, P.gate.wpr, act, gw);
      load_words(ucode, S, P.up.wpr, act, uw);
      load_scales(gsc, S, P.gate.nblk, act, gs);
      load_scales(usc, S, P.up.nblk, act, us);
      uint32_t gw9[16], uw9[16];
      shift9(gw, gw9);
      shift9(uw, uw9);
      const uint16_t *xs = (act && has_tok) ? P.xrec + (size_t)tok * P.xrec_h + (size_t)S * moe::kSteps * 16
                                            : P.xrec_zero;
      step2<0>(gw, gw9, gs, uw, uw9, us, K, xs, accg, accu);
      step2<1>(gw, gw9, gs, uw, uw9, us, K, xs, accg, accu);
      step2<2>(gw, gw9, gs, uw, uw9, us, K, xs, accg, accu);
      step2<3>(gw, gw9, gs, uw, uw9, us, K, xs, accg, accu);
      step2<4>(gw, gw9, gs, uw, uw9, us, K, xs, accg, accu);
      step2<5>(gw, gw9, gs, uw, uw9, us, K, xs, accg, accu);
      step2<6>(gw, gw9, gs, uw, uw9, us, K, xs, accg, accu);
      step2<7>(gw, gw9, gs, uw, uw9, us, K, xs, accg, accu);
      step2<8>(gw, gw9, gs, uw, uw9, us, K, xs, accg, accu);
      step2<9>(gw, gw9, gs, uw, uw9, us, K, xs, accg, accu);
      step2<10>(gw, gw9, gs, uw, uw9, us, K, xs, accg, accu);
      step2<11>(gw, gw9, gs, uw, uw9, us, K, xs, accg, accu);
      step2<12>(gw, gw9, gs, uw, uw9, us, K, xs, accg, accu);
      step2<13>(gw, gw9, gs, uw, uw9, us, K, xs, accg, accu);
      step2<14>(gw, gw9, gs, uw, uw9, us, K, xs, accg, accu);
      step2<15>(gw, gw9, gs, uw, uw9, us, K, xs, accg, accu);
      step2<16>(gw, gw9, gs, uw, uw9, us, K, xs, accg, accu);
      step2<17>(gw, gw9, gs, uw, uw9, us, K, xs, accg, accu);
      step2<18>(gw, gw9, gs, uw, uw9, us, K, xs, accg, accu);
      step2<19>(gw, gw9, gs, uw, uw9, us, K, xs, accg, accu);
    }
    reduce_waves<WAVES>(red, wave, lane, accg, accu, 2);
    // D layout: lane holds rows 4g + i of the tile for token column r16
    if (wave == 0 && has_tok) {
      uint16_t *hr = P.hrec + (size_t)hrow * P.hrec_h;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float gv = accg[i], uv = accu[i];
        float inv_f;
        const int pos = rec_pos(rt * 16 + 4 * g + i, inv_f);
        const float h = gv / (1.0f + __expf(-gv)) * uv * inv_f;
        const _Float16 hi = (_Float16)h;
        const _Float16 lo = (_Float16)(h - (float)hi);
        hr[pos] = __builtin_bit_cast(uint16_t, hi);
        hr[pos + 8] = __builtin_bit_cast(uint16_t, lo);
      }
    }
    if (WAVES > 1) __syncthreads();  // red is reused by the next item
  }
}

// down for 16 rows of d_model: y = W_d h
template <int WAVES>
__global__ void __launch_bounds__(64 * WAVES) ffn_down_kernel(DecodeParams P) {
  __shared__ float red[WAVES][64][8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int ntile = P.d_model / 16;
  const int n_items = min(P.n_work[0], P.max_work) * ntile;
  const int nsb = P.down.nsb;
  const int rounds = (nsb + 4 * WAVES - 1) / (4 * WAVES);
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const moe::WorkEntry we = P.work[item / ntile];
    const int rt = item % ntile;
    if (!entry_ok(P, we)) continue;
    const uint8_t *blob = entry_blob(P, we);
    if (!blob) continue;
    int tok = 0, hrow = 0;
    const bool has_tok = r16 < we.m && entry_token(P, we, r16, tok, hrow);
    const int row = rt * 16 + r16;
    const uint8_t *dcode = blob + P.down.code_off + (size_t)row * P.down.wpr * 4;
    const uint8_t *dsc = blob + P.down.scale_off + (size_t)row * P.down.nblk * 2;
    f4 acc = {0.f, 0.f, 0.f, 0.f}, unused = {0.f, 0.f, 0.f, 0.f};
    const Consts K = make_consts();
    for (int R = 0; R < rounds; ++R) {
      const int S = 4 * WAVES * R + 4 * wave + g;
      const bool act = S < nsb;
      uint32_t dw[16];
      h2 ds[9];
      load_words(dcode, S, P.down.wpr, act, dw);
      load_scales(dsc, S, P.down.nblk, act, ds);
      uint32_t dw9[16];
      shift9(dw, dw9);
      const uint16_t *hs = (act && has_tok) ? P.hrec + (size_t)hrow * P.hrec_h + (size_t)S * moe::kSteps * 16
                                            : P.hrec_zero;
      step1<0>(dw, dw9, ds, K, hs, acc);
      step1<1>(dw, dw9, ds, K, hs, acc);
      step1<2>(dw, dw9, ds, K, hs, acc);
      step1<3>(dw, dw9, ds, K, hs, acc);
      step1<4>(dw, dw9, ds, K, hs, acc);
      step1<5>(dw, dw9, ds, K, hs, acc);
      step1<6>(dw, dw9, ds, K, hs, acc);
      step1<7>(dw, dw9, ds, K, hs, acc);
      step1<8>(dw, dw9, ds, K, hs, acc);
      step1<9>(dw, dw9, ds, K, hs, acc);
      step1<10>(dw, dw9, ds, K, hs, acc);
      step1<11>(dw, dw9, ds, K, hs, acc);
      step1<12>(dw, dw9, ds, K, hs, acc);
      step1<13>(dw, dw9, ds, K, hs, acc);
      step1<14>(dw, dw9, ds, K, hs, acc);
      step1<15>(dw, dw9, ds, K, hs, acc);
      step1<16>(dw, dw9, ds, K, hs, acc);
      step1<17>(dw, dw9, ds, K, hs, acc);
      step1<18>(dw, dw9, ds, K, hs, acc);
      step1<19>(dw, dw9, ds, K, hs, acc);
    }
    reduce_waves<WAVES>(red, wave, lane, acc, unused, 1);
    if (wave == 0 && has_tok) {
      float *y = we.expert >= 0 ? P.y_pairs + (size_t)hrow * P.d_model : P.y_shared + (size_t)tok * P.d_model;
      *reinterpret_cast<float4 *>(y + rt * 16 + 4 * g) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
    if (WAVES > 1) __syncthreads();
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

template <int WAVES>
static void launch_pair(int g1, int g2, int waves_down, const DecodeParams &P, hipStream_t s) {
  hipLaunchKernelGGL(ffn_gateup_kernel<WAVES>, dim3(g1), dim3(64 * WAVES), 0, s, P);
  if (waves_down == 1)
    hipLaunchKernelGGL(ffn_down_kernel<1>, dim3(g2), dim3(64), 0, s, P);
  else if (waves_down == 2)
    hipLaunchKernelGGL(ffn_down_kernel<2>, dim3(g2), dim3(128), 0, s, P);
  else
    hipLaunchKernelGGL(ffn_down_kernel<4>, dim3(g2), dim3(256), 0, s, P);
}

static int waves_for(int nsb) { return nsb <= 4 ? 1 : (nsb <= 8 ? 2 : 4); }

hipError_t launch_ffn_decode(const moe_ctx *c, int layer, const float *x, int T, const int32_t *idx,
                             const int32_t *slot_of_pair, float *y_pairs, float *y_shared, hipStream_t s) {
  const moe_config &k = c->cfg;
  const int xh = xrec_halves(c->L.gate.nsb);
  // bucketing, work list and (on the single-workgroup path) the x record in one launch
  hipError_t e = launch_bucket_ex(c, idx, T, c->offsets_ws, c->perm_ws, true, 16, x, c->xrec, xh, s);
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
  const int ents = max_entries(T, k.top_k, k.n_experts, 16);
  const int items1 = ents * (k.d_ff / 16), items2 = ents * (k.d_model / 16);
  const int cap = 4096;  // persistent grid: workgroups loop over items
  const int g1 = items1 < cap ? items1 : cap, g2 = items2 < cap ? items2 : cap;
  const int w1 = waves_for(c->L.gate.nsb), w2 = waves_for(c->L.down.nsb);
  if (w1 == 1)
    launch_pair<1>(g1, g2, w2, P, s);
  else if (w1 == 2)
    launch_pair<2>(g1, g2, w2, P, s);
  else
    launch_pair<4>(g1, g2, w2, P, s);
  return hipGetLastError();
}

}  // namespace moe
