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
// Work: tiles of (up to 64 tokens of one expert) x (64 weight rows); K runs
// in blocks of 32 columns, one scale block each, dequantised into LDS.
#include "moe_internal.h"

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kTM = 64;   // tokens per tile
constexpr int kTN = 64;   // weight rows per tile
constexpr int kKB = 32;   // K per block (one scale block)
constexpr int kLd = kKB + 8;  // LDS row pitch in halves (16-byte aligned, spreads banks)

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
  const _Float16 *x16;  // [T][d_model]
  _Float16 *h16;        // [T*k + T][d_ff]
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
  if (we.m < 1 || we.m > kTM || we.first < 0) return false;
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

// 16 dequantised weights of one row, columns c0..c0+15 (c0 % 16 == 0), into LDS
__device__ inline void deq16(const uint8_t *blob, const moe::MatLayout &M, int row, int c0, _Float16 *dst) {
  const uint32_t *codes = reinterpret_cast<const uint32_t *>(blob + M.code_off) + (size_t)row * M.wpr;
  const _Float16 s = *reinterpret_cast<const _Float16 *>(blob + M.scale_off + ((size_t)row * M.nblk + c0 / 32) * 2);
  const int w0 = c0 / 10;
  uint32_t w[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) w[i] = (w0 + i < M.wpr) ? codes[w0 + i] : 0u;
  _Float16 out[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int c = c0 + i;
    const int wi = c / 10 - w0, j = c % 10;
    const uint32_t word = wi == 0 ? w[0] : (wi == 1 ? w[1] : w[2]);
    const int sh = j < 5 ? 3 * j : 16 + 3 * (j - 5);
    const int q = (int)((word >> sh) & 7u);
    out[i] = (_Float16)(q - 4) * s;
  }
#pragma unroll
  for (int i = 0; i < 16; i += 8)
    *reinterpret_cast<h8 *>(dst + i) =
        (h8){out[i], out[i + 1], out[i + 2], out[i + 3], out[i + 4], out[i + 5], out[i + 6], out[i + 7]};
}

__device__ inline f4 mfma(h8 a, h8 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }

// gate & up for one tile, h = silu(g) * u -> h16
__global__ void __launch_bounds__(256) prefill_gateup_kernel(PrefillParams P) {
  __shared__ _Float16 xs[kTM][kLd];
  __shared__ _Float16 wg[kTN][kLd];
  __shared__ _Float16 wu[kTN][kLd];
  __shared__ int tok_sh[kTM], row_sh[kTM];
  const int ntile = P.d_ff / kTN;
  const int item = blockIdx.x;
  if (item >= min(P.n_work[0], P.max_work) * ntile) return;
  const moe::WorkEntry we = P.work[item / ntile];
  const int nt = item % ntile;
  if (!entry_ok(P, we)) return;
  const uint8_t *blob = entry_blob(P, we);
  if (!blob) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < kTM) {
    int tok = -1, row = -1;
    if (tid < we.m && !entry_token(P, we, tid, tok, row)) tok = row = -1;
    tok_sh[tid] = tok;
    row_sh[tid] = row;
  }
  __syncthreads();
  const int wm = wave >> 1, wn = wave & 1;  // 2 x 2 waves, 32 x 32 each
  f4 ag[2][2], au[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      ag[a][b] = (f4){0.f, 0.f, 0.f, 0.f};
      au[a][b] = (f4){0.f, 0.f, 0.f, 0.f};
    }
  // loader roles: x rows (64 x 4 chunks of 8 halves); weights (2 mats x 64 rows x 2 halves of 16)
  const int xr = tid >> 2, xc = (tid & 3) * 8;
  const int wmat = tid >> 7, wrow = (tid >> 1) & 63, wh = tid & 1;
  const moe::MatLayout &WM = wmat == 0 ? P.gate : P.up;
  _Float16(*wdst)[kLd] = wmat == 0 ? wg : wu;
  for (int k0 = 0; k0 < P.d_model; k0 += kKB) {
    {
      const int tk = tok_sh[xr];
      h8 v = (h8){0, 0, 0, 0, 0, 0, 0, 0};
      if (tk >= 0) v = *reinterpret_cast<const h8 *>(P.x16 + (size_t)tk * P.d_model + k0 + xc);
      *reinterpret_cast<h8 *>(&xs[xr][xc]) = v;
    }
    deq16(blob, WM, nt * kTN + wrow, k0 + 16 * wh, &wdst[wrow][16 * wh]);
    __syncthreads();
    const int r = lane & 15, kg = (lane >> 4) * 8;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const h8 A = *reinterpret_cast<const h8 *>(&xs[wm * 32 + a * 16 + r][kg]);
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const h8 Bg = *reinterpret_cast<const h8 *>(&wg[wn * 32 + b * 16 + r][kg]);
        const h8 Bu = *reinterpret_cast<const h8 *>(&wu[wn * 32 + b * 16 + r][kg]);
        ag[a][b] = mfma(A, Bg, ag[a][b]);
        au[a][b] = mfma(A, Bu, au[a][b]);
      }
    }
    __syncthreads();
  }
  // D: lane holds tokens 4*(lane/16)+i (of the 16-row subtile) for column lane%16
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = wm * 32 + a * 16 + 4 * (lane >> 4) + i;
        const int col = nt * kTN + wn * 32 + b * 16 + (lane & 15);
        const int hrow = row_sh[m];
        if (hrow < 0) continue;
        const float gv = ag[a][b][i], uv = au[a][b][i];
        const float h = gv / (1.0f + __expf(-gv)) * uv;
        P.h16[(size_t)hrow * P.d_ff + col] = (_Float16)h;
      }
}

// down for one tile: y = W_d h
__global__ void __launch_bounds__(256) prefill_down_kernel(PrefillParams P) {
  __shared__ _Float16 hs[kTM][kLd];
  __shared__ _Float16 wd[kTN][kLd];
  __shared__ int row_sh[kTM], tok_sh[kTM];
  const int ntile = P.d_model / kTN;
  const int item = blockIdx.x;
  if (item >= min(P.n_work[0], P.max_work) * ntile) return;
  const moe::WorkEntry we = P.work[item / ntile];
  const int nt = item % ntile;
  if (!entry_ok(P, we)) return;
  const uint8_t *blob = entry_blob(P, we);
  if (!blob) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < kTM) {
    int tok = -1, row = -1;
    if (tid < we.m && !entry_token(P, we, tid, tok, row)) tok = row = -1;
    tok_sh[tid] = tok;
    row_sh[tid] = row;
  }
  __syncthreads();
  const int wm = wave >> 1, wn = wave & 1;
  f4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = (f4){0.f, 0.f, 0.f, 0.f};
  const int xr = tid >> 2, xc = (tid & 3) * 8;
  const int wrow = tid >> 1, wh = tid & 1;  // 128 loaders for 64 rows x 2 halves
  for (int k0 = 0; k0 < P.d_ff; k0 += kKB) {
    {
      const int hr = row_sh[xr];
      h8 v = (h8){0, 0, 0, 0, 0, 0, 0, 0};
      if (hr >= 0) v = *reinterpret_cast<const h8 *>(P.h16 + (size_t)hr * P.d_ff + k0 + xc);
      *reinterpret_cast<h8 *>(&hs[xr][xc]) = v;
    }
    if (tid < 2 * kTN) deq16(blob, P.down, nt * kTN + wrow, k0 + 16 * wh, &wd[wrow][16 * wh]);
    __syncthreads();
    const int r = lane & 15, kg = (lane >> 4) * 8;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const h8 A = *reinterpret_cast<const h8 *>(&hs[wm * 32 + a * 16 + r][kg]);
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const h8 B = *reinterpret_cast<const h8 *>(&wd[wn * 32 + b * 16 + r][kg]);
        acc[a][b] = mfma(A, B, acc[a][b]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = wm * 32 + a * 16 + 4 * (lane >> 4) + i;
        const int col = nt * kTN + wn * 32 + b * 16 + (lane & 15);
        const int hrow = row_sh[m];
        if (hrow < 0) continue;
        float *y = we.expert >= 0 ? P.y_pairs + (size_t)hrow * P.d_model : P.y_shared + (size_t)tok_sh[m] * P.d_model;
        y[col] = acc[a][b][i];
      }
}

__global__ void __launch_bounds__(256) to_fp16_kernel(const float *__restrict__ x, size_t n, _Float16 *__restrict__ y) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = (_Float16)x[i];
}

}  // namespace

namespace moe {

hipError_t launch_bucket_ex(const moe_ctx *c, const int32_t *idx, int T, int32_t *offsets, int32_t *perm, bool build,
                            int entry_m, const float *x, uint16_t *xrec, int xrec_h, hipStream_t s);

hipError_t launch_ffn_prefill(const moe_ctx *c, int layer, const float *x, int T, const int32_t *idx,
                              const int32_t *slot_of_pair, float *y_pairs, float *y_shared, hipStream_t s) {
  const moe_config &k = c->cfg;
  if (k.d_ff % kTN || k.d_model % kTN) return hipErrorInvalidValue;
  hipError_t e = launch_bucket_ex(c, idx, T, c->offsets_ws, c->perm_ws, true, kTM, nullptr, nullptr, 0, s);
  if (e != hipSuccess) return e;
  const size_t nx = (size_t)T * k.d_model;
  hipLaunchKernelGGL(to_fp16_kernel, dim3((unsigned)((nx + 255) / 256)), dim3(256), 0, s, x, nx, (_Float16 *)c->x16);
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
  P.y_pairs = y_pairs;
  P.y_shared = y_shared;
  P.d_model = k.d_model;
  P.d_ff = k.d_ff;
  // entries hold <= 64 tokens: at most pairs/64 + min(E, pairs) routed ones + the shared ones
  const int pairs = T * k.top_k;
  const int ents = pairs / kTM + (pairs < k.n_experts ? pairs : k.n_experts) + (T + kTM - 1) / kTM;
  hipLaunchKernelGGL(prefill_gateup_kernel, dim3(ents * (k.d_ff / kTN)), dim3(256), 0, s, P);
  hipLaunchKernelGGL(prefill_down_kernel, dim3(ents * (k.d_model / kTN)), dim3(256), 0, s, P);
  return hipGetLastError();
}

}  // namespace moe
