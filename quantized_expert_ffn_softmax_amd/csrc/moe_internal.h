// Internal declarations of libmoe (gfx950).  Not installed; the public
// boundary is include/libmoe.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "fill.h"
#include "libmoe.h"

namespace moe {

// ---------------------------------------------------------------------------
// Blob layout (the 3-bit stand-in for the pages' IQ3 experts; see libmoe.h)
// ---------------------------------------------------------------------------
constexpr int kScaleBlock = 32;   // inputs per fp16 scale
constexpr int kCodesPerWord = 10; // 3-bit codes per uint32
constexpr int kSbCols = 160;      // lcm(10, 32): the column period of the layout
constexpr int kSbWords = 16;      // words in one 160-column superblock
constexpr int kSbBlocks = 5;      // scale blocks in one superblock
constexpr int kSteps = 20;        // 16x16x32 MFMA steps per superblock (80 pairs / 4)

struct MatLayout {
  int rows, cols;
  int wpr;       // words per row
  int nblk;      // scale blocks per row = cols / 32
  int nsb;       // superblocks per row = ceil(cols / 160)
  uint32_t code_off, scale_off;  // byte offsets inside the blob
};

struct BlobLayout {
  MatLayout gate, up, down;
  uint32_t stride;
};

inline int words_per_row(int cols) {
  int w = (cols + kCodesPerWord - 1) / kCodesPerWord;
  return (w + 3) / 4 * 4;
}

inline BlobLayout make_layout(int d_model, int d_ff) {
  BlobLayout L{};
  uint32_t pos = 0;
  MatLayout *m[3] = {&L.gate, &L.up, &L.down};
  int rows[3] = {d_ff, d_ff, d_model};
  int cols[3] = {d_model, d_model, d_ff};
  for (int i = 0; i < 3; ++i) {
    MatLayout &M = *m[i];
    M.rows = rows[i];
    M.cols = cols[i];
    M.wpr = words_per_row(cols[i]);
    M.nblk = cols[i] / kScaleBlock;
    M.nsb = (cols[i] + kSbCols - 1) / kSbCols;
    M.code_off = pos;
    pos += (uint32_t)M.rows * M.wpr * 4;
    M.scale_off = pos;
    pos += (uint32_t)M.rows * M.nblk * 2;
  }
  L.stride = (pos + 255u) / 256u * 256u;
  return L;
}

// Decode path: activations in "MFMA step order", split into two fp16 halves.
// For one token and one matrix with nsb superblocks the record holds, for each
// superblock S and step t, 8 hi halves then 8 lo halves (32 bytes); the 8
// halves are the columns of pairs p = 4t..4t+3 of the superblock, pair p
// being (c, c+5) with c = 160 S + 10 (p / 5) + p % 5.
inline int xrec_halves(int nsb) { return nsb * kSteps * 16; }

// One unit of decode work: up to kEntryTokens tokens of one expert (or of the
// shared expert) in one layer.  The decode kernels put a token's hi half in
// MFMA column n and its lo half in column n + 4, and keep an entry's whole
// activation record (4 columns) in LDS, hence 4.
constexpr int kEntryTokens = 4;
// The second work list of the decode path: entries of up to 8 tokens (the
// kernels built for it put token n's hi half in MFMA column n and its lo half
// in column n + 8, every column in use).
constexpr int kEntryTokens8 = 8;
// Superblocks per row the decode kernels are built for: all of a unit's
// word quads are requested at once, which bounds K (d_model, d_ff <= 2048).
constexpr int kDecodeMaxNsb = 13;
struct WorkEntry {
  int32_t expert;  // routed expert index, or -1 for the shared expert
  int32_t first;   // routed: index into perm of the first pair; shared: first token
  int32_t m;       // tokens in this entry, 1..kEntryTokens
  int32_t pad;
};

}  // namespace moe

struct moe_ctx {
  moe_config cfg;
  moe::BlobLayout L;
  bool resident;
  int device;

  // slot table (device)
  int32_t *slot_of;   // [n_layers * n_experts]
  int32_t *id_of;     // [n_slots]
  uint32_t *stamp;    // [n_slots]
  const uint8_t *host_dev;  // host_store as mapped into the device address space (null: not mapped)
  int64_t *dstats;    // device: lookups, hits, misses, calls

  // workspace (device)
  float *logits_ws;      // [max_tokens][n_experts]
  int32_t *offsets_ws;   // [n_experts + 1]
  int32_t *perm_ws;      // [max_pairs]
  int32_t *chunk_ws;     // [n_chunks][n_experts] for the large bucketing
  moe::WorkEntry *work;  // [max_work]
  moe::WorkEntry *work8; // [max_work8]: the decode path's second list, entries of <= kEntryTokens8
  int32_t *n_work;       // [4]: entries, routed entries (work), then the same for work8
  // x record: [max_tokens + 1][xrec_halves(gate.nsb)] (last row zero); the
  // decode path's layout, or on the prefill path its own layout of the same
  // size per token (each call rebuilds the rows it uses)
  uint16_t *xrec;
  uint16_t *hrec;        // decode h record: [max_pairs + max_tokens + 1][xrec_halves(down.nsb)]
  uint16_t *h16;         // prefill h record: [max_pairs + max_tokens][down.nsb * 160 * 2] fp16 (hi, lo), pads zero
  int32_t *slot_ws;      // [max_pairs] slots when the caller passes none
  float *route_part;     // [route_ks][route_small_t][n_experts] partial logits (decode-size router)
  int32_t route_ks;      // column slices of the decode-size router
  int32_t route_small_t; // largest T routed by the decode-size router (<= 64)
  int32_t max_pairs;
  int32_t max_work;
  int32_t max_work8;
  int32_t n_chunks_max;
  int32_t n_cu;          // compute units of the context's device
  int32_t decode_occ[4]; // decode FFN workgroups per CU: gate/up, down, gate/up K in halves, in quarters (at create)

  // miss path
  int32_t *dmiss;        // device: [0]=unique, [1]=misses, [2]=error, then (id, slot) pairs
  int32_t *hmiss;        // pinned host mirror
  hipStream_t side;
  hipEvent_t ev_main, ev_copy;
};

// error helpers (host)
moe_status moe_fail(moe_status s, const std::string &msg);
#define MOE_HIP(call)                                                        \
  do {                                                                       \
    hipError_t _e = (call);                                                  \
    if (_e != hipSuccess)                                                    \
      return moe_fail(MOE_ERR_HIP, std::string(#call) + ": " + hipGetErrorString(_e)); \
  } while (0)
#define MOE_CHECK(cond, code, msg)                                           \
  do {                                                                       \
    if (!(cond)) return moe_fail((code), (msg));                             \
  } while (0)

// launch wrappers implemented in the kernel files (return hipError_t)
namespace moe {
hipError_t launch_router(const moe_ctx *c, const float *x, int T, const float *wr, const float *bias,
                         float *logits, int32_t *idx, float *w, hipStream_t s);
// the decode-size router's first kernel alone (partial logits into
// c->route_part); T <= c->route_small_t
hipError_t launch_router_partials(const moe_ctx *c, const float *x, int T, const float *wr, hipStream_t s);
// capped cache, T <= 2 (the decode layer uses it at T = 1): the router's top-k from c->route_part and the
// resolve (no fill kernel; a call that cannot pin its working set gives every
// pair slot -1) in one single-workgroup launch
hipError_t launch_route_resolve(moe_ctx *c, int layer, int T, const float *bias, float *logits, int32_t *idx,
                                float *w, int32_t *slot_of_pair, hipStream_t s);
hipError_t launch_bucket(const moe_ctx *c, const int32_t *idx, int T, int32_t *offsets, int32_t *perm,
                         bool build_work, hipStream_t s);
// bucketing with the work list of entry_m-token entries (and, with work8, the
// second list of kEntryTokens8-token entries) and, with x, the decode record
hipError_t launch_bucket_ex(const moe_ctx *c, const int32_t *idx, int T, int32_t *offsets, int32_t *perm, bool build,
                            int entry_m, const float *x, uint16_t *xrec, int xrec_h, hipStream_t s,
                            moe::WorkEntry *work8);
// fill: misses are filled with no host round trip, and a call that cannot
// pin its working set gives every pair slot -1; the fill kernel is launched
// unless launch_fill is false (the caller then runs launch_bucket_fill)
hipError_t launch_resolve(moe_ctx *c, int layer, const int32_t *idx, int T, int32_t *slot_of_pair, bool fill,
                          hipStream_t s, bool launch_fill = true);
hipError_t decode_occupancy(moe_ctx *c);  // fills c->decode_occ for c's superblock counts
hipError_t launch_ffn_decode(const moe_ctx *c, int layer, const float *x, int T, const int32_t *idx,
                             const int32_t *slot_of_pair, float *y_pairs, float *y_shared, hipStream_t s);
// the decode FFN kernels alone, on the work list, perm and x record already
// in the context's workspace (from launch_ffn_decode's bucketing or from
// launch_route_bucket)
hipError_t launch_ffn_decode_kernels(const moe_ctx *c, int layer, int T, const int32_t *slot_of_pair, float *y_pairs,
                                     float *y_shared, hipStream_t s);
// resident cache: the lookup count (as launch_resolve records it) + the
// bucketing with its work list (entry_m) + the x record, in one launch;
// T * top_k <= 1024, n_experts <= 1024
hipError_t launch_bucket_lookup(const moe_ctx *c, const int32_t *idx, int T, int entry_m, const float *x,
                                uint16_t *xrec, int xrec_h, hipStream_t s);
// resident cache, T <= 2 (the decode layer uses it at T = 1): the router's top-k from c->route_part, the lookup
// count, the bucketing with its work lists and the x record, in one launch
hipError_t launch_route_bucket_lookup(const moe_ctx *c, int T, const float *bias, float *logits, int32_t *idx, float *w,
                                     int entry_m, const float *x, uint16_t *xrec, int xrec_h, hipStream_t s);
// the zero-copy fill's arguments for c's cache, `chunks` workgroups per blob
FillArgs fill_args(const moe_ctx *c, int chunks);
// capped cache: the bucketing with its work lists, the x record (with x) and,
// in further workgroups of the same launch, the zero-copy fill of the misses
// that launch_resolve (launch_fill = false) listed; T * top_k <= 1024,
// n_experts <= 1024
hipError_t launch_bucket_fill(const moe_ctx *c, const int32_t *idx, int T, int entry_m, const float *x,
                              uint16_t *xrec, int xrec_h, hipStream_t s);
hipError_t launch_ffn_prefill(const moe_ctx *c, int layer, const float *x, int T, const int32_t *idx,
                              const int32_t *slot_of_pair, float *y_pairs, float *y_shared, hipStream_t s);
hipError_t launch_combine(const float *y_pairs, const float *w, const float *y_shared, int T, int k, int d,
                          float *out, hipStream_t s);
hipError_t launch_chain_norm(const float *out, int T, int d, float *x_next, hipStream_t s);
hipError_t launch_combine_norm(const float *y_pairs, const float *w, const float *y_shared, int T, int k, int d,
                               float *out, float *x_next, hipStream_t s);
}  // namespace moe
