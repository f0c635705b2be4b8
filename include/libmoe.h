/*
 * libmoe -- routed MoE layer with 3-bit block-quantised experts, for AMD
 * Instinct MI355X (gfx950).  Plain C ABI: device or host pointers and sizes,
 * no framework types.
 *
 * The layer is the one the Strata engine runs on the pages
 * ("一张 RTX 4090 跑千亿模型，Strata 实测 155 tok/s", section 如何做到：三层存储):
 * every token is routed to 10 of a layer's 512 experts plus one shared
 * expert; the (layer, expert) identities -- 48 x 512 = 24,576 of them
 * ("从一张到四张 RTX 4090 ...", section 先看结果: 48 layers) -- live in a
 * pool of VRAM slots; a hit is computed straight from its slot, a miss is
 * fetched from host RAM over PCIe first.  The pages name the IQ3 formats but
 * print neither their layout, the router's scoring, the activation nor the
 * eviction policy; the readings used here are spelled out per call below.
 *
 * Conventions for every call:
 *  - returns MOE_OK or a negative moe_status; on a validation error nothing
 *    is enqueued and no state changes; moe_last_error() gives detail;
 *  - pointers are DEVICE pointers unless marked (host);
 *  - `stream` is a hipStream_t (NULL = the null stream); work is enqueued
 *    on it asynchronously unless the call says otherwise;
 *  - tensors are row-major and contiguous; the caller owns every tensor it
 *    passes; a context owns only its own slot table, workspace, pinned miss
 *    list, side stream and events;
 *  - one host thread uses a context at a time.
 *
 * Expert blob (one per identity, and one shared blob per layer), at
 * moe_expert_bytes(d_model, d_ff) bytes apart: gate [d_ff][d_model], up
 * [d_ff][d_model], down [d_model][d_ff]; each matrix is `codes`
 * [rows][wpr] uint32 followed by `scales` [rows][cols/32] fp16, with
 * wpr = ceil(cols/10) rounded up to a multiple of 4.  Weight (r, c) has code
 * q = (codes[r][c/10] >> sh(c%10)) & 7 with sh(j) = 3j for j < 5 and
 * 16 + 3(j-5) otherwise, and value (q - 4) * scales[r][c/32].  Unused code
 * slots and pad words are zero.  Block scales must satisfy
 * 2^-14 <= |s| <= 255.875 or s = 0: the FFN kernels form f * fp16((q - 4) * s)
 * with f = 1, 8 or 64, which leaves fp16's normal range outside it.
 */
#ifndef LIBMOE_H
#define LIBMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID = -1,  /* bad argument (null, out of range, wrong shape) */
  MOE_ERR_ALIGN = -2,    /* pointer not aligned as the call requires */
  MOE_ERR_CAPACITY = -3, /* a resolve touches more identities than the pool can pin */
  MOE_ERR_HIP = -4,      /* a HIP runtime call failed; moe_last_error() has its text */
  MOE_ERR_OOM = -5       /* the context could not allocate its own state */
} moe_status;

enum { MOE_PATH_AUTO = 0, MOE_PATH_DECODE = 1, MOE_PATH_PREFILL = 2 };

typedef struct moe_ctx moe_ctx;

typedef struct {
  int32_t d_model;      /* multiple of 64, <= 8192 (the blob format itself allows 32) */
  int32_t d_ff;         /* multiple of 64, <= 8192 */
  int32_t n_experts;    /* routed experts per layer, 1..1024 */
  int32_t top_k;        /* 1..min(n_experts, 32) */
  int32_t n_layers;     /* >= 1 */
  int32_t n_slots;      /* VRAM slots; == n_layers*n_experts means every identity is
                           resident at slot = identity (no host store, no LRU) */
  int32_t max_tokens;   /* largest T any call will pass; sizes the workspace */
  const void *host_store; /* (host, pinned) [n_layers*n_experts][blob]; required when
                             n_slots < n_layers*n_experts, else may be NULL */
  void *slot_pool;        /* [n_slots][blob], 256-byte aligned */
  const void *shared_pool;/* [n_layers][blob], 256-byte aligned */
} moe_config;

typedef struct {
  int64_t lookups;      /* unique (layer, expert) identities asked for */
  int64_t hits;         /* of those, already resident */
  int64_t misses;       /* copied in from the host store */
  uint64_t bytes_h2d;   /* bytes copied host -> device for misses */
  int64_t resolve_calls;
  int64_t failed_calls; /* calls that could not pin their working set (moe_cache_resolve_async
                           reports its capacity failures only here) */
} moe_resolve_info;

/* Bytes between consecutive blobs: the layout above rounded up to 256.
 * 2,228,224 at (2048, 768); 51,200 at (256, 128); 0 for invalid dims. */
size_t moe_expert_bytes(int32_t d_model, int32_t d_ff);

/* Validates cfg and allocates the context's own state: slot table
 * (slot_of[n_layers*n_experts], id_of[n_slots], stamp[n_slots]) in device
 * memory, workspace sized by max_tokens, a pinned miss list, a side stream
 * and events.  Does not touch slot_pool / shared_pool / host_store, which the
 * caller fills.  The cache starts empty (every slot free, clock 0). */
moe_status moe_create(const moe_config *cfg, moe_ctx **out);

/* Synchronises the context's side stream and frees its own state. */
moe_status moe_destroy(moe_ctx *ctx);

/* Router of one layer (the pages: 10 of 512 experts per token).  Reading:
 *   logits[t][e] = sum_c x[t][c] * w_router[e][c] + bias[e]    (fp32)
 *   idx[t][0..k)  = the k experts with the largest logits, ordered by logit
 *                   descending, ties to the lower expert index
 *   w[t][j]       = exp(l_j - l_max) / sum_j' exp(l_j' - l_max), i.e. the
 *                   softmax over all experts renormalised over the k chosen.
 * x [T][d_model], w_router [n_experts][d_model], bias [n_experts] or NULL,
 * logits [T][n_experts] or NULL (not returned), idx [T][top_k] int32,
 * w [T][top_k].  1 <= T <= max_tokens.  Asynchronous. */
moe_status moe_route(moe_ctx *ctx, int32_t layer, const float *x, int32_t T,
                     const float *w_router, const float *bias, float *logits,
                     int32_t *idx, float *w, void *stream);

/* Maps the routed pairs of one layer to VRAM slots (the pages' hot cache:
 * hits from VRAM, misses over PCIe from host RAM).  idx [T][top_k] as from
 * moe_route; slot_of_pair [T][top_k] int32 out (may be NULL when every
 * identity is resident, in which case nothing is enqueued for it).
 * Resident mode (n_slots == n_layers*n_experts): slot = layer*E + expert,
 * asynchronous.  Capped mode: LRU reading -- each call advances a clock; hits
 * get stamp = clock; misses, in ascending identity order, take the lowest free
 * slot, else the slot with the smallest (stamp, slot) among slots whose stamp
 * is older than this call; the call synchronises on its resolve kernel,
 * copies each missed blob host_store[id] -> slot_pool[slot] with
 * hipMemcpyAsync on the side stream (after the work already on `stream`),
 * and makes `stream` wait for those copies before returning.  If one call
 * touches more identities than n_slots, it returns MOE_ERR_CAPACITY and the
 * slot table is left as before the call.  info (host) may be NULL; it gets this
 * call's counts. */
moe_status moe_cache_resolve(moe_ctx *ctx, int32_t layer, const int32_t *idx, int32_t T,
                             int32_t *slot_of_pair, moe_resolve_info *info, void *stream);

/* The same slot assignment with no host round trip, so that a whole decode
 * step can be enqueued (or captured in a HIP graph) without synchronising:
 * the resolve kernel is followed on `stream` by a fill kernel that copies each
 * missed blob from host_store[id] to slot_pool[slot] by reading the pinned host
 * store directly (zero-copy over the host link).  host_store must be mapped
 * into the device address space (memory from hipHostMalloc is); otherwise the
 * call returns MOE_ERR_INVALID and enqueues nothing.  The clock and the slot
 * table live in device memory and are shared with moe_cache_resolve: the two
 * may be mixed on one context, and give the same slots call for call.  A call
 * that touches more identities than n_slots changes no table entry, writes -1
 * to every slot_of_pair entry (moe_expert_ffn then writes no output for those
 * pairs) and counts one failed call in moe_get_stats; nothing else reports it.
 * Calls on one context must not overlap; they are ordered by `stream`. */
moe_status moe_cache_resolve_async(moe_ctx *ctx, int32_t layer, const int32_t *idx, int32_t T,
                                   int32_t *slot_of_pair, void *stream);

/* Expert FFNs of one layer (each token runs the 10 of 512 routed experts its
 * router chose plus the layer's one shared expert: "一张 RTX 4090 跑千亿模型，
 * Strata 实测 155 tok/s", section 如何做到：三层存储; the gated form below,
 * W_d (silu(W_g x) * W_u x), is the plainest reading of an expert FFN, which
 * the pages do not spell out):  for every pair p = t*top_k + j,
 *   y_pairs[p] = W_d (silu(W_g x_t) * (W_u x_t))  with the expert blob at
 *                slot_pool[slot_of_pair[p]] (or the resident slot
 *                layer*E + idx[p] when slot_of_pair is NULL),
 *   y_shared[t] = the same with the layer's shared blob,
 * silu(z) = z / (1 + exp(-z)).  x [T][d_model] fp32; y_pairs
 * [T*top_k][d_model] fp32; y_shared [T][d_model] fp32.
 * path: MOE_PATH_DECODE -- dequantised weights rounded once to fp16,
 * activations kept at fp32 accuracy (split in two fp16 halves), fp32
 * accumulation; takes d_model and d_ff up to 2048 (13 superblocks of 160
 * columns), MOE_ERR_INVALID above; MOE_PATH_PREFILL -- the same precision
 * (dequantised weights rounded once to fp16, x and h carried as two fp16
 * halves, fp32 accumulation) as a grouped GEMM, needs d_model and d_ff to be
 * multiples of 64 and the call's activation records to stay under 4 GiB --
 * T * 5 * ceil(d_model / 160) * 128 bytes for x and (T * top_k + T) * 5 *
 * ceil(d_ff / 160) * 128 bytes for h (MOE_ERR_INVALID otherwise; d_ff =
 * 8192 reaches it near T = 12,000); MOE_PATH_AUTO -- decode for T <= 64 when
 * the dims allow it, prefill otherwise when it can take the call, else
 * decode.  Expert ids outside [0, n_experts) are ignored
 * (their y_pairs rows are not written).  Uses the context's workspace: calls
 * on one context must not overlap.  Asynchronous; deterministic (no
 * floating-point atomics). */
moe_status moe_expert_ffn(moe_ctx *ctx, int32_t layer, const float *x, int32_t T,
                          const int32_t *idx, const int32_t *slot_of_pair,
                          float *y_pairs, float *y_shared, int32_t path, void *stream);

/* The layer's output from its routed experts and its shared expert (same
 * section as moe_expert_ffn; the weighting -- the router's softmax weights
 * on the routed outputs, the shared expert ungated -- is the plainest
 * reading, the pages give no formula):
 * out[t] = sum_{j = 0..k-1, ascending} w[t][j] * y_pairs[t*k + j] + y_shared[t]
 * (the shared expert added last).  fp32 throughout. */
moe_status moe_combine(moe_ctx *ctx, const float *y_pairs, const float *w,
                       const float *y_shared, int32_t T, float *out, void *stream);

/* One whole decode layer; on a resident cache in six launches instead of the
 * seven of the separate calls (five for a single token, whose top-k joins
 * the bucketing launch) (the pages' engine has a fused-kernel mode,
 * "融合核": "从一张到四张 RTX 4090 ...", section 调参：前后 40 多次重启):
 * the router's two launches; one launch for the resident lookup count, the
 * bucketing and the activation record; the two FFN kernels; the combine
 * (and, with x_next, the normalisation that chains layers).  Results, bit for
 * bit, and counters (moe_get_stats: lookups, hits, resolve calls) are those of
 *   moe_route(ctx, layer, x, T, w_router, bias, logits, idx, w)
 *   moe_cache_resolve(ctx, layer, idx, T, NULL, NULL)
 *   moe_expert_ffn(ctx, layer, x, T, idx, NULL, y_pairs, y_shared, MOE_PATH_DECODE)
 *   x_next ? moe_combine_norm(ctx, y_pairs, w, y_shared, T, out, x_next)
 *          : moe_combine(ctx, y_pairs, w, y_shared, T, out).
 * Arguments as there; logits and x_next may be NULL; x_next must differ from
 * x and out.  Needs T * top_k <= 1,024 and d_model, d_ff <= 2048.
 *
 * On a capped cache (its host_store mapped into the device address space,
 * i.e. from hipHostMalloc) the layer resolves through the LRU table in the
 * context's own slot array.  Results, table, stamps and counters are those of
 * the separate calls with moe_cache_resolve_async in place of
 * moe_cache_resolve, the slots' contents included.  The pages put the cost
 * of a miss in the host link ("一张 RTX 4090 跑千亿模型 ...", section
 * 如何做到：三层存储); the missed blobs are copied from the mapped host store
 * as moe_cache_resolve_async's fill kernel copies them, but by spare
 * workgroups of the bucketing launch, which does not depend on the resolve:
 * seven launches instead of the separate calls' eight, and six for a single
 * token, whose top-k and resolve share one workgroup.  A call that cannot
 * pin its working set changes nothing in the table, counts one failed call
 * and leaves its pairs' y_pairs rows unwritten (out is then not
 * meaningful).
 *
 * MOE_ERR_INVALID otherwise (a capped cache whose host_store is not mapped,
 * shapes out of range), nothing enqueued.  Asynchronous; uses the context's
 * workspace. */
moe_status moe_decode_layer(moe_ctx *ctx, int32_t layer, const float *x, int32_t T,
                            const float *w_router, const float *bias, float *logits,
                            int32_t *idx, float *w, float *y_pairs, float *y_shared,
                            float *out, float *x_next, void *stream);

/* --- KV tier --------------------------------------------------------------
 * The pages' engine keeps the KV cache as int8 at 1,056 bytes per cell, locks
 * only the first 32,768 of a layer's 131,072 cells in VRAM and streams the
 * rest from pinned host RAM, with an optional prefetch ("单卡5090跑125B 大模型
 * ...", section 2.2; "一张 RTX 4090 跑千亿模型，Strata 实测 155 tok/s",
 * section 四个发现); it reports the share of block reads served from VRAM
 * (section 7.2 of the first page: 98.8%).  The cell layout is not printed;
 * the reading: `values` int8 codes in groups of 64, then one fp16 scale per
 * group (1,024 values: 1,024 + 32 = 1,056 bytes); a group's scale is
 * s = fp16(absmax / 127) and its codes q = clamp(rint(v / s), -127, 127)
 * (float32 division, ties to even; s = 0 stores zero codes); a value reads
 * back as q * s.  Cell c of a layer lives in HBM when c < cells_resident,
 * else in host memory at index c - cells_resident.  The caller owns both
 * stores; the handle owns a staging buffer of two slots of stage_cells cells
 * and the counters.  One host thread uses a handle at a time. */
typedef struct moe_kv moe_kv;

typedef struct {
  int32_t n_layers;
  int32_t values;          /* per cell: 1,024, 2,048, 3,072 or 4,096 */
  int32_t cells_total;     /* per layer */
  int32_t cells_resident;  /* the first cells of each layer kept in HBM, 0..cells_total */
  int32_t block_cells;     /* cells per block of the read accounting, >= 1 */
  int32_t stage_cells;     /* capacity of each of the two staging slots, 1..cells_total */
  void *resident;          /* device [n_layers][cells_resident][cell_bytes], 16-byte aligned */
  void *host;              /* (host, pinned by hipHostMalloc) [n_layers][cells_total - cells_resident][cell_bytes] */
} moe_kv_config;

typedef struct {
  int64_t cells_written;
  int64_t cells_read;
  int64_t block_reads;       /* blocks touched by reads (a read of a block's cells counts once) */
  int64_t vram_block_reads;  /* of those, served entirely from HBM (resident or staged cells) */
  int64_t host_bytes;        /* bytes reads took from host memory over the link */
  int64_t prefetch_bytes;    /* bytes prefetches copied into the staging slots */
} moe_kv_stats;

/* Bytes per cell (values + 2 * values / 64), 0 for an unsupported `values`. */
size_t moe_kv_cell_bytes(int32_t values);

/* Validates cfg, maps `host` into the device address space and allocates the
 * staging buffer.  MOE_ERR_INVALID for a bad cfg or a host buffer that is not
 * mapped pinned memory; MOE_ERR_OOM if the staging buffer cannot be made. */
moe_status moe_kv_create(const moe_kv_config *cfg, moe_kv **out);
moe_status moe_kv_destroy(moe_kv *kv);

/* Quantises vals [n][values] (device, fp32) into cells [first, first + n) of
 * `layer`: resident cells in HBM, the others straight into host memory
 * (stores over the link), and into a staging copy too when one holds them.
 * Asynchronous on `stream`. */
moe_status moe_kv_write(moe_kv *kv, int32_t layer, int32_t first, int32_t n,
                        const float *vals, void *stream);

/* Reads cells [first, first + n) of `layer` back into out [n][values]
 * (device, fp32, q * s): resident cells from HBM, the others from a staging
 * slot that holds them, else from host memory (loads over the link).  The
 * block accounting (moe_kv_get_stats) is done at enqueue, from the staging
 * state at that moment.  Asynchronous on `stream`. */
moe_status moe_kv_read(moe_kv *kv, int32_t layer, int32_t first, int32_t n,
                       float *out, void *stream);

/* Brings the host cells of [first, first + n) (n <= stage_cells) into the
 * older of the two staging slots by one hipMemcpyAsync on `stream`; reads
 * enqueued after it use that copy.  The slot's previous range is dropped at
 * enqueue: a read of it must be ordered before this call's copy (same stream,
 * or an event), and a read of the new range after it.  Writes keep staged
 * copies equal to host memory. */
moe_status moe_kv_prefetch(moe_kv *kv, int32_t layer, int32_t first, int32_t n, void *stream);

/* Cumulative counters (host state; no synchronisation). */
moe_status moe_kv_get_stats(moe_kv *kv, moe_kv_stats *out);

/* --- observability and test support ------------------------------------- */

/* Token -> expert bucketing as moe_expert_ffn does it internally:
 * offsets [n_experts+1] int32 (exclusive scan of per-expert pair counts,
 * offsets[E] = T*top_k) and perm [T*top_k] int32 (pair ids grouped by expert
 * ascending, ascending pair id inside a group).  Asynchronous. */
moe_status moe_bucket(moe_ctx *ctx, const int32_t *idx, int32_t T, int32_t *offsets,
                      int32_t *perm, void *stream);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): moe_bucket without a
 * context.  offsets [n_experts+1] and perm [T*top_k] as moe_bucket writes
 * them for idx [T][top_k] (out-of-range expert ids ignored).  Past 1,024 pairs
 * the per-chunk expert counts live in a static device array of 2 MiB per GPU
 * (512 chunks x 1,024 experts), so T*top_k must be <= 131,072 and
 * n_experts <= 1,024 (MOE_ERR_INVALID otherwise, nothing enqueued); no call
 * allocates.  Every call on one GPU shares that array: calls that overlap in
 * time on one GPU (different streams, or host threads) race and must be
 * ordered by the caller.  Asynchronous on `stream`. */
moe_status moe_bucket_noalloc(const int32_t *idx, int32_t T, int32_t top_k, int32_t n_experts,
                              int32_t *offsets, int32_t *perm, void *stream);

/* Copies the slot table to host arrays (any may be NULL): slot_of
 * [n_layers*n_experts], id_of [n_slots], stamp [n_slots].  Synchronises the
 * device.  In resident mode the table is the identity and stamps are 0. */
moe_status moe_cache_snapshot(moe_ctx *ctx, int32_t *slot_of, int32_t *id_of, uint32_t *stamp);

/* Frees every slot, sets the clock and the cumulative counts to 0.
 * Synchronises the device.  The recovery path after any error. */
moe_status moe_cache_reset(moe_ctx *ctx);

/* Cumulative counts since creation or the last reset (host out). */
moe_status moe_get_stats(moe_ctx *ctx, moe_resolve_info *cumulative);

/* Stacking helper for multi-layer runs (not part of the layer): each token's
 * output centred over its d_model features and scaled to unit RMS,
 * c = out[t] - mean_c(out[t][c]);  x_next[t] = c / sqrt(mean_c(c^2) + 1e-6),
 * fp32.  out [T][d_model], x_next [T][d_model] (may not alias).  Asynchronous. */
moe_status moe_chain_norm(moe_ctx *ctx, const float *out, int32_t T, float *x_next, void *stream);

/* moe_combine followed by moe_chain_norm in one kernel (one workgroup per
 * token), for stacks that chain layers: out[t] as moe_combine writes it, and
 * x_next[t] as moe_chain_norm would compute it from that out -- bit for bit the
 * two calls' results, one dispatch instead of two.  Same shapes, alignment and
 * asynchrony as those calls; out and x_next must not overlap. */
moe_status moe_combine_norm(moe_ctx *ctx, const float *y_pairs, const float *w,
                            const float *y_shared, int32_t T, float *out, float *x_next,
                            void *stream);

/* --- measurement support ------------------------------------------------
 * Probes of what the device actually sustains, so that the layer's roofline
 * fractions can be quoted against measured peaks beside the data-sheet ones
 * (the pages print no figure for this hardware).  Both only enqueue one
 * kernel on `stream`; the caller times it (e.g. with events around the call).
 *
 * moe_peak_hbm_read: n_blocks workgroups of 256 threads load every byte of
 * buf[0, bytes) once with 16-byte loads (8 in flight per thread) and write
 * nothing unless the data XOR to one fixed 32-bit value; sink
 * [n_blocks] uint32 is scratch for that case.  buf and bytes must be
 * multiples of 16 (MOE_ERR_ALIGN otherwise).  Use bytes well above the
 * 256 MiB last-level cache so that the figure is HBM's.
 *
 * moe_peak_mfma_f16: n_blocks workgroups of 4 waves; every wave runs `iters`
 * rounds of 4 independent v_mfma_f32_32x32x16_f16 on register operands, so
 * one launch is n_blocks * 4 * iters * 4 * 32768 flops; sink [n_blocks]
 * float is scratch (written only under a condition no run meets).
 * Invalid arguments return MOE_ERR_INVALID and enqueue nothing. */
moe_status moe_peak_hbm_read(const void *buf, uint64_t bytes, uint32_t *sink, int32_t n_blocks, void *stream);
moe_status moe_peak_mfma_f16(int32_t iters, int32_t n_blocks, float *sink, void *stream);

const char *moe_status_str(moe_status s);
/* Detail of the last error on the calling thread ("" if none). */
const char *moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* LIBMOE_H */
