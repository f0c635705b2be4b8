// libmoe C ABI: argument validation, context lifetime, the miss path of the
// expert cache, and dispatch to the kernels.
#include <stdio.h>
#include <string.h>

#include <string>

#include "moe_internal.h"

static thread_local std::string g_last_error;

moe_status moe_fail(moe_status s, const std::string &msg) {
  g_last_error = msg;
  return s;
}

extern "C" const char *moe_last_error(void) { return g_last_error.c_str(); }

extern "C" const char *moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID: return "invalid argument";
    case MOE_ERR_ALIGN: return "misaligned pointer";
    case MOE_ERR_CAPACITY: return "slot pool too small for one call's working set";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_OOM: return "out of memory";
  }
  return "unknown status";
}

static bool dims_ok(int32_t d_model, int32_t d_ff) {
  return d_model >= 32 && d_ff >= 32 && d_model <= 8192 && d_ff <= 8192 && d_model % 32 == 0 &&
         d_ff % 32 == 0;
}

extern "C" size_t moe_expert_bytes(int32_t d_model, int32_t d_ff) {
  if (!dims_ok(d_model, d_ff)) return 0;
  return moe::make_layout(d_model, d_ff).stride;
}

static bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

template <typename T>
static hipError_t dalloc(T **p, size_t n) {
  *p = nullptr;
  if (n == 0) n = 1;
  return hipMalloc((void **)p, n * sizeof(T));
}

static void free_ctx(moe_ctx *c) {
  if (!c) return;
  void *dev[] = {c->slot_of, c->id_of, c->stamp, c->dstats, c->logits_ws, c->offsets_ws, c->perm_ws,
                 c->chunk_ws, c->work, c->work8, c->n_work, c->xrec, c->hrec, c->h16,
                 c->slot_ws, c->dmiss, c->route_part};
  for (void *p : dev)
    if (p) (void)hipFree(p);
  if (c->hmiss) (void)hipHostFree(c->hmiss);
  if (c->ev_main) (void)hipEventDestroy(c->ev_main);
  if (c->ev_copy) (void)hipEventDestroy(c->ev_copy);
  if (c->side) (void)hipStreamDestroy(c->side);
  delete c;
}

extern "C" moe_status moe_create(const moe_config *cfg, moe_ctx **out) {
  MOE_CHECK(cfg && out, MOE_ERR_INVALID, "moe_create: null cfg or out");
  *out = nullptr;
  const moe_config &k = *cfg;
  // the kernels copy a row's scales in 4-byte pieces: an even number of
  // scale blocks per row keeps every row 4-byte aligned
  MOE_CHECK(dims_ok(k.d_model, k.d_ff) && k.d_model % 64 == 0 && k.d_ff % 64 == 0, MOE_ERR_INVALID,
            "moe_create: d_model and d_ff must be multiples of 64 in [64, 8192]");
  MOE_CHECK(k.n_experts >= 1 && k.n_experts <= 1024, MOE_ERR_INVALID, "moe_create: n_experts must be 1..1024");
  MOE_CHECK(k.top_k >= 1 && k.top_k <= k.n_experts && k.top_k <= 32, MOE_ERR_INVALID,
            "moe_create: top_k must be 1..min(n_experts, 32)");
  MOE_CHECK(k.n_layers >= 1 && (int64_t)k.n_layers * k.n_experts <= (1 << 24), MOE_ERR_INVALID,
            "moe_create: n_layers out of range");
  const int64_t ids = (int64_t)k.n_layers * k.n_experts;
  MOE_CHECK(k.n_slots >= 1 && k.n_slots <= ids, MOE_ERR_INVALID, "moe_create: n_slots must be 1..n_layers*n_experts");
  MOE_CHECK(k.max_tokens >= 1 && k.max_tokens <= (1 << 20), MOE_ERR_INVALID, "moe_create: max_tokens must be 1..2^20");
  MOE_CHECK(k.slot_pool && k.shared_pool, MOE_ERR_INVALID, "moe_create: slot_pool and shared_pool are required");
  MOE_CHECK(aligned(k.slot_pool, 256) && aligned(k.shared_pool, 256), MOE_ERR_ALIGN,
            "moe_create: slot_pool and shared_pool must be 256-byte aligned");
  const bool resident = (int64_t)k.n_slots == ids;
  MOE_CHECK(resident || k.host_store, MOE_ERR_INVALID, "moe_create: a capped cache needs host_store");
  if (k.host_store) MOE_CHECK(aligned(k.host_store, 16), MOE_ERR_ALIGN, "moe_create: host_store must be 16-byte aligned");

  moe_ctx *c = new (std::nothrow) moe_ctx();
  MOE_CHECK(c, MOE_ERR_OOM, "moe_create: host allocation failed");
  c->cfg = k;
  c->L = moe::make_layout(k.d_model, k.d_ff);
  c->resident = resident;
  c->host_dev = nullptr;
  hipError_t e = hipGetDevice(&c->device);
  c->n_cu = 0;
  if (e == hipSuccess) e = hipDeviceGetAttribute(&c->n_cu, hipDeviceAttributeMultiprocessorCount, c->device);
  if (c->n_cu < 1) c->n_cu = 1;
  c->max_pairs = k.max_tokens * k.top_k;
  c->max_work = c->max_pairs / moe::kEntryTokens + (c->max_pairs < k.n_experts ? c->max_pairs : k.n_experts) +
                k.max_tokens / moe::kEntryTokens + 4;
  c->max_work8 = c->max_pairs / moe::kEntryTokens8 + (c->max_pairs < k.n_experts ? c->max_pairs : k.n_experts) +
                 k.max_tokens / moe::kEntryTokens8 + 4;
  c->n_chunks_max = (c->max_pairs + 255) / 256;
  const int gsb = c->L.gate.nsb, dsb = c->L.down.nsb;
  if (e == hipSuccess) e = moe::decode_occupancy(c);
  const int64_t hrows = (int64_t)c->max_pairs + k.max_tokens;
#define TRY(x)                                                          \
  do {                                                                  \
    if (e == hipSuccess) e = (x);                                       \
  } while (0)
  TRY(dalloc(&c->slot_of, ids));
  TRY(dalloc(&c->id_of, k.n_slots));
  TRY(dalloc(&c->stamp, k.n_slots));
  TRY(dalloc(&c->dstats, 8));
  TRY(dalloc(&c->logits_ws, (size_t)k.max_tokens * k.n_experts));
  TRY(dalloc(&c->offsets_ws, k.n_experts + 1));
  TRY(dalloc(&c->perm_ws, c->max_pairs));
  TRY(dalloc(&c->chunk_ws, (size_t)c->n_chunks_max * k.n_experts));
  TRY(dalloc(&c->work, c->max_work));
  TRY(dalloc(&c->work8, c->max_work8));
  TRY(dalloc(&c->n_work, 4));
  // activation records carry one extra all-zero row (for MFMA columns without a token)
  const size_t xrec_n = (size_t)(k.max_tokens + 1) * moe::xrec_halves(gsb);
  const size_t hrec_n = (size_t)(hrows + 1) * moe::xrec_halves(dsb);
  TRY(dalloc(&c->xrec, xrec_n));
  TRY(dalloc(&c->hrec, hrec_n));
  // prefill h record: hi and lo halves, rows of whole superblocks (the x
  // record shares xrec)
  TRY(dalloc(&c->h16, (size_t)hrows * dsb * moe::kSbCols * 2));
  TRY(dalloc(&c->slot_ws, c->max_pairs));
  // decode-size router: about 256 workgroups in all, at least one 16-column
  // chunk per wave (8 waves per workgroup)
  c->route_ks = 256 / ((k.n_experts + 15) / 16);
  if (c->route_ks < 1) c->route_ks = 1;
  while (c->route_ks > 1 && k.d_model / 16 < c->route_ks * 8) c->route_ks /= 2;
  // the MFMA router (and its partials) serves up to 64 tokens
  c->route_small_t = k.max_tokens < 64 ? k.max_tokens : 64;
  TRY(dalloc(&c->route_part, (size_t)c->route_ks * c->route_small_t * k.n_experts));

  TRY(dalloc(&c->dmiss, 3 + 2 * (size_t)c->max_pairs + 2 * (size_t)k.n_experts));
  if (e == hipSuccess)
    e = hipHostMalloc((void **)&c->hmiss, (3 + 2 * (size_t)c->max_pairs + 2 * (size_t)k.n_experts) * sizeof(int32_t),
                      hipHostMallocDefault);
  TRY(hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking));
  TRY(hipEventCreateWithFlags(&c->ev_main, hipEventDisableTiming));
  TRY(hipEventCreateWithFlags(&c->ev_copy, hipEventDisableTiming));
  if (e == hipSuccess && k.host_store) {
    // the zero-copy miss fill needs the store mapped into the device address
    // space (pinned memory from hipHostMalloc is); otherwise only the copying
    // path is available
    void *dp = nullptr;
    if (hipHostGetDevicePointer(&dp, const_cast<void *>(k.host_store), 0) == hipSuccess && dp)
      c->host_dev = static_cast<const uint8_t *>(dp);
    (void)hipGetLastError();
  }
  // empty cache: every identity unmapped, every slot free
  TRY(hipMemset(c->slot_of, 0xff, ids * sizeof(int32_t)));
  TRY(hipMemset(c->id_of, 0xff, (size_t)k.n_slots * sizeof(int32_t)));
  TRY(hipMemset(c->stamp, 0, (size_t)k.n_slots * sizeof(uint32_t)));
  TRY(hipMemset(c->dstats, 0, 8 * sizeof(int64_t)));
  TRY(hipMemset(c->n_work, 0, 4 * sizeof(int32_t)));
  // record positions past a matrix's columns are never written: they stay zero
  TRY(hipMemset(c->xrec, 0, xrec_n * sizeof(uint16_t)));
  TRY(hipMemset(c->hrec, 0, hrec_n * sizeof(uint16_t)));
  TRY(hipMemset(c->h16, 0, (size_t)hrows * dsb * moe::kSbCols * 2 * sizeof(uint16_t)));  // pad slots stay zero
  TRY(hipDeviceSynchronize());
#undef TRY
  if (e != hipSuccess) {
    moe_status st = (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation) ? MOE_ERR_OOM : MOE_ERR_HIP;
    free_ctx(c);
    return moe_fail(st, std::string("moe_create: ") + hipGetErrorString(e));
  }
  *out = c;
  return MOE_OK;
}

extern "C" moe_status moe_destroy(moe_ctx *c) {
  MOE_CHECK(c, MOE_ERR_INVALID, "moe_destroy: null ctx");
  (void)hipStreamSynchronize(c->side);
  free_ctx(c);
  return MOE_OK;
}

static hipStream_t as_stream(void *s) { return (hipStream_t)s; }

extern "C" moe_status moe_route(moe_ctx *c, int32_t layer, const float *x, int32_t T, const float *w_router,
                                const float *bias, float *logits, int32_t *idx, float *w, void *stream) {
  MOE_CHECK(c, MOE_ERR_INVALID, "moe_route: null ctx");
  MOE_CHECK(layer >= 0 && layer < c->cfg.n_layers, MOE_ERR_INVALID, "moe_route: layer out of range");
  MOE_CHECK(T >= 1 && T <= c->cfg.max_tokens, MOE_ERR_INVALID, "moe_route: T must be 1..max_tokens");
  MOE_CHECK(x && w_router && idx && w, MOE_ERR_INVALID, "moe_route: null x, w_router, idx or w");
  MOE_CHECK(aligned(x, 16) && aligned(w_router, 16), MOE_ERR_ALIGN, "moe_route: x and w_router must be 16-byte aligned");
  hipError_t e = moe::launch_router(c, x, T, w_router, bias, logits ? logits : c->logits_ws, idx, w, as_stream(stream));
  if (e != hipSuccess) return moe_fail(MOE_ERR_HIP, std::string("moe_route: ") + hipGetErrorString(e));
  return MOE_OK;
}

extern "C" moe_status moe_cache_resolve(moe_ctx *c, int32_t layer, const int32_t *idx, int32_t T,
                                        int32_t *slot_of_pair, moe_resolve_info *info, void *stream) {
  MOE_CHECK(c, MOE_ERR_INVALID, "moe_cache_resolve: null ctx");
  MOE_CHECK(layer >= 0 && layer < c->cfg.n_layers, MOE_ERR_INVALID, "moe_cache_resolve: layer out of range");
  MOE_CHECK(T >= 1 && T <= c->cfg.max_tokens, MOE_ERR_INVALID, "moe_cache_resolve: T must be 1..max_tokens");
  MOE_CHECK(idx, MOE_ERR_INVALID, "moe_cache_resolve: null idx");
  MOE_CHECK(c->resident || slot_of_pair, MOE_ERR_INVALID, "moe_cache_resolve: a capped cache needs slot_of_pair");
  hipStream_t s = as_stream(stream);
  hipError_t e = moe::launch_resolve(c, layer, idx, T, slot_of_pair, false, s);
  if (e != hipSuccess) return moe_fail(MOE_ERR_HIP, std::string("moe_cache_resolve: ") + hipGetErrorString(e));
  if (c->resident) {
    if (info) {
      // counts of this call need the unique set: read it back (synchronises)
      MOE_HIP(hipMemcpyAsync(c->hmiss, c->dmiss, 3 * sizeof(int32_t), hipMemcpyDeviceToHost, s));
      MOE_HIP(hipStreamSynchronize(s));
      info->lookups = c->hmiss[0];
      info->hits = c->hmiss[0];
      info->misses = 0;
      info->bytes_h2d = 0;
      info->resolve_calls = 1;
      info->failed_calls = 0;
    }
    return MOE_OK;
  }
  // capped: wait for the resolve kernel, then fetch the miss list
  const int maxm = c->max_pairs < c->cfg.n_experts ? c->max_pairs : c->cfg.n_experts;
  MOE_HIP(hipMemcpyAsync(c->hmiss, c->dmiss, (3 + 2 * (size_t)maxm) * sizeof(int32_t), hipMemcpyDeviceToHost, s));
  MOE_HIP(hipStreamSynchronize(s));
  const int nuniq = c->hmiss[0], nmiss = c->hmiss[1], err = c->hmiss[2];
  if (err == 1) {
    return moe_fail(MOE_ERR_CAPACITY, "moe_cache_resolve: the call touches " + std::to_string(nuniq) +
                                          " identities but the pool has " + std::to_string(c->cfg.n_slots) + " slots");
  }
  if (err) return moe_fail(MOE_ERR_CAPACITY, "moe_cache_resolve: no eligible slot; call moe_cache_reset");
  const size_t stride = c->L.stride;
  if (nmiss > 0) {
    // the work already on `s` (which may read evicted slots) has completed:
    // the synchronisation above covered it.  Copies go on the side stream.
    MOE_HIP(hipEventRecord(c->ev_main, s));
    MOE_HIP(hipStreamWaitEvent(c->side, c->ev_main, 0));
    int i = 0;
    while (i < nmiss) {
      // merge runs of consecutive (id, slot)
      int id0 = c->hmiss[3 + 2 * i], sl0 = c->hmiss[4 + 2 * i], n = 1;
      while (i + n < nmiss && c->hmiss[3 + 2 * (i + n)] == id0 + n && c->hmiss[4 + 2 * (i + n)] == sl0 + n) ++n;
      MOE_HIP(hipMemcpyAsync((char *)c->cfg.slot_pool + (size_t)sl0 * stride,
                             (const char *)c->cfg.host_store + (size_t)id0 * stride, (size_t)n * stride,
                             hipMemcpyHostToDevice, c->side));
      i += n;
    }
    MOE_HIP(hipEventRecord(c->ev_copy, c->side));
    MOE_HIP(hipStreamWaitEvent(s, c->ev_copy, 0));
  }
  if (info) {
    info->lookups = nuniq;
    info->hits = nuniq - nmiss;
    info->misses = nmiss;
    info->bytes_h2d = (uint64_t)nmiss * stride;
    info->resolve_calls = 1;
    info->failed_calls = 0;
  }
  return MOE_OK;
}

extern "C" moe_status moe_cache_resolve_async(moe_ctx *c, int32_t layer, const int32_t *idx, int32_t T,
                                              int32_t *slot_of_pair, void *stream) {
  MOE_CHECK(c, MOE_ERR_INVALID, "moe_cache_resolve_async: null ctx");
  MOE_CHECK(layer >= 0 && layer < c->cfg.n_layers, MOE_ERR_INVALID, "moe_cache_resolve_async: layer out of range");
  MOE_CHECK(T >= 1 && T <= c->cfg.max_tokens, MOE_ERR_INVALID, "moe_cache_resolve_async: T must be 1..max_tokens");
  MOE_CHECK(idx, MOE_ERR_INVALID, "moe_cache_resolve_async: null idx");
  MOE_CHECK(c->resident || slot_of_pair, MOE_ERR_INVALID, "moe_cache_resolve_async: a capped cache needs slot_of_pair");
  MOE_CHECK(c->resident || c->host_dev, MOE_ERR_INVALID,
            "moe_cache_resolve_async: host_store is not mapped into the device address space (allocate it with "
            "hipHostMalloc)");
  hipError_t e = moe::launch_resolve(c, layer, idx, T, slot_of_pair, true, as_stream(stream));
  if (e != hipSuccess) return moe_fail(MOE_ERR_HIP, std::string("moe_cache_resolve_async: ") + hipGetErrorString(e));
  return MOE_OK;
}

static moe_status check_ffn_args(moe_ctx *c, int32_t layer, const float *x, int32_t T, const int32_t *idx,
                                 const int32_t *slot_of_pair, float *y_pairs, float *y_shared) {
  MOE_CHECK(c, MOE_ERR_INVALID, "moe_expert_ffn: null ctx");
  MOE_CHECK(layer >= 0 && layer < c->cfg.n_layers, MOE_ERR_INVALID, "moe_expert_ffn: layer out of range");
  MOE_CHECK(T >= 1 && T <= c->cfg.max_tokens, MOE_ERR_INVALID, "moe_expert_ffn: T must be 1..max_tokens");
  MOE_CHECK(x && idx && y_pairs && y_shared, MOE_ERR_INVALID, "moe_expert_ffn: null x, idx, y_pairs or y_shared");
  MOE_CHECK(c->resident || slot_of_pair, MOE_ERR_INVALID, "moe_expert_ffn: a capped cache needs slot_of_pair");
  MOE_CHECK(aligned(x, 16) && aligned(y_pairs, 16) && aligned(y_shared, 16), MOE_ERR_ALIGN,
            "moe_expert_ffn: x, y_pairs and y_shared must be 16-byte aligned");
  return MOE_OK;
}

extern "C" moe_status moe_expert_ffn(moe_ctx *c, int32_t layer, const float *x, int32_t T, const int32_t *idx,
                                     const int32_t *slot_of_pair, float *y_pairs, float *y_shared, int32_t path,
                                     void *stream) {
  moe_status st = check_ffn_args(c, layer, x, T, idx, slot_of_pair, y_pairs, y_shared);
  if (st != MOE_OK) return st;
  MOE_CHECK(path == MOE_PATH_AUTO || path == MOE_PATH_DECODE || path == MOE_PATH_PREFILL, MOE_ERR_INVALID,
            "moe_expert_ffn: unknown path");
  // the prefill kernels address the x and h records with 32-bit byte offsets
  const uint64_t xrec_bytes = (uint64_t)T * 5 * c->L.gate.nsb * 128;
  const uint64_t hrec_bytes = ((uint64_t)T * c->cfg.top_k + T) * 5 * c->L.down.nsb * 128;
  const bool prefill_ok = c->cfg.d_model % 64 == 0 && c->cfg.d_ff % 64 == 0 && xrec_bytes <= UINT32_MAX &&
                          hrec_bytes <= UINT32_MAX;
  const bool decode_ok = c->L.gate.nsb <= moe::kDecodeMaxNsb && c->L.down.nsb <= moe::kDecodeMaxNsb;
  if (path == MOE_PATH_AUTO) path = ((T <= 64 && decode_ok) || !prefill_ok) ? MOE_PATH_DECODE : MOE_PATH_PREFILL;
  MOE_CHECK(path != MOE_PATH_PREFILL || prefill_ok, MOE_ERR_INVALID,
            "moe_expert_ffn: the prefill path needs d_model and d_ff to be multiples of 64 and the call's x and h "
            "records under 4 GiB");
  MOE_CHECK(path != MOE_PATH_DECODE || decode_ok, MOE_ERR_INVALID,
            "moe_expert_ffn: the decode path takes d_model and d_ff up to 2048 (13 superblocks of 160 columns)");
  hipStream_t s = as_stream(stream);
  hipError_t e = path == MOE_PATH_DECODE
                     ? moe::launch_ffn_decode(c, layer, x, T, idx, slot_of_pair, y_pairs, y_shared, s)
                     : moe::launch_ffn_prefill(c, layer, x, T, idx, slot_of_pair, y_pairs, y_shared, s);
  if (e != hipSuccess) return moe_fail(MOE_ERR_HIP, std::string("moe_expert_ffn: ") + hipGetErrorString(e));
  return MOE_OK;
}

extern "C" moe_status moe_combine(moe_ctx *c, const float *y_pairs, const float *w, const float *y_shared,
                                  int32_t T, float *out, void *stream) {
  MOE_CHECK(c, MOE_ERR_INVALID, "moe_combine: null ctx");
  MOE_CHECK(T >= 1 && T <= c->cfg.max_tokens, MOE_ERR_INVALID, "moe_combine: T must be 1..max_tokens");
  MOE_CHECK(y_pairs && w && y_shared && out, MOE_ERR_INVALID, "moe_combine: null pointer");
  MOE_CHECK(aligned(y_pairs, 16) && aligned(y_shared, 16) && aligned(out, 16), MOE_ERR_ALIGN,
            "moe_combine: y_pairs, y_shared and out must be 16-byte aligned");
  hipError_t e = moe::launch_combine(y_pairs, w, y_shared, T, c->cfg.top_k, c->cfg.d_model, out, as_stream(stream));
  if (e != hipSuccess) return moe_fail(MOE_ERR_HIP, std::string("moe_combine: ") + hipGetErrorString(e));
  return MOE_OK;
}

extern "C" moe_status moe_bucket(moe_ctx *c, const int32_t *idx, int32_t T, int32_t *offsets, int32_t *perm,
                                 void *stream) {
  MOE_CHECK(c, MOE_ERR_INVALID, "moe_bucket: null ctx");
  MOE_CHECK(T >= 1 && T <= c->cfg.max_tokens, MOE_ERR_INVALID, "moe_bucket: T must be 1..max_tokens");
  MOE_CHECK(idx && offsets && perm, MOE_ERR_INVALID, "moe_bucket: null pointer");
  hipError_t e = moe::launch_bucket(c, idx, T, offsets, perm, false, as_stream(stream));
  if (e != hipSuccess) return moe_fail(MOE_ERR_HIP, std::string("moe_bucket: ") + hipGetErrorString(e));
  return MOE_OK;
}

extern "C" moe_status moe_cache_snapshot(moe_ctx *c, int32_t *slot_of, int32_t *id_of, uint32_t *stamp) {
  MOE_CHECK(c, MOE_ERR_INVALID, "moe_cache_snapshot: null ctx");
  MOE_HIP(hipDeviceSynchronize());
  const int64_t ids = (int64_t)c->cfg.n_layers * c->cfg.n_experts;
  if (c->resident) {
    for (int64_t i = 0; slot_of && i < ids; ++i) slot_of[i] = (int32_t)i;
    for (int64_t i = 0; id_of && i < c->cfg.n_slots; ++i) id_of[i] = (int32_t)i;
    if (stamp) memset(stamp, 0, (size_t)c->cfg.n_slots * sizeof(uint32_t));
    return MOE_OK;
  }
  if (slot_of) MOE_HIP(hipMemcpy(slot_of, c->slot_of, ids * sizeof(int32_t), hipMemcpyDeviceToHost));
  if (id_of) MOE_HIP(hipMemcpy(id_of, c->id_of, (size_t)c->cfg.n_slots * sizeof(int32_t), hipMemcpyDeviceToHost));
  if (stamp) MOE_HIP(hipMemcpy(stamp, c->stamp, (size_t)c->cfg.n_slots * sizeof(uint32_t), hipMemcpyDeviceToHost));
  return MOE_OK;
}

extern "C" moe_status moe_cache_reset(moe_ctx *c) {
  MOE_CHECK(c, MOE_ERR_INVALID, "moe_cache_reset: null ctx");
  MOE_HIP(hipDeviceSynchronize());
  const int64_t ids = (int64_t)c->cfg.n_layers * c->cfg.n_experts;
  MOE_HIP(hipMemset(c->slot_of, 0xff, ids * sizeof(int32_t)));
  MOE_HIP(hipMemset(c->id_of, 0xff, (size_t)c->cfg.n_slots * sizeof(int32_t)));
  MOE_HIP(hipMemset(c->stamp, 0, (size_t)c->cfg.n_slots * sizeof(uint32_t)));
  MOE_HIP(hipMemset(c->dstats, 0, 8 * sizeof(int64_t)));
  MOE_HIP(hipDeviceSynchronize());
  return MOE_OK;
}

extern "C" moe_status moe_get_stats(moe_ctx *c, moe_resolve_info *cum) {
  MOE_CHECK(c && cum, MOE_ERR_INVALID, "moe_get_stats: null pointer");
  MOE_HIP(hipDeviceSynchronize());
  int64_t st[8];
  MOE_HIP(hipMemcpy(st, c->dstats, sizeof(st), hipMemcpyDeviceToHost));
  cum->lookups = st[0];
  cum->hits = st[1];
  cum->misses = st[2];
  cum->resolve_calls = st[3];
  cum->bytes_h2d = (uint64_t)st[2] * c->L.stride;  // every miss brings in one blob
  cum->failed_calls = st[4];
  return MOE_OK;
}

extern "C" moe_status moe_chain_norm(moe_ctx *c, const float *out, int32_t T, float *x_next, void *stream) {
  MOE_CHECK(c, MOE_ERR_INVALID, "moe_chain_norm: null ctx");
  MOE_CHECK(T >= 1 && T <= c->cfg.max_tokens, MOE_ERR_INVALID, "moe_chain_norm: T must be 1..max_tokens");
  MOE_CHECK(out && x_next, MOE_ERR_INVALID, "moe_chain_norm: null pointer");
  MOE_CHECK(aligned(out, 16) && aligned(x_next, 16), MOE_ERR_ALIGN, "moe_chain_norm: pointers must be 16-byte aligned");
  hipError_t e = moe::launch_chain_norm(out, T, c->cfg.d_model, x_next, as_stream(stream));
  if (e != hipSuccess) return moe_fail(MOE_ERR_HIP, std::string("moe_chain_norm: ") + hipGetErrorString(e));
  return MOE_OK;
}

extern "C" moe_status moe_combine_norm(moe_ctx *c, const float *y_pairs, const float *w, const float *y_shared,
                                       int32_t T, float *out, float *x_next, void *stream) {
  MOE_CHECK(c, MOE_ERR_INVALID, "moe_combine_norm: null ctx");
  MOE_CHECK(T >= 1 && T <= c->cfg.max_tokens, MOE_ERR_INVALID, "moe_combine_norm: T must be 1..max_tokens");
  MOE_CHECK(y_pairs && w && y_shared && out && x_next, MOE_ERR_INVALID, "moe_combine_norm: null pointer");
  MOE_CHECK(aligned(y_pairs, 16) && aligned(y_shared, 16) && aligned(out, 16) && aligned(x_next, 16), MOE_ERR_ALIGN,
            "moe_combine_norm: y_pairs, y_shared, out and x_next must be 16-byte aligned");
  MOE_CHECK(out != x_next, MOE_ERR_INVALID, "moe_combine_norm: out and x_next must differ");
  hipError_t e = moe::launch_combine_norm(y_pairs, w, y_shared, T, c->cfg.top_k, c->cfg.d_model, out, x_next,
                                          as_stream(stream));
  if (e != hipSuccess) return moe_fail(MOE_ERR_HIP, std::string("moe_combine_norm: ") + hipGetErrorString(e));
  return MOE_OK;
}

extern "C" moe_status moe_decode_layer(moe_ctx *c, int32_t layer, const float *x, int32_t T, const float *w_router,
                                       const float *bias, float *logits, int32_t *idx, float *w, float *y_pairs,
                                       float *y_shared, float *out, float *x_next, void *stream) {
  MOE_CHECK(c, MOE_ERR_INVALID, "moe_decode_layer: null ctx");
  MOE_CHECK(c->resident || c->host_dev, MOE_ERR_INVALID,
            "moe_decode_layer: a capped cache needs host_store mapped into the device address space (allocate it "
            "with hipHostMalloc); otherwise use the separate calls");
  MOE_CHECK(layer >= 0 && layer < c->cfg.n_layers, MOE_ERR_INVALID, "moe_decode_layer: layer out of range");
  MOE_CHECK(T >= 1 && T <= c->cfg.max_tokens, MOE_ERR_INVALID, "moe_decode_layer: T must be 1..max_tokens");
  MOE_CHECK(x && w_router && idx && w && y_pairs && y_shared && out, MOE_ERR_INVALID,
            "moe_decode_layer: null x, w_router, idx, w, y_pairs, y_shared or out");
  MOE_CHECK(aligned(x, 16) && aligned(w_router, 16) && aligned(y_pairs, 16) && aligned(y_shared, 16) &&
                aligned(out, 16) && (!x_next || aligned(x_next, 16)),
            MOE_ERR_ALIGN, "moe_decode_layer: x, w_router, y_pairs, y_shared, out and x_next must be 16-byte aligned");
  MOE_CHECK(out != x_next && x != x_next, MOE_ERR_INVALID, "moe_decode_layer: x_next must differ from x and out");
  MOE_CHECK(c->L.gate.nsb <= moe::kDecodeMaxNsb && c->L.down.nsb <= moe::kDecodeMaxNsb, MOE_ERR_INVALID,
            "moe_decode_layer: the decode path takes d_model and d_ff up to 2048");
  MOE_CHECK(T * c->cfg.top_k <= 1024 && c->cfg.n_experts <= 1024, MOE_ERR_INVALID,
            "moe_decode_layer: needs T * top_k <= 1024");
  hipStream_t s = as_stream(stream);
  const int xh = moe::xrec_halves(c->L.gate.nsb);
  float *lg = logits ? logits : c->logits_ws;
  hipError_t e = hipSuccess;
  if (c->resident) {
    // a single token: the top-k joins the bucketing launch (five launches;
    // at two tokens the two top-ks one after another in one workgroup cost
    // more than the launch they save)
    if (T == 1 && T <= c->route_small_t) {
      e = moe::launch_router_partials(c, x, T, w_router, s);
      if (e == hipSuccess)
        e = moe::launch_route_bucket_lookup(c, T, bias, lg, idx, w, moe::kEntryTokens, x, c->xrec, xh, s);
    } else {
      e = moe::launch_router(c, x, T, w_router, bias, lg, idx, w, s);
      if (e == hipSuccess) e = moe::launch_bucket_lookup(c, idx, T, moe::kEntryTokens, x, c->xrec, xh, s);
    }
    if (e == hipSuccess) e = moe::launch_ffn_decode_kernels(c, layer, T, nullptr, y_pairs, y_shared, s);
  } else {
    // capped: the router and the resolve (for a single token the top-k and
    // the resolve share one workgroup), then one launch for the
    // bucketing, the x record and the zero-copy fill of the resolve's misses
    // (no fill launch of its own), then the FFN on the filled slots
    if (T == 1 && T <= c->route_small_t) {
      e = moe::launch_router_partials(c, x, T, w_router, s);
      if (e == hipSuccess) e = moe::launch_route_resolve(c, layer, T, bias, lg, idx, w, c->slot_ws, s);
    } else {
      e = moe::launch_router(c, x, T, w_router, bias, lg, idx, w, s);
      if (e == hipSuccess) e = moe::launch_resolve(c, layer, idx, T, c->slot_ws, true, s, false);
    }
    if (e == hipSuccess) e = moe::launch_bucket_fill(c, idx, T, moe::kEntryTokens, x, c->xrec, xh, s);
    if (e == hipSuccess) e = moe::launch_ffn_decode_kernels(c, layer, T, c->slot_ws, y_pairs, y_shared, s);
  }
  if (e == hipSuccess)
    e = x_next ? moe::launch_combine_norm(y_pairs, w, y_shared, T, c->cfg.top_k, c->cfg.d_model, out, x_next, s)
               : moe::launch_combine(y_pairs, w, y_shared, T, c->cfg.top_k, c->cfg.d_model, out, s);
  if (e != hipSuccess) return moe_fail(MOE_ERR_HIP, std::string("moe_decode_layer: ") + hipGetErrorString(e));
  return MOE_OK;
}
