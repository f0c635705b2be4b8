// KV tier: int8 KV cells, the first cells of each layer resident in HBM, the
// rest in pinned host memory, read on demand (zero-copy) or from a staging
// copy that a prefetch brings in by DMA.
//
// The pages' engine keeps KV as int8 at 1,056 bytes per cell, locks only the
// first 32,768 of a layer's 131,072 cells in VRAM and streams the rest from
// 1.55 GiB of pinned RAM, with an optional prefetch ("单卡5090跑125B 大模型
// ...", section 2.2; "一张 RTX 4090 跑千亿模型，Strata 实测 155 tok/s",
// section 四个发现).  The cell layout is not printed; the reading here: V
// values (1,024: one token's K and V of one layer) as int8 codes in groups of
// 64, then one fp16 scale per group; s = fp16(absmax / 127),
// q = clamp(rint(v / s), -127, 127), a value reads back as q * s.
//
// One wave per cell, in chunks of 1,024 values: at step q (0..3) of a chunk
// lane l holds values 256 q + 4 l .. 256 q + 4 l + 3, so every load and store
// instruction of the wave covers one contiguous span (1 KB of fp32, 256 B of
// codes); a group of 64 values is 16 lanes of one step (absmax by four
// shuffles).
#include <mutex>

#include "moe_internal.h"

struct moe_kv {
  moe_kv_config cfg;
  uint32_t cb;              // bytes per cell
  uint8_t *resident;        // device [layers][resident][cb]
  uint8_t *host;            // host [layers][total - resident][cb]
  uint8_t *host_dev;        // the same, mapped into the device address space
  uint8_t *stage;           // device [2][stage_cells][cb]
  int stage_layer[2], stage_first[2], stage_n[2];  // what each staging slot holds (-1: nothing)
  int next_slot;
  moe_kv_stats st;
};

namespace {

constexpr int kKvGroup = 64;
constexpr int kKvWaves = 4;  // cells per workgroup

struct KvPlace {
  uint8_t *resident, *host_dev, *stage;
  uint32_t cb;
  int layer, R, host_cells, stage_cells;
  // staged ranges of this layer (first, n) per slot; n = 0 when the slot holds another layer
  int s_first[2], s_n[2];
};

__device__ inline uint8_t *resident_cell(const KvPlace &K, int c) {
  return K.resident + ((size_t)K.layer * K.R + c) * K.cb;
}
__device__ inline uint8_t *host_cell(const KvPlace &K, int c) {
  return K.host_dev + ((size_t)K.layer * K.host_cells + (c - K.R)) * K.cb;
}
__device__ inline uint8_t *staged_cell(const KvPlace &K, int c) {
#pragma unroll
  for (int s = 0; s < 2; ++s)
    if (c >= K.s_first[s] && c < K.s_first[s] + K.s_n[s])
      return K.stage + ((size_t)s * K.stage_cells + (c - K.s_first[s])) * K.cb;
  return nullptr;
}

typedef float f4 __attribute__((ext_vector_type(4)));

// quantise cells [first, first + n) from vals [n][V] fp32
__global__ void __launch_bounds__(64 * kKvWaves) kv_write_kernel(KvPlace K, int first, int n, int V,
                                                                 const float *__restrict__ vals) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * kKvWaves + (threadIdx.x >> 6);
  if (i >= n) return;  // whole waves
  const int c = first + i;
  uint8_t *dst = c < K.R ? resident_cell(K, c) : host_cell(K, c);
  uint8_t *dst2 = c < K.R ? nullptr : staged_cell(K, c);  // a staged copy is kept equal
  for (int j0 = 0; j0 < V; j0 += 1024) {
    f4 v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = *reinterpret_cast<const f4 *>(vals + (size_t)i * V + j0 + 256 * q + 4 * lane);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float m = fmaxf(fmaxf(fabsf(v[q].x), fabsf(v[q].y)), fmaxf(fabsf(v[q].z), fabsf(v[q].w)));
      m = fmaxf(m, __shfl_xor(m, 1, 64));
      m = fmaxf(m, __shfl_xor(m, 2, 64));
      m = fmaxf(m, __shfl_xor(m, 4, 64));
      m = fmaxf(m, __shfl_xor(m, 8, 64));  // the group's absmax (lanes 16 h .. 16 h + 15)
      const _Float16 s16 = (_Float16)(m / 127.0f);
      const float s = (float)s16;
      const float e[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
      uint32_t packed = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float r = s == 0.f ? 0.f : fminf(fmaxf(rintf(e[t] / s), -127.f), 127.f);
        packed |= (uint32_t)(uint8_t)(int8_t)(int)r << (8 * t);
      }
      const int off = j0 + 256 * q + 4 * lane;
      *reinterpret_cast<uint32_t *>(dst + off) = packed;
      if (dst2) *reinterpret_cast<uint32_t *>(dst2 + off) = packed;
      if ((lane & 15) == 0) {
        const int g = off / kKvGroup;
        *reinterpret_cast<_Float16 *>(dst + V + 2 * g) = s16;
        if (dst2) *reinterpret_cast<_Float16 *>(dst2 + V + 2 * g) = s16;
      }
    }
  }
}

// read cells [first, first + n) back into out [n][V] fp32: resident cells
// from HBM, the others from a staging copy when one holds them, else from
// host memory
__global__ void __launch_bounds__(64 * kKvWaves) kv_read_kernel(KvPlace K, int first, int n, int V,
                                                                float *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * kKvWaves + (threadIdx.x >> 6);
  if (i >= n) return;
  const int c = first + i;
  const uint8_t *src = c < K.R ? resident_cell(K, c) : nullptr;
  if (!src) src = staged_cell(K, c);
  if (!src) src = host_cell(K, c);
  for (int j0 = 0; j0 < V; j0 += 1024) {
    uint32_t w[4];
    float s[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int off = j0 + 256 * q + 4 * lane;
      w[q] = *reinterpret_cast<const uint32_t *>(src + off);
      s[q] = (float)*reinterpret_cast<const _Float16 *>(src + V + 2 * (off / kKvGroup));
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<f4 *>(out + (size_t)i * V + j0 + 256 * q + 4 * lane) =
          (f4){(float)(int8_t)(w[q] & 0xff) * s[q], (float)(int8_t)((w[q] >> 8) & 0xff) * s[q],
               (float)(int8_t)((w[q] >> 16) & 0xff) * s[q], (float)(int8_t)(w[q] >> 24) * s[q]};
  }
}

KvPlace place_of(const moe_kv *kv, int layer) {
  KvPlace K;
  K.resident = kv->resident;
  K.host_dev = kv->host_dev;
  K.stage = kv->stage;
  K.cb = kv->cb;
  K.layer = layer;
  K.R = kv->cfg.cells_resident;
  K.host_cells = kv->cfg.cells_total - kv->cfg.cells_resident;
  K.stage_cells = kv->cfg.stage_cells;
  for (int s = 0; s < 2; ++s) {
    const bool mine = kv->stage_layer[s] == layer;
    K.s_first[s] = mine ? kv->stage_first[s] : 0;
    K.s_n[s] = mine ? kv->stage_n[s] : 0;
  }
  return K;
}

int64_t overlap(int64_t a0, int64_t a1, int64_t b0, int64_t b1) {
  const int64_t lo = a0 > b0 ? a0 : b0, hi = a1 < b1 ? a1 : b1;
  return hi > lo ? hi - lo : 0;
}

// cells of [c0, c1) of `layer` that a read takes from host memory: past the
// resident window and in neither staged range
int64_t host_cells_of(const moe_kv *kv, int layer, int64_t c0, int64_t c1) {
  const int64_t a0 = c0 > kv->cfg.cells_resident ? c0 : kv->cfg.cells_resident;
  if (c1 <= a0) return 0;
  int64_t r[2][2];
  for (int s = 0; s < 2; ++s) {
    const bool mine = kv->stage_layer[s] == layer;
    r[s][0] = mine ? kv->stage_first[s] : 0;
    r[s][1] = mine ? kv->stage_first[s] + kv->stage_n[s] : 0;
  }
  const int64_t both = overlap(a0, c1, r[0][0] > r[1][0] ? r[0][0] : r[1][0], r[0][1] < r[1][1] ? r[0][1] : r[1][1]);
  return (c1 - a0) - overlap(a0, c1, r[0][0], r[0][1]) - overlap(a0, c1, r[1][0], r[1][1]) + both;
}

}  // namespace

extern "C" size_t moe_kv_cell_bytes(int32_t values) {
  if (values < kKvGroup || values > 4096 || values % 1024) return 0;
  return (size_t)values + 2 * (size_t)(values / kKvGroup);
}

extern "C" moe_status moe_kv_create(const moe_kv_config *cfg, moe_kv **out) {
  MOE_CHECK(cfg && out, MOE_ERR_INVALID, "moe_kv_create: null cfg or out");
  *out = nullptr;
  const moe_kv_config &k = *cfg;
  MOE_CHECK(moe_kv_cell_bytes(k.values) > 0, MOE_ERR_INVALID,
            "moe_kv_create: values per cell must be 1,024, 2,048, 3,072 or 4,096");
  MOE_CHECK(k.n_layers >= 1 && k.cells_total >= 1 && k.cells_resident >= 0 && k.cells_resident <= k.cells_total,
            MOE_ERR_INVALID, "moe_kv_create: need n_layers >= 1 and 0 <= cells_resident <= cells_total");
  MOE_CHECK(k.block_cells >= 1 && k.stage_cells >= 1 && k.stage_cells <= k.cells_total, MOE_ERR_INVALID,
            "moe_kv_create: need block_cells >= 1 and 1 <= stage_cells <= cells_total");
  MOE_CHECK(k.cells_resident == 0 || k.resident, MOE_ERR_INVALID, "moe_kv_create: null resident buffer");
  MOE_CHECK(k.cells_resident == k.cells_total || k.host, MOE_ERR_INVALID, "moe_kv_create: null host buffer");
  MOE_CHECK((!k.resident || ((uintptr_t)k.resident % 16) == 0) && (!k.host || ((uintptr_t)k.host % 16) == 0),
            MOE_ERR_ALIGN, "moe_kv_create: resident and host buffers must be 16-byte aligned");
  moe_kv *kv = new moe_kv();
  kv->cfg = k;
  kv->cb = (uint32_t)moe_kv_cell_bytes(k.values);
  kv->resident = (uint8_t *)k.resident;
  kv->host = (uint8_t *)k.host;
  kv->host_dev = nullptr;
  if (k.host) {
    void *dp = nullptr;
    if (hipHostGetDevicePointer(&dp, k.host, 0) != hipSuccess || !dp) {
      (void)hipGetLastError();
      delete kv;
      return moe_fail(MOE_ERR_INVALID, "moe_kv_create: host buffer is not mapped pinned memory (use hipHostMalloc)");
    }
    kv->host_dev = (uint8_t *)dp;
  }
  for (int s = 0; s < 2; ++s) kv->stage_layer[s] = kv->stage_first[s] = -1, kv->stage_n[s] = 0;
  kv->next_slot = 0;
  kv->st = moe_kv_stats{};
  if (hipMalloc((void **)&kv->stage, 2 * (size_t)k.stage_cells * kv->cb) != hipSuccess) {
    (void)hipGetLastError();
    delete kv;
    return moe_fail(MOE_ERR_OOM, "moe_kv_create: could not allocate the staging buffer");
  }
  *out = kv;
  return MOE_OK;
}

extern "C" moe_status moe_kv_destroy(moe_kv *kv) {
  MOE_CHECK(kv, MOE_ERR_INVALID, "moe_kv_destroy: null kv");
  (void)hipDeviceSynchronize();
  (void)hipFree(kv->stage);
  delete kv;
  return MOE_OK;
}

static moe_status kv_range(const moe_kv *kv, int32_t layer, int32_t first, int32_t n, const char *fn) {
  MOE_CHECK(kv, MOE_ERR_INVALID, std::string(fn) + ": null kv");
  MOE_CHECK(layer >= 0 && layer < kv->cfg.n_layers, MOE_ERR_INVALID, std::string(fn) + ": layer out of range");
  MOE_CHECK(n >= 1 && first >= 0 && (int64_t)first + n <= kv->cfg.cells_total, MOE_ERR_INVALID,
            std::string(fn) + ": cells [first, first + n) must lie in [0, cells_total)");
  return MOE_OK;
}

extern "C" moe_status moe_kv_write(moe_kv *kv, int32_t layer, int32_t first, int32_t n, const float *vals,
                                   void *stream) {
  moe_status st = kv_range(kv, layer, first, n, "moe_kv_write");
  if (st != MOE_OK) return st;
  MOE_CHECK(vals && ((uintptr_t)vals % 16) == 0, MOE_ERR_INVALID, "moe_kv_write: vals null or not 16-byte aligned");
  hipLaunchKernelGGL(kv_write_kernel, dim3((n + kKvWaves - 1) / kKvWaves), dim3(64 * kKvWaves), 0,
                     (hipStream_t)stream, place_of(kv, layer), first, n, kv->cfg.values, vals);
  MOE_HIP(hipGetLastError());
  kv->st.cells_written += n;
  return MOE_OK;
}

extern "C" moe_status moe_kv_prefetch(moe_kv *kv, int32_t layer, int32_t first, int32_t n, void *stream) {
  moe_status st = kv_range(kv, layer, first, n, "moe_kv_prefetch");
  if (st != MOE_OK) return st;
  MOE_CHECK(n <= kv->cfg.stage_cells, MOE_ERR_INVALID, "moe_kv_prefetch: n exceeds stage_cells");
  const int R = kv->cfg.cells_resident;
  const int s = kv->next_slot;
  // the host cells of the range, one DMA copy (they are contiguous in host memory)
  const int h0 = first > R ? first : R, h1 = first + n;
  if (h1 > h0) {
    const size_t host_cells = (size_t)(kv->cfg.cells_total - R);
    MOE_HIP(hipMemcpyAsync(kv->stage + ((size_t)s * kv->cfg.stage_cells + (h0 - first)) * kv->cb,
                           kv->host + ((size_t)layer * host_cells + (h0 - R)) * kv->cb, (size_t)(h1 - h0) * kv->cb,
                           hipMemcpyHostToDevice, (hipStream_t)stream));
    kv->st.prefetch_bytes += (int64_t)(h1 - h0) * kv->cb;
  }
  kv->stage_layer[s] = layer;
  kv->stage_first[s] = first;
  kv->stage_n[s] = n;
  kv->next_slot = s ^ 1;
  return MOE_OK;
}

extern "C" moe_status moe_kv_read(moe_kv *kv, int32_t layer, int32_t first, int32_t n, float *out, void *stream) {
  moe_status st = kv_range(kv, layer, first, n, "moe_kv_read");
  if (st != MOE_OK) return st;
  MOE_CHECK(out && ((uintptr_t)out % 16) == 0, MOE_ERR_INVALID, "moe_kv_read: out null or not 16-byte aligned");
  hipLaunchKernelGGL(kv_read_kernel, dim3((n + kKvWaves - 1) / kKvWaves), dim3(64 * kKvWaves), 0,
                     (hipStream_t)stream, place_of(kv, layer), first, n, kv->cfg.values, out);
  MOE_HIP(hipGetLastError());
  // block-read accounting at enqueue time (everything it needs is host state)
  const int64_t B = kv->cfg.block_cells;
  for (int64_t c = first; c < (int64_t)first + n;) {
    const int64_t end = ((c / B) + 1) * B < (int64_t)first + n ? ((c / B) + 1) * B : (int64_t)first + n;
    const int64_t from_host = host_cells_of(kv, layer, c, end);
    kv->st.block_reads += 1;
    kv->st.vram_block_reads += from_host == 0;
    kv->st.host_bytes += from_host * kv->cb;
    c = end;
  }
  kv->st.cells_read += n;
  return MOE_OK;
}

extern "C" moe_status moe_kv_get_stats(moe_kv *kv, moe_kv_stats *out) {
  MOE_CHECK(kv && out, MOE_ERR_INVALID, "moe_kv_get_stats: null pointer");
  *out = kv->st;
  return MOE_OK;
}
