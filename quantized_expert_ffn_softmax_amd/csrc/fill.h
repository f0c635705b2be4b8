// Zero-copy miss fill, shared by the fill kernel and the bucketing launch of
// a capped decode layer: one workgroup copies one chunk of one missed blob
// from the pinned host store (mapped into the device address space; the
// reads cross the host link) into the slot the resolve kernel gave it.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

struct FillArgs {
  const int32_t *dmiss;    // the resolve's miss list: [1] misses, then (identity, slot) pairs from [3]
  const uint8_t *host;     // host store as mapped into the device address space
  uint8_t *pool;           // slot pool
  uint64_t stride;         // blob stride (a multiple of 256)
  int64_t n_ids;           // identities in the host store
  int n_slots;
  int chunks;              // workgroups per missed blob
};

// chunk `chunk` of miss i (if that miss exists) by the workgroup's nt
// threads: 16-byte loads, four in flight per thread before their stores
__device__ inline void fill_chunk(const FillArgs &F, int i, int chunk, int tid, int nt) {
  if (i >= F.dmiss[1]) return;
  const int64_t id = F.dmiss[3 + 2 * i];
  const int slot = F.dmiss[4 + 2 * i];
  if (id < 0 || id >= F.n_ids || slot < 0 || slot >= F.n_slots) return;  // never copy out of range
  const uint64_t n16 = F.stride / 16, per = (n16 + F.chunks - 1) / F.chunks;
  const uint64_t b0 = (uint64_t)chunk * per, b1 = b0 + per < n16 ? b0 + per : n16;
  const uint4 *src = reinterpret_cast<const uint4 *>(F.host + (uint64_t)id * F.stride);
  uint4 *dst = reinterpret_cast<uint4 *>(F.pool + (uint64_t)slot * F.stride);
  uint64_t q = b0 + tid;
  for (; q + 3 * (uint64_t)nt < b1; q += 4 * (uint64_t)nt) {
    const uint4 a0 = src[q], a1 = src[q + nt], a2 = src[q + 2 * nt], a3 = src[q + 3 * nt];
    dst[q] = a0;
    dst[q + nt] = a1;
    dst[q + 2 * nt] = a2;
    dst[q + 3 * nt] = a3;
  }
  for (; q < b1; q += nt) dst[q] = src[q];
}

}  // namespace moe
