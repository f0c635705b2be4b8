// Host stand-in for the HIP runtime, so that the library's index-producing
// kernels (bucketing and work list, cache resolve and miss fill, the decode
// activation record) compile for the CPU under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Every out-of-bounds access of a work list,
// perm, record or slot-table index then stops a test on the CPU.  Test
// infrastructure only: the library itself is never built against this header.
//
// Execution model: a launch runs its workgroups one after another.  The
// threads of one workgroup are fibers (ucontext) on the calling thread; each
// runs until it reaches a barrier or a wave operation (shuffle, ballot, DPP
// row move, lane read), and a scheduler resumes the fibers of a rendezvous
// once all of its members have arrived.  __shared__ becomes `static`, which
// is per-workgroup storage because workgroups never overlap.  The scheduler
// visits the runnable fibers in an order shuffled per pass (seeded by
// HOSTK_SEED), so LDS atomics see varying arrival orders.  If no fiber can
// run while some have not finished, a barrier or wave operation was skipped
// by some thread of the block: the run aborts with a message.
#pragma once
#include <sys/mman.h>
#include <ucontext.h>

#include <algorithm>
#include <cmath>
#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <random>
#include <set>
#include <string>
#include <tuple>
#include <type_traits>
#include <vector>

#if defined(__has_feature)
#if __has_feature(address_sanitizer)
#define HH_ASAN 1
#include <sanitizer/common_interface_defs.h>
#endif
#endif

#define __global__
#define __device__
#define __host__
#define __shared__ static
#define __launch_bounds__(...)
#define __forceinline__ inline
#define __align__(n) __attribute__((aligned(n)))

struct dim3 {
  unsigned x, y, z;
  dim3(unsigned a = 1, unsigned b = 1, unsigned c = 1) : x(a), y(b), z(c) {}
};
struct uint4 {
  unsigned x, y, z, w;
};
struct ulonglong2 {
  unsigned long long x, y;
};

typedef int hipError_t;
enum { hipSuccess = 0, hipErrorInvalidValue = 1, hipErrorInvalidDevice = 101, hipErrorInvalidSymbol = 701 };
typedef struct hh_stream *hipStream_t;
typedef struct hh_event *hipEvent_t;
inline const char *hipGetErrorString(hipError_t) { return "host stand-in error"; }
inline hipError_t hipGetLastError() { return hipSuccess; }
inline hipError_t hipGetDevice(int *d) {
  *d = 0;
  return hipSuccess;
}
#define HIP_SYMBOL(s) (s)
template <typename T>
inline hipError_t hipGetSymbolAddress(void **p, T &sym) {
  *p = (void *)&sym;
  return hipSuccess;
}

inline unsigned __float_as_uint(float f) {
  unsigned u;
  std::memcpy(&u, &f, 4);
  return u;
}
inline float __uint_as_float(unsigned u) {
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

template <typename A, typename B>
inline std::common_type_t<A, B> min(A a, B b) {
  return b < a ? b : a;
}
template <typename A, typename B>
inline std::common_type_t<A, B> max(A a, B b) {
  return a < b ? b : a;
}

namespace hh {

[[noreturn]] inline void fatal(const char *what) {
  std::fprintf(stderr, "host stand-in: %s\n", what);
  std::fflush(stderr);
  std::abort();
}

struct Rendezvous {
  int n = 0, count = 0, gen = 0;
};

struct Fiber {
  ucontext_t ctx;
  char *stack = nullptr;
  bool done = false;
  const Rendezvous *wait = nullptr;  // blocked on this rendezvous ...
  int wait_gen = 0;                  // ... until its generation moves on
#ifdef HH_ASAN
  void *fake = nullptr;
#endif
};

// Fiber stacks: 16 KiB each (ASan clears a switched-to stack's shadow on
// every switch, so small stacks keep the run fast), over a PROT_NONE guard
// page so that an overflow faults instead of corrupting a neighbour.
constexpr size_t kStack = 16 * 1024;
constexpr size_t kGuard = 4096;
inline char *new_stack() {
  void *p = mmap(nullptr, kStack + kGuard, PROT_READ | PROT_WRITE, MAP_PRIVATE | MAP_ANONYMOUS, -1, 0);
  if (p == MAP_FAILED) return nullptr;
  if (mprotect(p, kGuard, PROT_NONE) != 0) return nullptr;
  return static_cast<char *>(p) + kGuard;
}

struct State {
  dim3 block, grid, tid, bid;
  std::vector<Fiber> fib;
  int cur = -1;  // running fiber, -1: the scheduler
  ucontext_t sched;
  Rendezvous bar;
  Rendezvous wave[16];
  uint64_t xch[16][64];  // one slot per lane of each wave
  const std::function<void(int)> *job = nullptr;
  bool serial = false;
  std::set<std::string> serial_kernels;
  std::mt19937 rng{std::getenv("HOSTK_SEED") ? (unsigned)std::atoi(std::getenv("HOSTK_SEED")) : 1u};
  long blocks_run = 0;
  ~State() {
    for (Fiber &f : fib)
      if (f.stack) munmap(f.stack - kGuard, kStack + kGuard);
  }
#ifdef HH_ASAN
  const void *main_bottom = nullptr;
  size_t main_size = 0;
#endif
};
inline State &st() {
  static State s;
  return s;
}

// back to the scheduler from the running fiber (finished: the fiber ends)
inline void to_scheduler(bool finished) {
  State &S = st();
  Fiber &f = S.fib[S.cur];
#ifdef HH_ASAN
  __sanitizer_start_switch_fiber(finished ? nullptr : &f.fake, S.main_bottom, S.main_size);
#endif
  if (finished) {
    f.done = true;
    return;  // the fiber's entry returns; uc_link resumes the scheduler
  }
  swapcontext(&f.ctx, &S.sched);
#ifdef HH_ASAN
  __sanitizer_finish_switch_fiber(f.fake, nullptr, nullptr);
#endif
}

inline void fiber_entry(int i) {
  State &S = st();
#ifdef HH_ASAN
  __sanitizer_finish_switch_fiber(nullptr, &S.main_bottom, &S.main_size);
#endif
  (*S.job)(i);
  to_scheduler(true);
}

inline void arrive(Rendezvous &r, const char *what) {
  State &S = st();
  if (S.serial) {
    std::fprintf(stderr, "host stand-in: %s in a kernel named as free of barriers and wave operations\n", what);
    std::abort();
  }
  const int g = r.gen;
  if (++r.count == r.n) {
    r.count = 0;
    ++r.gen;
    return;
  }
  Fiber &f = S.fib[S.cur];
  f.wait = &r;
  f.wait_gen = g;
  to_scheduler(false);
}

inline int lane() { return (int)(st().tid.x & 63); }
inline int wave() { return (int)(st().tid.x >> 6); }

// every lane publishes v, then takes the value of lane src(l) (its own if
// src(l) < 0)
template <typename F>
inline uint64_t wave_xchg(uint64_t v, F src, const char *what) {
  State &S = st();
  const int w = wave(), l = lane();
  S.xch[w][l] = v;
  arrive(S.wave[w], what);
  const int s = src(l);
  const uint64_t r = S.xch[w][s < 0 ? l : s];
  arrive(S.wave[w], what);
  return r;
}

template <typename T>
inline uint64_t to_u64(T v) {
  static_assert(sizeof(T) <= 8, "wave operation on a value wider than 64 bits");
  uint64_t u = 0;
  std::memcpy(&u, &v, sizeof(T));
  return u;
}
template <typename T>
inline T from_u64(uint64_t u) {
  T v;
  std::memcpy(&v, &u, sizeof(T));
  return v;
}

// one workgroup of n threads
inline void run_block(int n) {
  State &S = st();
  for (int w = 0; w < 16; ++w) S.wave[w] = Rendezvous{64, 0, 0};
  S.bar = Rendezvous{n, 0, 0};
  if (S.serial) {
    for (int t = 0; t < n; ++t) {
      S.tid = dim3((unsigned)t);
      (*S.job)(t);
    }
    return;
  }
  if ((int)S.fib.size() < n) S.fib.resize(n);
  for (int t = 0; t < n; ++t) {
    Fiber &f = S.fib[t];
    if (!f.stack) f.stack = new_stack();
    if (!f.stack) fatal("out of memory for fiber stacks");
    f.done = false;
    f.wait = nullptr;
    getcontext(&f.ctx);
    f.ctx.uc_stack.ss_sp = f.stack;
    f.ctx.uc_stack.ss_size = kStack;
    f.ctx.uc_link = &S.sched;
    makecontext(&f.ctx, (void (*)())fiber_entry, 1, t);
  }
  std::vector<int> order(n);
  for (int t = 0; t < n; ++t) order[t] = t;
  for (int alive = n; alive > 0;) {
    std::shuffle(order.begin(), order.end(), S.rng);
    bool ran = false;
    alive = 0;
    for (int t : order) {
      Fiber &f = S.fib[t];
      if (f.done) continue;
      ++alive;
      if (f.wait && f.wait->gen == f.wait_gen) continue;
      f.wait = nullptr;
      S.cur = t;
      S.tid = dim3((unsigned)t);
#ifdef HH_ASAN
      void *fake = nullptr;
      __sanitizer_start_switch_fiber(&fake, f.stack, kStack);
#endif
      swapcontext(&S.sched, &f.ctx);
#ifdef HH_ASAN
      __sanitizer_finish_switch_fiber(fake, nullptr, nullptr);
#endif
      S.cur = -1;
      ran = true;
      if (f.done) --alive;
    }
    if (alive > 0 && !ran) fatal("every unfinished thread waits at a barrier or wave operation some thread skipped");
  }
}

// run k(args...) over a 1-D grid, blocks in order
template <typename K, typename... A>
inline void launch(const char *name, K k, dim3 grid, dim3 block, A... args) {
  if (block.y != 1 || block.z != 1 || grid.y != 1 || grid.z != 1 || block.x < 1 || block.x > 1024 ||
      block.x % 64 != 0 || grid.x < 1) {
    std::fprintf(stderr, "host stand-in: %s launched as (%u,%u,%u)x(%u,%u,%u), outside the modelled shapes\n", name,
                 grid.x, grid.y, grid.z, block.x, block.y, block.z);
    std::abort();
  }
  State &S = st();
  S.block = block;
  S.grid = grid;
  S.serial = S.serial_kernels.count(name) != 0;
  const std::tuple<A...> targs(args...);
  const std::function<void(int)> job = [&](int) { std::apply(k, targs); };
  S.job = &job;
  for (unsigned b = 0; b < grid.x; ++b) {
    S.bid = dim3(b);
    run_block((int)block.x);
    ++S.blocks_run;
  }
  S.job = nullptr;
  S.serial = false;
}

// kernels free of barriers and wave operations: their threads run one after
// another with no fiber switches (a rendezvous reached then aborts)
inline void add_serial_kernel(const char *name) { st().serial_kernels.insert(name); }

}  // namespace hh

#define threadIdx (hh::st().tid)
#define blockIdx (hh::st().bid)
#define blockDim (hh::st().block)
#define gridDim (hh::st().grid)
#define hipLaunchKernelGGL(K, G, B, SH, S, ...) hh::launch(#K, K, G, B, __VA_ARGS__)

inline void __syncthreads() { hh::arrive(hh::st().bar, "__syncthreads"); }
inline void __threadfence_block() {}
inline void __threadfence() {}

template <typename T, typename V>
inline T atomicAdd(T *p, V v) {
  const T old = *p;
  *p = (T)(old + (T)v);
  return old;
}

template <typename T>
inline T __shfl_up(T v, unsigned off, int width = 64) {
  if (width != 64) hh::fatal("__shfl_up width other than 64 not modelled");
  return hh::from_u64<T>(
      hh::wave_xchg(hh::to_u64(v), [&](int l) { return l >= (int)off ? l - (int)off : -1; }, "__shfl_up"));
}
template <typename T>
inline T __shfl_xor(T v, int m, int width = 64) {
  if (width != 64 || m < 0 || m > 63) hh::fatal("__shfl_xor form not modelled");
  return hh::from_u64<T>(hh::wave_xchg(hh::to_u64(v), [&](int l) { return l ^ m; }, "__shfl_xor"));
}
inline uint64_t __ballot(int pred) {
  hh::State &S = hh::st();
  const int w = hh::wave(), l = hh::lane();
  S.xch[w][l] = pred ? 1u : 0u;
  hh::arrive(S.wave[w], "__ballot");
  uint64_t m = 0;
  for (int i = 0; i < 64; ++i) m |= (S.xch[w][i] ? 1ull : 0ull) << i;
  hh::arrive(S.wave[w], "__ballot");
  return m;
}
inline int __popcll(unsigned long long v) { return __builtin_popcountll(v); }

inline int __builtin_amdgcn_readlane(int v, int src) {
  if (src < 0 || src > 63) hh::fatal("readlane of a lane outside the wave");
  return (int)hh::wave_xchg((uint64_t)(uint32_t)v, [&](int) { return src; }, "readlane");
}
inline int __builtin_amdgcn_readfirstlane(int v) { return __builtin_amdgcn_readlane(v, 0); }

// The DPP moves the kernels use, with bound_ctrl off: a lane with no source
// lane, or in a row outside row_mask, keeps `old`.
//   0x111..0x11f row_shr:n  -- lane i of a 16-lane row takes lane i - n of the row
//   0x142 row_bcast:15      -- every lane of row r > 0 takes lane 15 of row r - 1
//   0x143 row_bcast:31      -- every lane of rows 2 and 3 takes lane 31
inline int __builtin_amdgcn_update_dpp(int old, int src, int ctrl, int row_mask, int bank_mask, bool bound_ctrl) {
  if (bank_mask != 0xf || bound_ctrl) hh::fatal("DPP bank_mask/bound_ctrl form not modelled");
  auto from = [ctrl](int l) -> int {
    const int row = l >> 4, i = l & 15;
    if (ctrl >= 0x111 && ctrl <= 0x11f) {
      const int n = ctrl - 0x110;
      return i >= n ? l - n : -1;
    }
    if (ctrl == 0x142) return row > 0 ? (row - 1) * 16 + 15 : -1;
    if (ctrl == 0x143) return row >= 2 ? 31 : -1;
    hh::fatal("DPP control not modelled");
  };
  const int l = hh::lane();
  const uint64_t v = hh::wave_xchg((uint64_t)(uint32_t)src, from, "update_dpp");
  const bool written = ((row_mask >> (l >> 4)) & 1) && from(l) >= 0;
  return written ? (int)(uint32_t)v : old;
}
