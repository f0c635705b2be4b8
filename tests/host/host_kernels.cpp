// CPU build of the library's index-producing kernels (token bucketing and
// work list, cache resolve and miss fill, decode activation record), run on
// host threads against the stand-in runtime in hip/hip_runtime.h.  Built with
// AddressSanitizer and UBSan; every buffer is allocated at exactly the size
// the library's context gives it (moe_create), so a kernel index past the end
// of a work list, perm, offsets, record, miss list or slot table aborts the
// run.  Results go to a binary file that the pytest side compares with the
// oracle.  Test infrastructure only.
//
//   host_kernels bucket   E T k entry_m build d  in.bin out.bin
//   host_kernels noalloc  E T k                  in.bin out.bin
//   host_kernels resolve  L E S T k calls fill resident d_model d_ff  in.bin out.bin
//   host_kernels bucket_lookup  E T k d_model  in.bin out.bin
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../quantized_expert_ffn_softmax_amd/csrc/bucket.hip"
#include "../../quantized_expert_ffn_softmax_amd/csrc/cache.hip"

moe_status moe_fail(moe_status s, const std::string &msg) {
  std::fprintf(stderr, "moe_fail(%d): %s\n", (int)s, msg.c_str());
  return s;
}

namespace {

[[noreturn]] void die(const char *m) {
  std::fprintf(stderr, "host_kernels: %s\n", m);
  std::exit(2);
}

// an exactly sized heap buffer (AddressSanitizer guards both ends)
template <typename T>
T *exact(size_t n, int fill_byte) {
  if (n == 0) n = 1;  // malloc(0) may return null; one element, never read by a correct kernel
  T *p = static_cast<T *>(std::malloc(n * sizeof(T)));
  if (!p) die("out of memory");
  std::memset(p, fill_byte, n * sizeof(T));
  return p;
}

std::vector<int32_t> read_i32(const char *path, size_t n) {
  std::vector<int32_t> v(n);
  FILE *f = std::fopen(path, "rb");
  if (!f) die("cannot open input");
  if (n && std::fread(v.data(), 4, n, f) != n) die("short input");
  std::fclose(f);
  return v;
}

struct Out {
  FILE *f;
  explicit Out(const char *path) : f(std::fopen(path, "wb")) {
    if (!f) die("cannot open output");
  }
  ~Out() { std::fclose(f); }
  template <typename T>
  void put(const T *p, size_t n) {
    if (n && std::fwrite(p, sizeof(T), n, f) != n) die("short write");
  }
};

// the context sizes moe_create gives a call of at most max_tokens tokens
struct Sizes {
  int max_pairs, max_work, max_work8, n_chunks_max;
};
Sizes ctx_sizes(int max_tokens, int k, int E) {
  Sizes z;
  z.max_pairs = max_tokens * k;
  z.max_work = z.max_pairs / moe::kEntryTokens + (z.max_pairs < E ? z.max_pairs : E) + max_tokens / moe::kEntryTokens + 4;
  z.max_work8 =
      z.max_pairs / moe::kEntryTokens8 + (z.max_pairs < E ? z.max_pairs : E) + max_tokens / moe::kEntryTokens8 + 4;
  z.n_chunks_max = (z.max_pairs + 255) / 256;
  return z;
}

int run_bucket(char **a) {
  const int E = std::atoi(a[0]), T = std::atoi(a[1]), k = std::atoi(a[2]), entry_m = std::atoi(a[3]);
  const int build = std::atoi(a[4]), d = std::atoi(a[5]);
  const char *in = a[6], *out = a[7];
  const int n = T * k;
  std::vector<int32_t> iv = read_i32(in, (size_t)n + (d > 0 ? (size_t)T * d : 0));
  moe_ctx c{};
  c.cfg.n_experts = E;
  c.cfg.top_k = k;
  c.cfg.max_tokens = T;
  c.cfg.d_model = d > 0 ? d : 64;
  c.cfg.d_ff = 64;
  c.L = moe::make_layout(c.cfg.d_model, c.cfg.d_ff);
  const Sizes z = ctx_sizes(T, k, E);
  c.max_pairs = z.max_pairs;
  c.max_work = z.max_work;
  c.n_chunks_max = z.n_chunks_max;
  int32_t *idx = exact<int32_t>(n, 0);
  std::memcpy(idx, iv.data(), (size_t)n * 4);
  c.chunk_ws = exact<int32_t>((size_t)z.n_chunks_max * E, 0xa5);
  c.work = exact<moe::WorkEntry>(z.max_work, 0xa5);
  c.work8 = exact<moe::WorkEntry>(z.max_work8, 0xa5);
  c.n_work = exact<int32_t>(4, 0xa5);
  int32_t *offsets = exact<int32_t>(E + 1, 0xa5);
  int32_t *perm = exact<int32_t>(n, 0xa5);
  float *x = nullptr;
  uint16_t *xrec = nullptr;
  const int xh = moe::xrec_halves(c.L.gate.nsb);
  const size_t xrec_n = (size_t)(T + 1) * xh;
  if (d > 0) {
    x = exact<float>((size_t)T * d, 0);
    std::memcpy(x, iv.data() + n, (size_t)T * d * 4);
    xrec = exact<uint16_t>(xrec_n, 0);  // zeroed at create, as the library does
  }
  // the decode entry size also builds the second list (8-token entries)
  moe::WorkEntry *w8 = entry_m == moe::kEntryTokens ? c.work8 : nullptr;
  const hipError_t e =
      moe::launch_bucket_ex(&c, idx, T, offsets, perm, build != 0, entry_m, x, xrec, xh, (hipStream_t) nullptr, w8);
  if (e != hipSuccess) die("launch_bucket_ex failed");
  Out o(out);
  o.put(offsets, E + 1);
  o.put(perm, n);
  if (build) {
    const int nw = c.n_work[0];
    if (nw < 0 || nw > z.max_work) die("n_work outside the work list");
    o.put(c.n_work, 2);
    o.put(reinterpret_cast<const int32_t *>(c.work), (size_t)nw * 4);
    if (w8) {
      const int nw8 = c.n_work[2];
      if (nw8 < 0 || nw8 > z.max_work8) die("n_work[2] outside the second work list");
      o.put(c.n_work + 2, 2);
      o.put(reinterpret_cast<const int32_t *>(c.work8), (size_t)nw8 * 4);
    }
  }
  if (d > 0) o.put(xrec, xrec_n);
  std::free(idx);
  std::free(c.chunk_ws);
  std::free(c.work);
  std::free(c.work8);
  std::free(c.n_work);
  std::free(offsets);
  std::free(perm);
  std::free(x);
  std::free(xrec);
  return 0;
}

int run_noalloc(char **a) {
  const int E = std::atoi(a[0]), T = std::atoi(a[1]), k = std::atoi(a[2]);
  const char *in = a[3], *out = a[4];
  const int n = T * k;
  std::vector<int32_t> iv = read_i32(in, n);
  int32_t *idx = exact<int32_t>(n, 0);
  std::memcpy(idx, iv.data(), (size_t)n * 4);
  int32_t *offsets = exact<int32_t>(E + 1, 0xa5);
  int32_t *perm = exact<int32_t>(n, 0xa5);
  const moe_status st = moe_bucket_noalloc(idx, T, k, E, offsets, perm, nullptr);
  Out o(out);
  const int32_t s32 = (int32_t)st;
  o.put(&s32, 1);
  if (st == MOE_OK) {
    o.put(offsets, E + 1);
    o.put(perm, n);
  }
  std::free(idx);
  std::free(offsets);
  std::free(perm);
  return 0;
}

int run_resolve(char **a) {
  const int L = std::atoi(a[0]), E = std::atoi(a[1]), S = std::atoi(a[2]), T = std::atoi(a[3]), k = std::atoi(a[4]);
  const int calls = std::atoi(a[5]), fill = std::atoi(a[6]), resident = std::atoi(a[7]);
  const int dm = std::atoi(a[8]), dff = std::atoi(a[9]);
  const char *in = a[10], *out = a[11];
  const int n = T * k;
  // input: per call, its layer then its T*k expert ids
  std::vector<int32_t> iv = read_i32(in, (size_t)calls * (1 + n));
  moe_ctx c{};
  c.cfg.d_model = dm;
  c.cfg.d_ff = dff;
  c.cfg.n_experts = E;
  c.cfg.top_k = k;
  c.cfg.n_layers = L;
  c.cfg.n_slots = S;
  c.cfg.max_tokens = T;
  c.L = moe::make_layout(dm, dff);
  c.resident = resident != 0;
  const Sizes z = ctx_sizes(T, k, E);
  c.max_pairs = z.max_pairs;
  const size_t ids = (size_t)L * E, stride = c.L.stride;
  c.slot_of = exact<int32_t>(ids, 0xff);  // -1: nothing resident
  c.id_of = exact<int32_t>(S, 0xff);
  c.stamp = exact<uint32_t>(S, 0);
  c.dstats = exact<int64_t>(8, 0);
  c.dmiss = exact<int32_t>(3 + 2 * (size_t)z.max_pairs + 2 * (size_t)E, 0xa5);
  uint8_t *host = nullptr, *pool = nullptr;
  if (!resident) {
    host = exact<uint8_t>(ids * stride, 0);
    for (size_t i = 0; i < ids; ++i)  // each identity's blob: a pattern of its own
      for (size_t b = 0; b < stride; ++b) host[i * stride + b] = (uint8_t)((i * 131 + b * 7 + (b >> 8)) & 0xff);
    pool = exact<uint8_t>((size_t)S * stride, 0);
    c.host_dev = host;
    c.cfg.slot_pool = pool;
  }
  int32_t *idx = exact<int32_t>(n, 0);
  int32_t *sop = exact<int32_t>(n, 0xa5);
  // fill == 2: no fill kernel; the fill runs in the bucketing launch of a
  // capped decode layer (launch_bucket_fill), which needs the bucketing workspace
  if (fill == 2) {
    c.max_work = z.max_work;
    c.max_work8 = z.max_work8;
    c.offsets_ws = exact<int32_t>(E + 1, 0xa5);
    c.perm_ws = exact<int32_t>(z.max_pairs, 0xa5);
    c.work = exact<moe::WorkEntry>(z.max_work, 0xa5);
    c.work8 = exact<moe::WorkEntry>(z.max_work8, 0xa5);
    c.n_work = exact<int32_t>(4, 0xa5);
  }
  Out o(out);
  for (int call = 0; call < calls; ++call) {
    const int32_t *rec = iv.data() + (size_t)call * (1 + n);
    const int layer = rec[0];
    if (layer < 0 || layer >= L) die("layer out of range");
    std::memcpy(idx, rec + 1, (size_t)n * 4);
    std::memset(sop, 0xa5, (size_t)n * 4);
    if (moe::launch_resolve(&c, layer, idx, T, sop, fill != 0, (hipStream_t) nullptr, fill != 2) != hipSuccess)
      die("launch_resolve failed");
    if (fill == 2 &&
        moe::launch_bucket_fill(&c, idx, T, moe::kEntryTokens, nullptr, nullptr, 0, (hipStream_t) nullptr) !=
            hipSuccess)
      die("launch_bucket_fill refused the shape");
    o.put(c.dmiss, 3);
    o.put(sop, n);
  }
  o.put(c.dstats, 6);
  if (!resident) {
    o.put(c.slot_of, ids);
    o.put(c.id_of, S);
    o.put(c.stamp, S);
    // every occupied slot holds its identity's blob (the fill path copies it
    // from the host store; without fill the host copies it, not modelled here)
    int32_t bad = 0;
    if (fill)
      for (int s = 0; s < S; ++s)
        if (c.id_of[s] >= 0 && std::memcmp(pool + (size_t)s * stride, host + (size_t)c.id_of[s] * stride, stride) != 0)
          ++bad;
    o.put(&bad, 1);
  }
  std::free(c.slot_of);
  std::free(c.id_of);
  std::free(c.stamp);
  std::free(c.dstats);
  std::free(c.dmiss);
  std::free(host);
  std::free(pool);
  std::free(idx);
  std::free(sop);
  std::free(c.offsets_ws);
  std::free(c.perm_ws);
  std::free(c.work);
  std::free(c.work8);
  std::free(c.n_work);
  return 0;
}

// A capped decode layer's first single-workgroup launch for one or two
// tokens: the router's top-k from given partial logits, then the resolve.
// Input: bias [E] (float32 bits), then per call its layer and the partials
// [KS][T][E].  Output per call: logits [T][E], idx [T][k], w [T][k], the
// miss-list head and slot_of_pair; then the counters and the table.
int run_route_resolve(char **a) {
  const int L = std::atoi(a[0]), E = std::atoi(a[1]), S = std::atoi(a[2]), T = std::atoi(a[3]), k = std::atoi(a[4]);
  const int KS = std::atoi(a[5]), calls = std::atoi(a[6]);
  const char *in = a[7], *out = a[8];
  const int n = T * k;
  const size_t per_call = 1 + (size_t)KS * T * E;
  std::vector<int32_t> iv = read_i32(in, (size_t)E + (size_t)calls * per_call);
  moe_ctx c{};
  c.cfg.d_model = 64;
  c.cfg.d_ff = 64;
  c.cfg.n_experts = E;
  c.cfg.top_k = k;
  c.cfg.n_layers = L;
  c.cfg.n_slots = S;
  c.cfg.max_tokens = T;
  c.L = moe::make_layout(64, 64);
  c.resident = false;
  c.route_ks = KS;
  c.route_small_t = T;
  const Sizes z = ctx_sizes(T, k, E);
  c.max_pairs = z.max_pairs;
  const size_t ids = (size_t)L * E;
  c.slot_of = exact<int32_t>(ids, 0xff);
  c.id_of = exact<int32_t>(S, 0xff);
  c.stamp = exact<uint32_t>(S, 0);
  c.dstats = exact<int64_t>(8, 0);
  c.dmiss = exact<int32_t>(3 + 2 * (size_t)z.max_pairs + 2 * (size_t)E, 0xa5);
  c.route_part = exact<float>((size_t)KS * T * E, 0);
  float *bias = exact<float>(E, 0);
  std::memcpy(bias, iv.data(), (size_t)E * 4);
  float *logits = exact<float>((size_t)T * E, 0xa5);
  int32_t *idx = exact<int32_t>(n, 0xa5);
  float *w = exact<float>(n, 0xa5);
  int32_t *sop = exact<int32_t>(n, 0xa5);
  Out o(out);
  for (int call = 0; call < calls; ++call) {
    const int32_t *rec = iv.data() + E + (size_t)call * per_call;
    const int layer = rec[0];
    if (layer < 0 || layer >= L) die("layer out of range");
    std::memcpy(c.route_part, rec + 1, (size_t)KS * T * E * 4);
    if (moe::launch_route_resolve(&c, layer, T, bias, logits, idx, w, sop, (hipStream_t) nullptr) != hipSuccess)
      die("launch_route_resolve refused the shape");
    o.put(reinterpret_cast<const int32_t *>(logits), (size_t)T * E);
    o.put(idx, n);
    o.put(reinterpret_cast<const int32_t *>(w), n);
    o.put(c.dmiss, 3);
    o.put(sop, n);
  }
  o.put(c.dstats, 6);
  o.put(c.slot_of, ids);
  o.put(c.id_of, S);
  o.put(c.stamp, S);
  std::free(c.slot_of);
  std::free(c.id_of);
  std::free(c.stamp);
  std::free(c.dstats);
  std::free(c.dmiss);
  std::free(c.route_part);
  std::free(bias);
  std::free(logits);
  std::free(idx);
  std::free(w);
  std::free(sop);
  return 0;
}

// The bucketing launch of a resident decode layer, which also records the
// lookup (as the resolve kernel does for a resident call).  Input: idx [T][k],
// x [T][d] (float32 bits).  With KS > 0 (T <= 2) the launch also finishes the
// router's top-k: the input is then bias [E], partial logits [KS][T][E] and x,
// and the output starts with logits [T][E], idx [T][k] and w [T][k].
int run_bucket_lookup(char **a, int KS) {
  const int E = std::atoi(a[0]), T = std::atoi(a[1]), k = std::atoi(a[2]), d = std::atoi(a[3]);
  const char *in = a[4], *out = a[5];
  const int n = T * k;
  const size_t head = KS > 0 ? (size_t)E + (size_t)KS * T * E : (size_t)n;
  std::vector<int32_t> iv = read_i32(in, head + (size_t)T * d);
  moe_ctx c{};
  c.cfg.n_experts = E;
  c.cfg.top_k = k;
  c.cfg.max_tokens = T;
  c.cfg.d_model = d;
  c.cfg.d_ff = 64;
  c.cfg.n_layers = 1;
  c.cfg.n_slots = E;
  c.resident = true;
  c.L = moe::make_layout(d, c.cfg.d_ff);
  const Sizes z = ctx_sizes(T, k, E);
  c.max_pairs = z.max_pairs;
  c.max_work = z.max_work;
  int32_t *idx = exact<int32_t>(n, 0xa5);
  if (KS == 0) std::memcpy(idx, iv.data(), (size_t)n * 4);
  float *bias = exact<float>(E, 0), *logits = exact<float>((size_t)T * E, 0xa5), *w = exact<float>(n, 0xa5);
  if (KS > 0) {
    c.route_ks = KS;
    c.route_small_t = T;
    c.route_part = exact<float>((size_t)KS * T * E, 0);
    std::memcpy(bias, iv.data(), (size_t)E * 4);
    std::memcpy(c.route_part, iv.data() + E, (size_t)KS * T * E * 4);
  }
  float *x = exact<float>((size_t)T * d, 0);
  std::memcpy(x, iv.data() + head, (size_t)T * d * 4);
  const int xh = moe::xrec_halves(c.L.gate.nsb);
  const size_t xrec_n = (size_t)(T + 1) * xh;
  uint16_t *xrec = exact<uint16_t>(xrec_n, 0);
  c.dmiss = exact<int32_t>(3 + 2 * (size_t)z.max_pairs + 2 * (size_t)E, 0xa5);
  c.dstats = exact<int64_t>(8, 0);
  c.offsets_ws = exact<int32_t>(E + 1, 0xa5);
  c.perm_ws = exact<int32_t>(z.max_pairs, 0xa5);
  c.work = exact<moe::WorkEntry>(z.max_work, 0xa5);
  c.work8 = exact<moe::WorkEntry>(z.max_work8, 0xa5);
  c.n_work = exact<int32_t>(4, 0xa5);
  for (int call = 0; call < 2; ++call) {  // twice: the counters accumulate
    const hipError_t e =
        KS > 0 ? moe::launch_route_bucket_lookup(&c, T, bias, logits, idx, w, moe::kEntryTokens, x, xrec, xh,
                                                 (hipStream_t) nullptr)
               : moe::launch_bucket_lookup(&c, idx, T, moe::kEntryTokens, x, xrec, xh, (hipStream_t) nullptr);
    if (e != hipSuccess) die("the bucketing launch refused the shape");
  }
  Out o(out);
  if (KS > 0) {
    o.put(reinterpret_cast<const int32_t *>(logits), (size_t)T * E);
    o.put(idx, n);
    o.put(reinterpret_cast<const int32_t *>(w), n);
  }
  o.put(c.offsets_ws, E + 1);
  o.put(c.perm_ws, n);
  const int nw = c.n_work[0];
  if (nw < 0 || nw > z.max_work) die("n_work outside the work list");
  o.put(c.n_work, 2);
  o.put(reinterpret_cast<const int32_t *>(c.work), (size_t)nw * 4);
  const int nw8 = c.n_work[2];
  if (nw8 < 0 || nw8 > z.max_work8) die("n_work[2] outside the second work list");
  o.put(c.n_work + 2, 2);
  o.put(reinterpret_cast<const int32_t *>(c.work8), (size_t)nw8 * 4);
  o.put(xrec, xrec_n);
  o.put(c.dmiss, 3);
  o.put(c.dstats, 6);
  std::free(idx);
  std::free(bias);
  std::free(logits);
  std::free(w);
  std::free(c.route_part);
  std::free(x);
  std::free(xrec);
  std::free(c.dmiss);
  std::free(c.dstats);
  std::free(c.offsets_ws);
  std::free(c.perm_ws);
  std::free(c.work);
  std::free(c.work8);
  std::free(c.n_work);
  return 0;
}

}  // namespace

int main(int argc, char **argv) {
  if (argc < 2) die("usage: host_kernels bucket|noalloc|resolve ...");
  // the miss fill has neither barriers nor wave operations: its threads run
  // one after another (the stand-in aborts if it ever reaches a rendezvous)
  hh::add_serial_kernel("fill_kernel");
  const std::string mode = argv[1];
  if (mode == "bucket" && argc == 10) return run_bucket(argv + 2);
  if (mode == "noalloc" && argc == 7) return run_noalloc(argv + 2);
  if (mode == "resolve" && argc == 14) return run_resolve(argv + 2);
  if (mode == "bucket_lookup" && argc == 8) return run_bucket_lookup(argv + 2, 0);
  if (mode == "route_bucket" && argc == 9) return run_bucket_lookup(argv + 3, std::atoi(argv[2]));
  if (mode == "route_resolve" && argc == 11) return run_route_resolve(argv + 2);
  die("bad arguments");
}
