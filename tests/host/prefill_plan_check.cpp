// Host check of the prefill kernels' schedule arithmetic (prefill_plan.h):
//   table  -- prints vm_after(t, first) for t = 0..4, first = 1 then 0, for
//             the test to compare with its own simulation of the issue order;
//   cover  -- for every d_ff multiple of 64 up to 8192 and every row block
//             of 256 columns, runs the gate/up write-out roles (whole pieces
//             and boundary halves) and checks that every column's hi and lo
//             halves are stored exactly once, by the row block that owns the
//             column, at the byte rec_byte gives, and that every image offset
//             stays inside the item's lines.  Prints "ok" or the first fault.
#include <cstdio>
#include <cstring>
#include <map>

#include "prefill_plan.h"

namespace pf = moe::pf;

static int table() {
  for (int first = 1; first >= 0; --first)
    for (int t = 0; t < 5; ++t) std::printf("%d %d %d\n", first, t, pf::vm_after(t, first != 0));
  return 0;
}

static int cover() {
  const int kGRows = 256;  // h columns of a gate/up item
  for (int dff = 64; dff <= 8192; dff += 64) {
    const int nsb = (dff + moe::kSbCols - 1) / moe::kSbCols;
    std::map<long, int> written;  // record byte -> times stored
    for (int c0 = 0; c0 < dff; c0 += kGRows) {
      const int c1 = c0 + kGRows < dff ? c0 + kGRows : dff;
      const int L0 = pf::item_L0(c0), nl = pf::item_nl(c0, c1);
      if (nl > 15 || L0 + nl > 5 * nsb) {
        std::printf("d_ff %d block %d: %d lines from %d\n", dff, c0, nl, L0);
        return 1;
      }
      // every column the block computes lands inside its image
      for (int c = c0; c < c1; ++c) {
        float inv_f;
        const int off = pf::rec_byte(c, inv_f) - L0 * pf::kRecRowB;
        if (off < 0 || off >= nl * pf::kRecRowB || off % pf::kRecRowB >= 64) {
          std::printf("d_ff %d column %d: image byte %d\n", dff, c, off);
          return 1;
        }
      }
      for (int wi = 0; wi < 128; ++wi)
        if (pf::full_piece_own(wi, c0, c1) == 0xffu)
          for (int j = 0; j < 8; ++j) ++written[(long)L0 * pf::kRecRowB + wi * 16 + 2 * j];
      for (int pq = 0; pq < 160; ++pq) {
        const pf::BoundaryRole r = pf::boundary_role(pq, c0, c1);
        if (!r.mine) continue;
        if (r.line < L0 || r.line >= L0 + nl) {
          std::printf("d_ff %d block %d: boundary line %d outside\n", dff, c0, r.line);
          return 1;
        }
        ++written[(long)r.line * pf::kRecRowB + r.piece * 16 + 2 * r.half];
      }
    }
    // exactly the columns' hi and lo halves, once each
    for (int c = 0; c < dff; ++c) {
      float inv_f;
      const long b = pf::rec_byte(c, inv_f);
      for (long h : {b, b + 64}) {
        auto it = written.find(h);
        if (it == written.end() || it->second != 1) {
          std::printf("d_ff %d column %d: byte %ld stored %d times\n", dff, c, h, it == written.end() ? 0 : it->second);
          return 1;
        }
      }
    }
    if ((long)written.size() != 2L * dff) {
      std::printf("d_ff %d: %zu bytes stored for %d columns\n", dff, written.size(), dff);
      return 1;
    }
  }
  std::printf("ok\n");
  return 0;
}

int main(int argc, char **argv) {
  if (argc > 1 && std::strcmp(argv[1], "table") == 0) return table();
  if (argc > 1 && std::strcmp(argv[1], "cover") == 0) return cover();
  std::fprintf(stderr, "usage: %s table|cover\n", argv[0]);
  return 2;
}
