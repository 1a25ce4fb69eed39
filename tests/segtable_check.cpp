// Host check of the segment-table clamp every kernel applies to its entry (SegTable::clamp in csrc/common.h).
//   segtable_check fuzz N SEED   N random tables with random totals: every clamped entry lies inside the
//                                totals (the ranges the library sizes its grids and buffers from).
//   segtable_check identity      reads "n_tokens total_kept max_seg max_doc max_kept n_seg" and n_seg lines of
//                                seven fields from stdin: each entry must come out unchanged.
// Prints "ok" and exits 0, or prints the first violation and exits 1.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "common.h"

static int inside(const tg_segment& s, int64_t nt, int64_t tk, int64_t ms, int64_t md, int64_t mk) {
  const int64_t n_doc = (int64_t)s.doc_end - s.doc_begin;
  if (s.seg_start < 0 || (int64_t)s.seg_start + s.seg_len > nt || s.seg_len < 0 || s.seg_len > ms) return 0;
  if (s.doc_begin < 0 || n_doc < 0 || s.doc_end > s.seg_len || n_doc > md) return 0;
  if (s.k_eff < 0 || s.k_eff > n_doc) return 0;
  if (s.kept_start < 0 || s.kept_len < 0 || (int64_t)s.kept_start + s.kept_len > tk || s.kept_len > mk) return 0;
  return 1;
}

static void show(const char* what, const tg_segment& s) {
  std::printf("%s: %d %d %d %d %d %d %d\n", what, s.seg_start, s.seg_len, s.doc_begin, s.doc_end, s.k_eff,
              s.kept_start, s.kept_len);
}

int main(int argc, char** argv) {
  if (argc >= 4 && std::strcmp(argv[1], "fuzz") == 0) {
    const long n = std::atol(argv[2]);
    std::mt19937_64 rng(std::strtoull(argv[3], nullptr, 10));
    const int32_t edge[] = {INT32_MIN, INT32_MIN + 1, -65537, -1, 0, 1, 63, 64, 65, 4096, 32768, 65536,
                            INT32_MAX - 1, INT32_MAX};
    auto field = [&](int32_t hi) -> int32_t {
      switch (rng() % 4) {
        case 0: return edge[rng() % (sizeof(edge) / sizeof(edge[0]))];
        case 1: return (int32_t)(rng() % ((uint64_t)hi + 2));
        case 2: return (int32_t)rng();
        default: return hi - (int32_t)(rng() % 3);
      }
    };
    for (long it = 0; it < n; ++it) {
      // totals that pass the host checks: n_tokens < 2^31, total_kept <= n_tokens, max_doc and max_kept <= max_seg
      const int32_t nt = (int32_t)(rng() % 2 ? rng() % 200000 : rng() % 0x80000000ULL);
      const int32_t tk = (int32_t)(rng() % ((uint64_t)nt + 1));
      const int32_t ms = (int32_t)(rng() % ((uint64_t)nt + 1));
      const int32_t md = (int32_t)(rng() % ((uint64_t)ms + 1));
      const int32_t mk = (int32_t)(rng() % ((uint64_t)ms + 1));
      tg_segment r{field(nt), field(ms), field(ms), field(ms), field(md), field(tk), field(mk), (int32_t)rng()};
      const tg_segment s = tg::SegTable::clamp(r, nt, tk, ms, md, mk);
      if (!inside(s, nt, tk, ms, md, mk)) {
        std::printf("totals %d %d %d %d %d\n", nt, tk, ms, md, mk);
        show("raw", r);
        show("clamped", s);
        return 1;
      }
    }
    std::printf("ok\n");
    return 0;
  }
  if (argc >= 2 && std::strcmp(argv[1], "identity") == 0) {
    long long nt, tk, ms, md, mk, ns;
    if (std::scanf("%lld %lld %lld %lld %lld %lld", &nt, &tk, &ms, &md, &mk, &ns) != 6) return 2;
    for (long long i = 0; i < ns; ++i) {
      tg_segment r{};
      if (std::scanf("%d %d %d %d %d %d %d", &r.seg_start, &r.seg_len, &r.doc_begin, &r.doc_end, &r.k_eff,
                     &r.kept_start, &r.kept_len) != 7)
        return 2;
      const tg_segment s = tg::SegTable::clamp(r, (int32_t)nt, (int32_t)tk, (int32_t)ms, (int32_t)md, (int32_t)mk);
      if (std::memcmp(&r, &s, sizeof r) != 0) {
        show("raw", r);
        show("clamped", s);
        return 1;
      }
    }
    std::printf("ok\n");
    return 0;
  }
  std::fprintf(stderr, "usage: segtable_check fuzz N SEED | identity < table\n");
  return 2;
}
