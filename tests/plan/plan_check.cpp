// Host check of the GEMM's tile plan and of the persistent walk over it,
// built from the kernel header itself (tests/test_tile_plan.py compiles and
// runs it on the CPU). For each shape and CU count:
// - every 64 x 64 cell of the M x N output is covered by exactly one tile
//   (tile edges and origins are multiples of 64), and no tile starts outside
//   the output;
// - the persistent launch's workgroups (ids w, w + grid, ...) take every tile
//   id exactly once, each keeping to one XCD (id % 8 == w % 8) when the grid
//   is a multiple of 8;
// - a narrow plan is used only when the partial last round exists, and it
//   fills exactly one round of narrow tiles at most.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "gemm_kernels.h"

using namespace fp8mp;

static int g_fail = 0;
#define CHECK(cond, ...)                              \
  do {                                                \
    if (!(cond)) {                                    \
      ++g_fail;                                       \
      std::printf("FAIL %s:%d ", __FILE__, __LINE__); \
      std::printf(__VA_ARGS__);                       \
      std::printf("\n");                              \
    }                                                 \
  } while (0)

template <int NARROW>
static void walk(int64_t m, int64_t n, int num_cus, const TilePlan& p) {
  using G2 = typename NarrowGeom<NARROW>::G;
  const int total = p.tm * p.tn + p.tm2 * p.tn2;
  const int64_t cm = (m + 63) / 64, cn = (n + 63) / 64;
  std::vector<int> cover((size_t)(cm * cn), 0);
  for (int bid = 0; bid < total; ++bid) {
    int64_t m0, n0;
    const bool nar = plan_tile<NARROW>(bid, p, m0, n0);
    const int bm = nar ? G2::BM : kBM, bn = nar ? G2::BN : kBN;
    CHECK(m0 >= 0 && n0 >= 0 && m0 < m && n0 < n, "tile %d at (%lld, %lld) outside %lld x %lld", bid, (long long)m0,
          (long long)n0, (long long)m, (long long)n);
    CHECK(m0 % 64 == 0 && n0 % 64 == 0, "tile origin not on the 64 grid");
    for (int64_t r = m0 / 64; r < (m0 + bm) / 64 && r < cm; ++r)
      for (int64_t c = n0 / 64; c < (n0 + bn) / 64 && c < cn; ++c) ++cover[(size_t)(r * cn + c)];
  }
  for (size_t i = 0; i < cover.size(); ++i)
    if (cover[i] != 1) {
      CHECK(false, "%lld x %lld on %d CUs: cell %zu covered %d times", (long long)m, (long long)n, num_cus, i, cover[i]);
      break;
    }
  // the persistent launch's workgroups
  const int grid = persistent_grid(total, num_cus);
  CHECK(grid >= 1 && grid <= total, "grid %d for %d tiles", grid, total);
  if (num_cus >= 8 && total >= num_cus) CHECK(grid % 8 == 0 && grid <= num_cus, "grid %d on %d CUs", grid, num_cus);
  std::vector<int> taken((size_t)total, 0);
  for (int w = 0; w < grid; ++w)
    for (int bid = w; bid < total; bid += grid) {
      ++taken[(size_t)bid];
      if (grid % 8 == 0) CHECK(bid % 8 == w % 8, "workgroup %d leaves its XCD at tile id %d", w, bid);
    }
  for (int bid = 0; bid < total; ++bid) CHECK(taken[(size_t)bid] == 1, "tile id %d taken %d times", bid, taken[(size_t)bid]);
}

static void check(int64_t m, int64_t n, int num_cus) {
  TilePlan p;
  const int kind = plan_tiles(m, n, num_cus, p);
  const int64_t whole = ((m + kBM - 1) / kBM) * ((n + kBN - 1) / kBN);
  if (kind != kNarrowNone) {
    CHECK(num_cus > 0 && whole > num_cus && whole % num_cus != 0, "narrow plan without a partial last round");
    CHECK(p.tm2 * p.tn2 <= num_cus, "more than one round of narrow tiles: %d", p.tm2 * p.tn2);
    CHECK((p.tm * p.tn) % num_cus == 0, "whole tiles do not fill whole rounds");
  } else {
    CHECK(p.tm * p.tn == whole && p.tm2 * p.tn2 == 0, "whole-tile plan does not cover the whole tiles");
  }
  switch (kind) {
    case kNarrowN192: walk<kNarrowN192>(m, n, num_cus, p); break;
    case kNarrowN128: walk<kNarrowN128>(m, n, num_cus, p); break;
    case kNarrowM192: walk<kNarrowM192>(m, n, num_cus, p); break;
    case kNarrowM128: walk<kNarrowM128>(m, n, num_cus, p); break;
    default: walk<kNarrowNone>(m, n, num_cus, p);
  }
}

int main() {
  // the workloads' GEMM shapes (7B MLP forward, dgrad, wgrad; 13B projections; 70B slice; tiny)
  const int64_t shapes[][2] = {{4096, 11008}, {4096, 4096}, {11008, 4096}, {8192, 15360}, {8192, 13824},
                               {16384, 28672}, {256, 1024}, {4000, 6900}, {4000, 4452}, {6900, 4000}, {4452, 4000},
                               {4100, 4100}, {8192, 8448}, {1, 1}, {257, 129}};
  const int cus[] = {256, 304, 80, 64, 8, 7, 1, 0};
  for (const auto& s : shapes)
    for (int c : cus) check(s[0], s[1], c);
  unsigned x = 12345u;
  auto rnd = [&](int lo, int hi) {
    x = x * 1664525u + 1013904223u;
    return lo + (int)((x >> 8) % (unsigned)(hi - lo + 1));
  };
  for (int i = 0; i < 300; ++i) check(rnd(1, 20000), rnd(1, 20000), cus[rnd(0, 6)]);
  std::printf("plan check: %d failures\n", g_fail);
  return g_fail == 0 ? 0 : 1;
}
