// CPU bounds check of the grouped GEMMs' index math (mixture_experts_layer_adjusted_amd/csrc/tile_walk.h),
// built with address and undefined-behaviour sanitisers and standard-library assertions.
//
// For one routing (T tokens, K picks each among N routed experts, Ns shared experts; seeded, with a
// chosen skew; or per-expert loads of 128 q + 1 rows, the most padding a routing can need; or of
// 256 q + 1 rows, an odd number of M-tiles in every segment, the most 256-row tiles) it builds the permuted layout by its definition: segment i holds the tokens that
// picked routed expert i in increasing token order, then one full-token segment per shared expert,
// each segment starting on a multiple of 128 rows; 256-row tiles (pairs of 128-row M-tiles, a
// segment with an odd count ending in a half tile) are numbered segment by segment.  It then runs
// the tile walks the kernels run, with the functions they call, and checks that
//  * the layout fits the workspace the library plans for this shape (walk_max_tiles M-tiles,
//    walk_max_pairs 256-row tiles): every row index the kernels form is below max_tiles * 128,
//    every table index below max_tiles;
//  * every tile a walk yields lies inside its segment (a half tile only at a segment's end), its
//    N-tile is below NT, and every (tile, N-tile) of every segment is yielded exactly once: by the
//    one-tile grids over 256-row and 128-row tiles, and by the persistent walk for several
//    workgroup counts;
//  * the persistent walk's indices, including the two tiles it looks ahead, stay below 2^31.
// Exit status 0 when every check holds; the first failed check aborts with its message.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <stdexcept>
#include <string>
#include <vector>

#include "../../mixture_experts_layer_adjusted_amd/csrc/tile_walk.h"

using namespace moe;

#define CHECK(c, msg)                                                                      \
  do {                                                                                     \
    if (!(c)) {                                                                            \
      std::fprintf(stderr, "check failed: %s (%s) at line %d\n", #c, msg, __LINE__);       \
      std::abort();                                                                        \
    }                                                                                      \
  } while (0)

struct Layout {
  std::vector<int> rows, seg_off, pair_off, pair_seg, tile_seg;
  int64_t max_tiles = 0, max_pairs = 0;
};

static Layout build(const std::vector<int>& rows, int64_t max_tiles, int64_t max_pairs) {
  Layout L;
  L.rows = rows;
  L.max_tiles = max_tiles;
  L.max_pairs = max_pairs;
  const int nseg = (int)rows.size();
  L.seg_off.assign(nseg + 1, 0);
  L.pair_off.assign(nseg + 1, 0);
  for (int s = 0; s < nseg; ++s) {
    const int padded = (rows[s] + 127) / 128 * 128;
    L.seg_off[s + 1] = L.seg_off[s] + padded;
    L.pair_off[s + 1] = L.pair_off[s] + (padded / 128 + 1) / 2;
  }
  CHECK(L.seg_off[nseg] <= max_tiles * 128, "layout larger than the planned workspace");
  CHECK(L.pair_off[nseg] <= max_pairs, "more 256-row tiles than planned");
  CHECK(max_pairs <= max_tiles, "pair table larger than the planned workspace");
  L.tile_seg.assign(max_tiles, -1);
  L.pair_seg.assign(max_tiles, -1);
  for (int s = 0; s < nseg; ++s) {
    for (int j = L.seg_off[s] / 128; j < L.seg_off[s + 1] / 128; ++j) L.tile_seg.at(j) = s;
    for (int j = L.pair_off[s]; j < L.pair_off[s + 1]; ++j) L.pair_seg.at(j) = s;
  }
  return L;
}

// check one yielded tile of TM rows (256: pair walk, 128: M-tile walk) and mark it
static void visit(const Layout& L, int seg, const WalkTile& t, int TM, int NT, std::vector<char>& seen) {
  CHECK(seg >= 0 && seg < (int)L.rows.size(), "segment index");
  CHECK(t.nt >= 0 && t.nt < NT, "N-tile index");
  CHECK(t.m0 >= L.seg_off[seg] && t.m0 < L.seg_off[seg + 1], "tile starts inside its segment");
  CHECK((t.m0 - L.seg_off[seg]) % TM == 0, "tile aligned within its segment");
  CHECK(t.tile_rows == TM || (TM == 256 && t.tile_rows == 128), "tile height");
  CHECK(t.m0 + t.tile_rows <= L.seg_off[seg + 1], "tile ends inside its segment");
  CHECK(t.tile_rows == TM || t.m0 + t.tile_rows == L.seg_off[seg + 1], "a half tile only at a segment's end");
  CHECK(t.m0 + t.tile_rows <= L.max_tiles * 128, "rows inside the workspace");
  const int64_t key = (t.m0 / 128) * NT + t.nt;
  CHECK(key >= 0 && key < (int64_t)seen.size(), "visit index");
  CHECK(!seen[key], "tile yielded twice");
  seen[key] = 1;
}

static void expect_all(const Layout& L, int TM, int NT, const std::vector<char>& seen, const char* walk) {
  for (size_t s = 0; s + 1 < L.seg_off.size(); ++s)
    for (int64_t m = L.seg_off[s]; m < L.seg_off[s + 1]; m += TM)
      for (int nt = 0; nt < NT; ++nt) CHECK(seen[(m / 128) * NT + nt], walk);
}

// one-tile grid over 256-row tiles (streaming and FP8 kernels) or 128-row tiles (decode-sized
// form), `chunk` workgroups per XCD
static void one_tile_grid(const Layout& L, int TM, int NT, int group_m, int chunk) {
  const int64_t max_slots = TM == 256 ? L.max_pairs : L.max_tiles;
  const int64_t span = (int64_t)kWalkXcds * chunk;
  const int64_t grid = (max_slots * NT + span - 1) / span * span;
  std::vector<char> seen((size_t)L.max_tiles * NT, 0);
  for (int64_t b = 0; b < grid; ++b) {
    const int64_t l = xcd_logical(b, chunk);
    CHECK(l >= 0 && l < grid, "logical index inside the grid");
    const int64_t slot = l / NT;
    if (slot >= L.max_tiles) continue;
    const int seg = TM == 256 ? L.pair_seg.at(slot) : L.tile_seg.at(slot);
    if (seg < 0) continue;
    const int first = TM == 256 ? L.pair_off[seg] : L.seg_off[seg] / 128;
    const int count = TM == 256 ? L.pair_off[seg + 1] - first : L.seg_off[seg + 1] / 128 - first;
    visit(L, seg, walk_tile(l, NT, group_m, TM, first, count, L.seg_off[seg], L.seg_off[seg + 1]), TM, NT, seen);
  }
  expect_all(L, TM, NT, seen, TM == 256 ? "one-tile grid misses a 256-row tile" : "one-tile grid misses an M-tile");
}

// the persistent walk over 256-row tiles with G workgroups
static void persistent_walk(const Layout& L, int NT, int group_m, int G) {
  std::vector<char> seen((size_t)L.max_tiles * NT, 0);
  CHECK(L.max_tiles * NT + 2LL * G < (1LL << 31), "walk indices fit in int");
  auto seg_of = [&](int64_t l) { return l / NT < L.max_tiles ? L.pair_seg.at(l / NT) : -1; };
  for (int b = 0; b < G; ++b) {
    int64_t l = persistent_first(b, G);
    CHECK(l >= 0 && l < G, "first tile of a workgroup");
    while (true) {
      const int seg = seg_of(l);
      if (seg < 0) break;
      (void)seg_of(l + G);       // the kernel reads the next two tiles' segments ahead
      (void)seg_of(l + 2 * G);
      const int first = L.pair_off[seg];
      visit(L, seg, walk_tile(l, NT, group_m, 256, first, L.pair_off[seg + 1] - first, L.seg_off[seg],
                              L.seg_off[seg + 1]), 256, NT, seen);
      l += G;
    }
  }
  expect_all(L, 256, NT, seen, "persistent walk misses a tile");
}

int main(int argc, char** argv) {
  if (argc != 7) {
    std::fprintf(stderr,
                 "usage: %s T N K Ns seed skew (0 uniform, 1 Zipf-like, 2 one favoured expert, "
                 "3 loads of 128 q + 1 rows, 4 loads of 256 q + 1 rows)\n", argv[0]);
    return 2;
  }
  const int T = std::atoi(argv[1]), N = std::atoi(argv[2]), K = std::atoi(argv[3]), Ns = std::atoi(argv[4]);
  const unsigned seed = (unsigned)std::atoi(argv[5]);
  const int skew = std::atoi(argv[6]);
  CHECK(T >= 0 && N >= 1 && K >= 1 && K <= N && Ns >= 0, "shape");
  std::vector<int> rows(N + Ns, 0);
  if (skew == 3 || skew == 4) {
    // one row per expert while the picks last, then 128 (256) more at a time (no load above T): a
    // load vector with sum T K and every load <= T is the load of some routing with K distinct picks
    const int64_t step = skew == 3 ? 128 : 256;
    int64_t left = (int64_t)T * K;
    for (int e = 0; e < N && left > 0; ++e, --left) rows[e] = 1;
    for (int e = 0; left > 0; e = (e + 1) % N) {
      const int64_t add = std::min<int64_t>({step, left, (int64_t)T - rows[e]});
      rows[e] += (int)add;
      left -= add;
    }
  } else {
    // K distinct experts per token, drawn with weights (uniform, r^-1.1, or one expert favoured)
    std::mt19937_64 rng(seed);
    std::vector<double> w(N);
    for (int e = 0; e < N; ++e) w[e] = skew == 1 ? 1.0 / std::pow(e + 1.0, 1.1) : (skew == 2 && e == N / 2 ? 1e6 : 1.0);
    for (int t = 0; t < T; ++t) {
      std::vector<double> ww = w;
      for (int k = 0; k < K; ++k) {
        std::discrete_distribution<int> d(ww.begin(), ww.end());
        const int e = d(rng);
        CHECK(ww[e] > 0, "distinct picks");
        ww[e] = 0;
        ++rows[e];
      }
    }
  }
  for (int s = 0; s < Ns; ++s) rows[N + s] = T;
  const int64_t max_tiles = walk_max_tiles(T, K, N, Ns);
  const Layout L = build(rows, max_tiles, walk_max_pairs(max_tiles, N + Ns));
  for (int NT : {1, 3, 8, 16, 28}) {
    for (int group_m : {4, 8}) {
      for (int chunk : {32, 64}) {
        one_tile_grid(L, 256, NT, group_m, chunk);
        one_tile_grid(L, 128, NT, group_m, chunk);
      }
      for (int G : {8, 256, 512}) persistent_walk(L, NT, group_m, G);
    }
  }
  std::printf("ok: T=%d N=%d K=%d Ns=%d rows=%d tiles=%d of %lld pairs=%d of %lld\n", T, N, K, Ns,
              L.seg_off.back(), L.seg_off.back() / 128, (long long)max_tiles, L.pair_off.back(),
              (long long)L.max_pairs);
  return 0;
}
