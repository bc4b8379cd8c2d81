// CPU check of the chunk-attention work list (csrc/attn_plan.h, the same header the
// kernel includes): over random cache shapes, query counts, head counts and grids,
//  - every workgroup's share holds at least one tile;
//  - the ranges of every query block, over all workgroups, cover its tiles exactly
//    once, held by consecutive workgroups in tile order;
//  - the workgroup holding a cut block's last tiles (the merger) finds the holders of
//    its earlier tiles at owner_of(block start) .. itself - 1;
//  - a workgroup holding a block's earlier tiles (a publisher) processes that range
//    first, and a merger range is the last range of its workgroup;
//  - owner_of maps every weighted position to the share that contains it.
// Usage: attn_partition <cases> <seed>; prints the number of failures.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../nvfp4_kv_cache_amd/csrc/attn_plan.h"

using namespace nvfp4kv;

static uint64_t rng_state;
static uint64_t rnd() {
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return rng_state;
}
static int pick(int lo, int hi) { return lo + int(rnd() % uint64_t(hi - lo + 1)); }

struct Range {
  int g, order, b, t0, t1;
};

static int failures = 0;
#define CHECK(cond, ...)                              \
  do {                                                \
    if (!(cond)) {                                    \
      if (failures < 20) {                            \
        printf("FAIL case %d: ", cs);                 \
        printf(__VA_ARGS__);                          \
        printf("\n");                                 \
      }                                               \
      ++failures;                                     \
    }                                                 \
  } while (0)

int main(int argc, char **argv) {
  const int cases = argc > 1 ? atoi(argv[1]) : 500;
  rng_state = argc > 2 ? strtoull(argv[2], nullptr, 10) * 2654435761ull + 1 : 88172645463325252ull;
  for (int cs = 0; cs < cases; ++cs) {
    AttnArgs a;
    memset(&a, 0, sizeof(a));
    a.H = pick(1, 32);
    a.n_seg = pick(0, 24);
    const int tpf = (rnd() & 1) ? 64 * pick(1, 30) : pick(1, 2000);
    for (int i = 0; i < a.n_seg; ++i) a.seg[i].ntok = (rnd() & 3) ? tpf * pick(1, 3) : pick(1, 5000);
    a.n_q = (rnd() & 3) ? pick(1, 6000) : 64 * pick(1, 80);
    const int bq = (rnd() & 1) ? 256 : 128;
    const int64_t max_grid = (rnd() & 3) ? (bq == 256 ? 256 : 512) : pick(1, 600);
    const int64_t G64 = attn_plan(a, bq, max_grid);
    CHECK(G64 >= 1 && G64 <= max_grid, "grid %lld", (long long)G64);
    if (G64 < 1) continue;
    const int G = int(G64);
    const int64_t U = a.work;
    const int T = a.tiles;
    const int blocks = int(U / a.w_block);
    CHECK(int64_t(blocks) * a.w_block == U, "work %lld not whole blocks", (long long)U);

    std::vector<Range> all;
    std::vector<int> nranges(G, 0);
    for (int g = 0; g < G; ++g) {
      const int64_t ubeg = U * g / G;
      int64_t u = U * (g + 1) / G;
      int b, t0, t1, k = 0;
      while (next_range(a, ubeg, u, b, t0, t1)) {
        CHECK(b >= 0 && b < blocks && 0 <= t0 && t0 < t1 && t1 <= T, "range b %d [%d,%d)", b, t0, t1);
        all.push_back({g, k++, b, t0, t1});
      }
      nranges[g] = k;
      CHECK(k >= 1, "workgroup %d of %d has no tile", g, G);
      // owner_of agrees with the share bounds
      for (int s = 0; s < 4; ++s) {
        const int64_t hi = U * (g + 1) / G;
        if (hi <= ubeg) break;
        const int64_t x = ubeg + int64_t(rnd() % uint64_t(hi - ubeg));
        CHECK(owner_of(x, U, G) == g, "owner_of(%lld) = %d, share %d", (long long)x, owner_of(x, U, G), g);
      }
    }
    // per block: ranges in workgroup order tile the block exactly
    std::vector<std::vector<Range>> per(blocks);
    for (const Range &r : all) per[r.b].push_back(r);
    for (int b = 0; b < blocks; ++b) {
      std::vector<Range> &v = per[b];
      CHECK(!v.empty(), "block %d has no range", b);
      if (v.empty()) continue;
      int next = 0, prev_g = -1;
      for (const Range &r : v) {   // `all` is in workgroup order, so v is too
        CHECK(r.t0 == next, "block %d: range [%d,%d) of wg %d after tile %d", b, r.t0, r.t1, r.g, next);
        CHECK(prev_g < 0 || r.g == prev_g + 1, "block %d: wg %d after wg %d", b, r.g, prev_g);
        next = r.t1;
        prev_g = r.g;
      }
      CHECK(next == T, "block %d covered up to tile %d of %d", b, next, T);
      const Range &last = v.back();
      const int gf = owner_of(int64_t(b) * a.w_block, U, G);
      CHECK(gf == v.front().g, "block %d: owner_of(start) %d, first holder %d", b, gf, v.front().g);
      if (v.size() > 1) {
        // merger: its range of this block is its last one
        CHECK(last.order == nranges[last.g] - 1, "block %d: merger wg %d range %d of %d", b, last.g, last.order,
              nranges[last.g]);
        // publishers: their range of this block is their first one
        for (size_t i = 0; i + 1 < v.size(); ++i)
          CHECK(v[i].order == 0, "block %d: publisher wg %d range %d", b, v[i].g, v[i].order);
      }
    }
  }
  printf("%d cases, %d failures\n", cases, failures);
  return failures ? 1 : 0;
}
