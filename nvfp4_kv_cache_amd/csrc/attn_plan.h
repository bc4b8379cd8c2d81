// Work list of one chunk-attention launch (stream-K style): tile counts, cost
// weights and the cut of the weighted (query block, key tile) list into one equal
// share per workgroup.  Plain C++: the kernel includes it with NVFP4KV_PLAN_FN set
// to a host+device qualifier, and a CPU test of the partition builds it with g++.
#pragma once

#include "../../include/nvfp4kv.h"
#include "nvfp4kv_internal.h"

#ifndef NVFP4KV_PLAN_FN
#define NVFP4KV_PLAN_FN inline
#endif

namespace nvfp4kv {

constexpr int kAttnKeys = 64;   // keys per tile

// Tile counts and weights of `a` (its segments, n_q and H set); returns the grid
// (at most max_grid workgroups, at least 1) or a negative status.
//
// Per query block the tiles are: the cache's full tiles, the cache segments' ragged
// tails, the own segment's full tiles, its ragged tail.  Weights are measured
// relative costs: a pipelined NVFP4 tile 16, a pipelined bf16 own tile 14 (no
// dequantization), a ragged tail 28 (not pipelined).  Every share must hold at least
// one tile start, so the grid is at most the total weight over the largest weight.
NVFP4KV_PLAN_FN int64_t attn_plan(AttnArgs &a, int block_queries, int64_t max_grid) {
  int nf = 0, nt = 0;
  for (int i = 0; i < a.n_seg; ++i) {
    nf += a.seg[i].ntok / kAttnKeys;
    nt += a.seg[i].ntok % kAttnKeys ? 1 : 0;
  }
  a.n_cfull = nf;
  a.n_ctail = nt;
  a.n_ofull = a.n_q / kAttnKeys;
  a.n_otail = a.n_q % kAttnKeys ? 1 : 0;
  a.tiles = nf + nt + a.n_ofull + a.n_otail;
  a.w_cfull = 16;
  a.w_ofull = 14;
  a.w_tail = 28;
  const int64_t wb = int64_t(nf) * a.w_cfull + int64_t(nt + a.n_otail) * a.w_tail + int64_t(a.n_ofull) * a.w_ofull;
  if (wb >= (int64_t(1) << 31)) return NVFP4KV_EINVAL;
  a.w_block = int32_t(wb);
  const int64_t blocks = int64_t((a.n_q + block_queries - 1) / block_queries) * a.H;
  if (blocks >= (int64_t(1) << 31)) return NVFP4KV_EINVAL;
  if (blocks * wb >= (int64_t(1) << 52)) return NVFP4KV_EINVAL;   // share bounds U g / G in int64
  a.work = blocks * wb;
  int64_t grid = max_grid;
  const int64_t wmax = a.w_tail;   // the largest weight
  if (grid > a.work / wmax) grid = a.work / wmax;
  if (grid < 1) grid = 1;
  return grid;
}

// Workgroup whose share [U g / G, U (g+1) / G) holds weighted position x.
NVFP4KV_PLAN_FN int owner_of(int64_t x, int64_t U, int G) {
  return int(((x + 1) * G + U - 1) / U) - 1;
}

// Number of a query block's tiles that start before weighted position x (0 <= x <=
// the block's weight), in the order above.
NVFP4KV_PLAN_FN int tiles_before(const AttnArgs &a, int x) {
  int n = 0;
  auto part = [&](int count, int w) {
    const int span = count * w;
    n += x >= span ? count : (x + w - 1) / w;
    x = x - span > 0 ? x - span : 0;
  };
  part(a.n_cfull, a.w_cfull);
  part(a.n_ctail, a.w_tail);
  part(a.n_ofull, a.w_ofull);
  part(a.n_otail, a.w_tail);
  return n;
}

// The next range of a workgroup's share [ubeg, u), walked from its end: the tiles
// [t0, t1) of query block b that start inside the share's part of that block, with
// u moved to the part's start.  False once the share is used up.  A share usually
// holds the first tiles of one block and the last tiles of the one before, so a
// workgroup's first range starts at key tile 0.
NVFP4KV_PLAN_FN bool next_range(const AttnArgs &a, int64_t ubeg, int64_t &u, int &b, int &t0, int &t1) {
  const int64_t WB = a.w_block;
  while (u > ubeg) {
    const int64_t b64 = (u - 1) / WB;
    const int p1 = int(u - b64 * WB);
    const int p0 = int(ubeg - b64 * WB > 0 ? ubeg - b64 * WB : 0);
    u = b64 * WB + p0;
    t0 = tiles_before(a, p0);
    t1 = tiles_before(a, p1);
    if (t0 < t1) {
      b = int(b64);
      return true;
    }
  }
  return false;
}

}  // namespace nvfp4kv
