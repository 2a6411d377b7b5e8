// How the tiled prefill GEMM's work items are split over the 8 XCDs of
// gfx950, shared by the GEMM (which can resolve its own item) and the
// grouping kernels (which resolve every workgroup's item ahead of it).
//
// Items are (expert e, row stripe s, token tile q) in expert-major order,
// token tile fastest, so neighbouring items stream the same weight stripe.
// Hardware places workgroup b on XCD b % 8, and XCD x takes the contiguous
// item range [bx[x], bx[x+1]).  The ranges split the estimated work evenly
// rather than the item count, since the launch lasts as long as its busiest
// XCD: an item costs kTileCost (its weight stripe is streamed whatever its
// token count) plus its active 16-token sub-tiles.  The grid holds G
// workgroups per XCD, at least an eighth of the items, and no range holds
// more than G.
#pragma once

#include <stdint.h>

#include "launch.h"

namespace mxmoe {

// Token tile q of a group of c sorted rows (an expert's tokens): {first
// row within the group, rows}.  The group's ceil(c / kPrefillTokens) tiles
// share its ceil(c / 16) sub-tiles of 16 rows as evenly as they go (the
// first tiles one sub-tile more), so the tiles of one expert take about
// equally long and stream each weight stripe side by side, where a full
// tile followed by a short remainder would drift apart.
__host__ __device__ __forceinline__ int2 token_tile(int c, int q) {
  const int nt = (c + kPrefillTokens - 1) / kPrefillTokens, ns = (c + 15) >> 4;
  const int base = ns / nt, extra = ns - base * nt;  // at most 8 sub-tiles per tile
  const int first = 16 * (q * base + (q < extra ? q : extra));
  const int rows = 16 * (base + (q < extra ? 1 : 0));
  return make_int2(first, rows < c - first ? rows : c - first);
}

// Per-stripe cost of an expert with cnt tokens: kTileCost per token tile
// plus its ceil(cnt / 16) sub-tiles.
__device__ __forceinline__ int expert_stripe_cost(int cnt) {
  return kTileCost * ((cnt + kPrefillTokens - 1) / kPrefillTokens) + ((cnt + 15) >> 4);
}

// The 9 range bounds, in every lane of the calling wave.  woff: prefix of
// the experts' per-stripe costs (E + 1 entries), toff: prefix of their
// token tiles (E + 1), both readable by the wave (LDS); nvalid =
// toff[E] * nstripes <= 8 * G.
__device__ __forceinline__ void xcd_bounds(const int* woff, const int* toff, int E, int nstripes, int G, int nvalid,
                                           int lane, int (&bx)[9]) {
  // Lane xx <= 8 finds the first item of XCD xx: the first whose work
  // prefix reaches xx/8 of the total.  The prefix of item (expert j,
  // stripe s, tile q) is woff[j] * nstripes + s * (woff[j+1] - woff[j])
  // + P(q), P the cost of the expert's tiles before q: its first `extra`
  // tiles cost kTileCost + base + 1, the others kTileCost + base
  // (token_tile's even split of its sub-tiles).
  int bnd = nvalid;
  const int64_t W = int64_t(woff[E]) * nstripes;
  const int64_t target = (W * lane + 7) / 8;
  if (lane == 0) {
    bnd = 0;
  } else if (lane < 8 && target < W) {
    int lo = 0, hi = E;  // woff[lo] * nstripes <= target < woff[hi] * nstripes
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (int64_t(woff[mid]) * nstripes <= target) lo = mid;
      else hi = mid;
    }
    const int gc = woff[lo + 1] - woff[lo];  // > 0: the target lies in expert lo's range
    const int nt = toff[lo + 1] - toff[lo];
    const int64_t rem = target - int64_t(woff[lo]) * nstripes;
    const int st = int(rem / gc);
    const int r2 = int(rem - int64_t(st) * gc);
    // the first tile q with P(q) >= r2; past the last tile's start, the
    // next stripe's (or expert's) first item follows: index st * nt + nt
    const int nsub = gc - kTileCost * nt, base = nsub / nt, extra = nsub - base * nt;
    const int big = kTileCost + base + 1;  // cost of each of the first `extra` tiles
    const int q = min(r2 <= extra * big ? (r2 + big - 1) / big
                                        : extra + (r2 - extra * big + big - 2) / (big - 1),
                      nt);
    bnd = toff[lo] * nstripes + st * nt + q;
  }
  // No XCD may own more than G items: clamp forward, then backward from
  // nvalid.  Since nvalid <= 8 G, every range ends up within G.
#pragma unroll
  for (int xx = 0; xx < 9; ++xx) bx[xx] = __builtin_amdgcn_readlane(bnd, xx);
#pragma unroll
  for (int xx = 0; xx < 8; ++xx) bx[xx + 1] = min(max(bx[xx + 1], bx[xx]), bx[xx] + G);
  bx[8] = nvalid;
#pragma unroll
  for (int xx = 7; xx >= 1; --xx) bx[xx] = max(bx[xx], bx[xx + 1] - G);
}

}  // namespace mxmoe
