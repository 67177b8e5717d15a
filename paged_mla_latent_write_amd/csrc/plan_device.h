// Device body of the split plan, shared by the standalone plan kernel
// (attn_common.hip) and the absorb kernel, which runs it in one extra
// workgroup so that the plan costs no launch of its own (head_gemm.hip).
#pragma once

#include "mla_internal.h"

namespace mla {

constexpr int kPlanLds = 4096;  // tile_start / wg_tile entries mirrored in LDS

// The split plan (one workgroup of NT threads; the caller supplies the LDS
// arrays: buf[NT], carry, and ts_lds / wt_lds of kPlanLds entries each).
// The binary searches read tile_start and wg_tile from the LDS copies when
// they fit (each probe of a global copy written here is a full memory round
// trip).
template <int NT>
__device__ __forceinline__ void plan_items_body(
    int32_t* buf, int32_t* carry, int32_t* ts_lds, int32_t* wt_lds,
    int mode, int32_t B, int32_t Nq, const int32_t* __restrict__ ctx,
    const int32_t* __restrict__ qsl, int32_t window, int32_t max_ctx, int32_t* __restrict__ item_b,
    int32_t* __restrict__ item_lo, int32_t* __restrict__ item_hi,
    int32_t* __restrict__ tile_start, int32_t G, int32_t* __restrict__ wg_tile,
    int32_t* __restrict__ wg_item, int32_t* __restrict__ item_wg) {
  const bool ts_fits = Nq + 1 <= kPlanLds, wt_fits = G + 1 <= kPlanLds;
  const int tid = threadIdx.x;
  if (tid == 0) (*carry) = 0;
  // (prefill) query_start_loc for the per-row request search, in the space
  // wg_tile takes later
  const bool qsl_fits = mode != kPlanDecode && B + 1 <= kPlanLds;
  if (qsl_fits)
    for (int b = tid; b <= B; b += NT) wt_lds[b] = qsl[b];
  __syncthreads();
  const int32_t* qsl_tab = qsl_fits ? wt_lds : qsl;
  for (int base = 0; base < Nq; base += NT) {
    const int i = base + tid;
    int32_t nt = 0;
    if (i < Nq) {
      int b, p;
      if (mode == kPlanDecode) {
        b = i;
        const int n = min(max(ctx[b], 0), max_ctx);
        p = n - 1;
      } else {
        int lo = 0, hi = B;  // largest b < B with qsl[b] <= i
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (qsl_tab[mid] <= i) lo = mid; else hi = mid;
        }
        b = lo;
        const int n = min(max(ctx[b], 0), max_ctx);
        const int m = qsl_tab[b + 1] - qsl_tab[b];
        p = min(n - m + (i - qsl_tab[b]), n - 1);
      }
      int lo_t = 0, hi_t = 0;
      if (p >= 0) {
        hi_t = p + 1;
        lo_t = window > 0 ? max(0, p - window + 1) : 0;
      }
      item_b[i] = b;
      item_lo[i] = lo_t;
      item_hi[i] = hi_t;
      nt = hi_t > lo_t ? (hi_t + kTile - 1) / kTile - lo_t / kTile : 0;
    }
    // inclusive scan over the block (Hillis-Steele)
    buf[tid] = nt;
    __syncthreads();
    for (int off = 1; off < NT; off <<= 1) {
      const int32_t add = tid >= off ? buf[tid - off] : 0;
      __syncthreads();
      buf[tid] += add;
      __syncthreads();
    }
    if (i < Nq) {
      tile_start[i] = (*carry) + buf[tid] - nt;
      if (ts_fits) ts_lds[i] = (*carry) + buf[tid] - nt;
    }
    __syncthreads();
    if (tid == NT - 1) (*carry) += buf[tid];
    __syncthreads();
  }
  if (tid == 0) {
    tile_start[Nq] = (*carry);
    if (ts_fits) ts_lds[Nq] = (*carry);
  }
  __syncthreads();
  const int32_t* ts_tab = ts_fits ? ts_lds : tile_start;
  // Workgroup ranges: the tile stream cut into G ranges of equal estimated
  // cost, a tile costing 1 and each item kSegmentCostTiles more.  On that
  // virtual axis item i starts at V_i = tile_start[i] + kSegmentCostTiles * i,
  // its surcharge first, then its tiles; a cut that falls in a surcharge moves
  // to the item's first tile (a range may then be empty).
  const int64_t W = (*carry);
  const int64_t VT = W + static_cast<int64_t>(kSegmentCostTiles) * Nq;
  for (int g = tid; g <= G; g += NT) {
    const int64_t vb = static_cast<int64_t>(g) * VT / G;
    int lo = 0, hi = Nq + 1;  // largest i <= Nq with V_i <= vb
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (ts_tab[mid] + static_cast<int64_t>(kSegmentCostTiles) * mid <= vb) lo = mid; else hi = mid;
    }
    const int64_t ts = ts_tab[lo];
    const int64_t n = lo < Nq ? ts_tab[lo + 1] - ts : 0;
    const int64_t into = vb - ts - static_cast<int64_t>(kSegmentCostTiles) * lo - kSegmentCostTiles;
    const int32_t t = static_cast<int32_t>(ts + min(max(into, int64_t{0}), n));
    wg_tile[g] = t;
    if (wt_fits) wt_lds[g] = t;
  }
  __syncthreads();
  const int32_t* wt_tab = wt_fits ? wt_lds : wg_tile;
  // Each workgroup's first item: the last item whose first tile is <= the
  // range's first tile (items with no tiles are skipped).
  for (int g = tid; g < G; g += NT) {
    const int32_t t = wt_tab[g];
    int lo = 0, hi = Nq;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (ts_tab[mid] <= t) lo = mid; else hi = mid;
    }
    wg_item[g] = lo;
  }
  // The first and last workgroup covering each item (equal when one workgroup
  // holds all of the item's tiles; both -1 for an item with no tiles): the
  // workgroup of tile t is the last g < G with wg_tile[g] <= t.
  for (int i = tid; i < Nq; i += NT) {
    const int32_t ts = ts_tab[i], te = ts_tab[i + 1];
    int32_t wgs[2] = {-1, -1};
    if (te > ts) {
      for (int e = 0; e < 2; ++e) {
        const int32_t t = e == 0 ? ts : te - 1;
        int lo = 0, hi = G;
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (wt_tab[mid] <= t) lo = mid; else hi = mid;
        }
        wgs[e] = lo;
      }
    }
    item_wg[2 * i] = wgs[0];
    item_wg[2 * i + 1] = wgs[1];
  }
}

}  // namespace mla
