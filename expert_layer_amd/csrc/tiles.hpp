// Persistent tile scheduler for the grouped expert GEMMs.
//
// Groups are the E routed experts plus (optionally) the shared expert as
// group E; group g owns slots [offsets[g], offsets[g+1]).  A group is cut into
// row chunks of at most `chunk_rows` rows; an item is (chunk, column tile).
// Every workgroup rebuilds the chunk prefix over groups in LDS from
// `offsets` (a few hundred integers), so the grid never depends on the
// routing result known only on the device: the grid is sized to fill the
// chip and each wave strides over the item list.
#pragma once

#include "common.hpp"

namespace moe355 {

constexpr int kMaxGroups = 1025;

struct ChunkTable {
  int prefix[kMaxGroups + 1];  // prefix[g] = chunks in groups < g
  int wsum[16];
};

// Build the chunk prefix for G groups.  Must be called by all threads of the
// workgroup (contains barriers).  Returns the total chunk count.
__device__ inline int build_chunks(ChunkTable& tab, const int32_t* __restrict__ offsets, int G,
                                   int chunk_rows) {
  const int nthreads = blockDim.x;
  const int per = (G + nthreads - 1) / nthreads;
  const int g0 = threadIdx.x * per;
  int local = 0;
  for (int g = g0; g < g0 + per && g < G; ++g) {
    const int rows = offsets[g + 1] - offsets[g];
    local += (rows + chunk_rows - 1) / chunk_rows;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int v = local;
  for (int off = 1; off < 64; off <<= 1) {
    const int n = __shfl_up(v, off);
    if (lane >= off) v += n;
  }
  if (lane == 63) tab.wsum[wave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < (nthreads + 63) / 64; ++w) {
      const int c = tab.wsum[w];
      tab.wsum[w] = run;
      run += c;
    }
    tab.prefix[G] = run;
  }
  __syncthreads();
  int run = v - local + tab.wsum[wave];
  for (int g = g0; g < g0 + per && g < G; ++g) {
    tab.prefix[g] = run;
    const int rows = offsets[g + 1] - offsets[g];
    run += (rows + chunk_rows - 1) / chunk_rows;
  }
  __syncthreads();
  return tab.prefix[G];
}

// The tiled Down kernels order their items with the shared expert's group
// (index E) first: slot vg of the order holds group vg - 1 (vg >= 1), slot 0
// the shared group, and prefix[] is built over that order.  The shared group
// is the largest one with full tiles, so the partly filled last round of
// items then holds small routed groups instead (Down 2-2.5 % faster; the
// Gate-Up kernels measured 1 % slower with it and keep the plain order).
__device__ __forceinline__ int sf_group(int vg, int E, int has_shared) {
  return has_shared ? (vg == 0 ? E : vg - 1) : vg;
}
__device__ inline int build_chunks_sf(ChunkTable& tab, const int32_t* __restrict__ offsets, int G, int E,
                                      int has_shared, int chunk_rows) {
  const int nthreads = blockDim.x;
  const int per = (G + nthreads - 1) / nthreads;
  const int g0 = threadIdx.x * per;
  int local = 0;
  for (int vg = g0; vg < g0 + per && vg < G; ++vg) {
    const int g = sf_group(vg, E, has_shared);
    const int rows = offsets[g + 1] - offsets[g];
    local += (rows + chunk_rows - 1) / chunk_rows;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int v = local;
  for (int off = 1; off < 64; off <<= 1) {
    const int n = __shfl_up(v, off);
    if (lane >= off) v += n;
  }
  if (lane == 63) tab.wsum[wave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < (nthreads + 63) / 64; ++w) {
      const int c = tab.wsum[w];
      tab.wsum[w] = run;
      run += c;
    }
    tab.prefix[G] = run;
  }
  __syncthreads();
  int run = v - local + tab.wsum[wave];
  for (int vg = g0; vg < g0 + per && vg < G; ++vg) {
    tab.prefix[vg] = run;
    const int g = sf_group(vg, E, has_shared);
    const int rows = offsets[g + 1] - offsets[g];
    run += (rows + chunk_rows - 1) / chunk_rows;
  }
  __syncthreads();
  return tab.prefix[G];
}

// Group owning chunk c: the last g with prefix[g] <= c (empty groups skipped).
__device__ inline int chunk_group(const ChunkTable& tab, int G, int c) {
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tab.prefix[mid] <= c)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// Order of a group's items: (row tile mt, column tile nt) of local item
// `local` among the group's mtg * NT.  Row tiles are taken in bands of BAND;
// inside a band the row tile varies fastest.  The 32 consecutive items one
// XCD runs in a round then cover BAND row tiles x 32 / BAND column tiles,
// whose operand slices that XCD's L2 serves to all of them, instead of every
// row tile of a large group against one or two column tiles.  Groups of at
// most BAND row tiles keep the plain row-fastest order.
constexpr int kBand = 4;   // row tiles per band of the tiled GEMMs' item order

template <int BAND>
__device__ inline void item_tile(int local, int mtg, int NT, int& mt, int& nt) {
  const int nb = mtg / BAND;              // full bands
  const int band_items = BAND * NT;
  const int band = local / band_items;
  if (band < nb) {
    const int r = local - band * band_items;
    mt = band * BAND + r % BAND;
    nt = r / BAND;
  } else {
    const int rem = mtg - nb * BAND;      // > 0 here
    const int r = local - nb * band_items;
    mt = nb * BAND + r % rem;
    nt = r / rem;
  }
}

// The Gate-Up tiled kernels' per-XCD round barrier keeps the row tiles that
// share a weight tile in step through L2.  It pays when groups average at
// least 1.5 row tiles (router shape, 2 tiles per group: 15 % faster with it);
// with about one tile per group (prefill) or fewer (the skewed fp8 shapes)
// the tiles share little and the waits cost 3-6 %, so it is left off.
inline bool round_barrier(const GemmArgs& a, int tile_rows) {
  return 2 * a.T * a.k >= (int64_t)3 * a.E * tile_rows;
}

// Groups of 64+ rows on average go to the LDS-tiled MFMA kernels; up to 16
// rows on average, the weight-streaming kernels use 16-row chunks.
inline bool large_groups(const GemmArgs& a) { return a.T * a.k >= (int64_t)a.E * 64; }
inline bool small_groups(const GemmArgs& a) { return a.T * a.k <= (int64_t)a.E * 16; }

}  // namespace moe355
