// grouped.h -- work decomposition shared by the grouped expert kernels.
//
// A "group" is one routed expert's rows of the permuted order (rows
// expert_offsets[g] .. expert_offsets[g+1], token = perm_pairs[row] / k) or,
// as group E, the shared expert's rows (every token in order).  Each group is
// cut into M-tiles; an item is (group, N-tile, M-tile), ordered so that
// neighbouring items share an operand (see decode_item).  Each block builds
// the per-group item prefix in LDS once from expert_offsets (no host round
// trip for the data-dependent group sizes) and then strides over the items;
// how items map to blocks and XCDs is up to each kernel.
#pragma once
#include <mutex>

#include "common.h"

namespace moe {

constexpr int kMaxGroups = 1280;

// The groups of one grouped launch: routed experts 0..E-1 (rows
// expert_offsets[g] .. expert_offsets[g+1] of the permuted order, token =
// perm_pairs[row] / k) and, if `shared`, one more group E holding every token
// in order (the shared expert, hidden size hs).
struct Groups {
  const int32_t* offsets;  // [E+1], NULL: no routed groups
  const int32_t* perm;
  int E, k, T;
  bool shared;
  __host__ __device__ int count() const { return (offsets ? E : 0) + (shared ? 1 : 0); }
};

struct GroupView {
  bool shared;
  int row0, nrows;
};

__device__ __forceinline__ GroupView group_view(const Groups& gs, int g) {
  GroupView v;
  v.shared = !gs.offsets || g >= gs.E;
  v.row0 = v.shared ? 0 : gs.offsets[g];
  v.nrows = v.shared ? gs.T : gs.offsets[g + 1] - v.row0;
  return v;
}

// ip[g] = number of items of the groups before g (an item is one BM-row
// M-tile times one N-tile; N-tiles per group: nt_routed or nt_shared), in
// LDS; ip[G] = total.  NTHREADS threads (a multiple of 64), G <= kMaxGroups.
// Returns the total.  wsum needs NTHREADS / 64 entries.
template <int BM, int NTHREADS = 256>
__device__ int item_prefix(int* ip, int* wsum, const Groups& gs, int nt_routed, int nt_shared) {
  constexpr int PER = (kMaxGroups + NTHREADS - 1) / NTHREADS;
  constexpr int NW = NTHREADS / kWave;
  const int G = gs.count();
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  int cnt[PER], local = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int g = tid * PER + q;
    cnt[q] = 0;
    if (g < G) {
      const GroupView v = group_view(gs, g);
      cnt[q] = (v.nrows + BM - 1) / BM * (v.shared ? nt_shared : nt_routed);
    }
    local += cnt[q];
  }
  int incl = local;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    base += w < wave ? wsum[w] : 0;
    total += wsum[w];
  }
  int run = base + incl - local;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int g = tid * PER + q;
    if (g < G) ip[g] = run;
    run += cnt[q];
  }
  if (tid == 0) ip[G] = total;
  __syncthreads();
  return total;
}

struct Item {
  int group, nt, m0, row0, nrows;
  bool shared;
};

// Item w -> (group, N-tile, first row).  Groups without items are skipped by
// taking the largest g with ip[g] <= w.  Inside a group, items are ordered in
// bands of up to BAND M-tiles: band by band, N-tile by N-tile, and the band's
// M-tiles fastest.  Items that run side by side on one XCD then share one
// weight slab (read from HBM once, the other M-tiles of the band hit L2) and
// at most BAND M-tiles of token rows.  BAND = 0 means one band of all M-tiles.
template <int BAND>
__device__ __forceinline__ Item decode_item(const int* ip, const Groups& gs, int BM, int nt_routed, int nt_shared,
                                            int w) {
  int lo = 0, hi = gs.count() - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (ip[mid] <= w) lo = mid;
    else hi = mid - 1;
  }
  const GroupView v = group_view(gs, lo);
  Item it;
  it.group = lo;
  it.shared = v.shared;
  it.row0 = v.row0;
  it.nrows = v.nrows;
  const int tiles = (v.nrows + BM - 1) / BM;
  const int nt = v.shared ? nt_shared : nt_routed;
  const int wl = w - ip[lo];
  const int band = BAND > 0 ? BAND : tiles;
  const int b = wl / (band * nt);                 // band index
  const int in_band = min(band, tiles - b * band);  // M-tiles in this band
  const int r = wl - b * band * nt;
  it.nt = r / in_band;
  it.m0 = (b * band + (r - it.nt * in_band)) * BM;
  return it;
}

// Item w -> (group, N-tile, first row) for kernels whose item w runs on XCD
// w mod 8 (item w to block w mod grid, grid a multiple of 8, block b on XCD
// b mod 8).  Inside a group the items go in runs of 8 N-tiles (fewer in the
// last run) times all M-tiles, N-tile fastest: the M-tiles of one N-tile get
// item numbers 8 apart, so they run side by side on one XCD and its L2 fetches
// their weight rows from HBM once for all of them.  A group of one M-tile
// keeps N-tile order.
__device__ __forceinline__ Item decode_item_xcd(const int* ip, const Groups& gs, int BM, int nt_routed, int nt_shared,
                                                int w) {
  int lo = 0, hi = gs.count() - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (ip[mid] <= w) lo = mid;
    else hi = mid - 1;
  }
  const GroupView v = group_view(gs, lo);
  Item it;
  it.group = lo;
  it.shared = v.shared;
  it.row0 = v.row0;
  it.nrows = v.nrows;
  const int tiles = (v.nrows + BM - 1) / BM;
  const int nt = v.shared ? nt_shared : nt_routed;
  const int wl = w - ip[lo];
  const int run = wl / (8 * tiles);
  const int r = wl - run * 8 * tiles;
  const int span = min(8, nt - run * 8);  // N-tiles in this run
  it.nt = run * 8 + r % span;
  it.m0 = (r / span) * BM;
  return it;
}

// Persistent grid: as many blocks as can be resident at once on the current
// device (occupancy x compute units); a kernel launches this many, or a
// multiple of it when it wants the dispatcher to balance the tail.  Cached
// per kernel (by address:
// instances of one kernel template share a type but not their occupancy) and
// device.
struct GridCacheEntry {
  const void* kernel;
  int device;
  int block_threads;
  int grid;
};

inline int persistent_grid_of(const void* kernel, int block_threads) {
  static std::mutex mu;
  static GridCacheEntry cache[64];
  static int used = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < used; ++i)
    if (cache[i].kernel == kernel && cache[i].device == dev && cache[i].block_threads == block_threads)
      return cache[i].grid;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block_threads, 0) != hipSuccess || per_cu < 1)
    per_cu = 1;
  const int grid = cus * per_cu;
  if (used < 64) cache[used++] = GridCacheEntry{kernel, dev, block_threads, grid};
  return grid;
}

template <class Kernel>
int persistent_grid(Kernel kernel, int block_threads = 256) {
  return persistent_grid_of(reinterpret_cast<const void*>(kernel), block_threads);
}

inline Groups make_groups(int T, int E, int k, const int32_t* offsets, const int32_t* perm, bool shared) {
  Groups gs;
  gs.offsets = offsets;
  gs.perm = perm;
  gs.E = E;
  gs.k = k;
  gs.T = T;
  gs.shared = shared;
  return gs;
}

}  // namespace moe
