// expert.hip -- grouped SwiGLU expert GEMMs on bf16 MFMA (gfx950).
//
// Layer definition: [Digest] "Step 3.5 Flash 技术论文深度解读" architecture
// table (routed experts of hidden 1,280) and activation-explosion cause 3
// (SwiGLU gate and up projection branches); the grouped layout follows
// [Blog] "Step 3.5 Flash: Open Frontier-Level Intelligence with 11B Active
// Parameters" §3.2.4 (fused MoE gather/scatter with grouped GEMM).
//
// Work decomposition.  A "group" is one expert's rows of the permuted order
// (or all T tokens for the shared expert).  Each group is cut into M-tiles of
// BM rows; an item is (group, N-tile, M-tile) with the M-tile index fastest,
// so items that run side by side on one XCD read the same weight slab and the
// same group's activation rows through that XCD's L2.  Blocks are persistent:
// each builds the per-group tile prefix in LDS once from expert_offsets (no
// host round trip for the data-dependent group sizes) and strides over the
// items.  Block b's first item is chosen so that every XCD owns a contiguous
// range of items at each step.
//
// Phase 1 (gate/up): item = BM rows x 64 hidden units; each of the 4 waves
// owns 16 hidden units j and computes both G = X W_g[j]^T and U = X W_u[j]^T
// so that SwiGLU (SiLU(G) * U) is applied in registers before the bf16 store.
// Phase 2 (down): item = BM rows x 64 output columns, reduction over h.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kUnroll = 8;  // K steps (of 32) per batch of loads
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
// LDS; ip[G] = total.  256 threads, G <= kMaxGroups.  Returns the total.
template <int BM>
__device__ int item_prefix(int* ip, int* wsum, const Groups& gs, int nt_routed, int nt_shared) {
  constexpr int PER = (kMaxGroups + 255) / 256;
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
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  const int total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
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

// Item w -> (group, N-tile, first row), M-tile index fastest inside a group.
// Groups without items are skipped by taking the largest g with ip[g] <= w.
__device__ __forceinline__ Item decode_item(const int* ip, const Groups& gs, int BM, int w) {
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
  const int wl = w - ip[lo];
  it.nt = wl / tiles;
  it.m0 = (wl - it.nt * tiles) * BM;
  return it;
}

}  // namespace

// Phase 1: hid[row, j] = SiLU(x_row . W_g[j]) * (x_row . W_u[j]) for the
// item's BM rows and 64 hidden units j.  Routed rows gather their token via
// perm_pairs; shared rows are tokens in order.
template <int BM>
__global__ __launch_bounds__(256) void k_gate_up(const uint16_t* __restrict__ x, Groups gs, int d, int h, int hs,
                                                 const uint16_t* __restrict__ w_gu,
                                                 const uint16_t* __restrict__ ws_gu, uint16_t* __restrict__ hid,
                                                 uint16_t* __restrict__ hid_shared) {
  __shared__ int ip[kMaxGroups + 1];
  __shared__ int wsum[4];
  constexpr int MB = BM / 16;
  const int items = item_prefix<BM>(ip, wsum, gs, h / 64, hs / 64);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int r16 = lane & 15, kq = lane >> 4;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int w = xcd_contiguous(blockIdx.x, gridDim.x); w < items; w += gridDim.x) {
    const Item it = decode_item(ip, gs, BM, w);
    const int H = it.shared ? hs : h;
    const int j = it.nt * 64 + wave * 16 + r16;
    const uint16_t* wbase = it.shared ? ws_gu : w_gu + (size_t)it.group * 2 * h * d;
    uint16_t* out = it.shared ? hid_shared : hid;
    const uint16_t* pg = wbase + (size_t)j * d + kq * 8;
    const uint16_t* pu = wbase + (size_t)(H + j) * d + kq * 8;
    const uint16_t* pa[MB];
    bool va[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = it.m0 + mb * 16 + r16;
      va[mb] = r < it.nrows;
      int tok = 0;
      if (va[mb]) tok = it.shared ? r : gs.perm[it.row0 + r] / gs.k;
      pa[mb] = x + (size_t)tok * d + kq * 8;
    }
    f32x4 ag[MB], au[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      ag[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
      au[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // K in batches of kUnroll steps: every load of a batch is issued before
    // its MFMAs, so each wave keeps kUnroll weight rows' worth of requests in
    // flight (the streaming regime is latency x bandwidth bound).
    int kk = 0;
    for (; kk + 32 * kUnroll <= d; kk += 32 * kUnroll) {
      u32x4 bg[kUnroll], bu[kUnroll], a[MB][kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        bg[u] = load16(pg + kk + 32 * u);
        bu[u] = load16(pu + kk + 32 * u);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) a[mb][u] = va[mb] ? load16(pa[mb] + kk + 32 * u) : zero;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          ag[mb] = mfma_16x16x32(a[mb][u], bg[u], ag[mb]);
          au[mb] = mfma_16x16x32(a[mb][u], bu[u], au[mb]);
        }
    }
    for (; kk < d; kk += 32) {
      const u32x4 bg = load16(pg + kk);
      const u32x4 bu = load16(pu + kk);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const u32x4 a = va[mb] ? load16(pa[mb] + kk) : zero;
        ag[mb] = mfma_16x16x32(a, bg, ag[mb]);
        au[mb] = mfma_16x16x32(a, bu, au[mb]);
      }
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = it.m0 + mb * 16 + kq * 4 + i;
        if (r < it.nrows) {
          const float g = ag[mb][i], u = au[mb][i];
          out[(size_t)(it.row0 + r) * H + j] = (uint16_t)f32_to_bf16(silu(g) * u);
        }
      }
    }
  }
}

// Phase 2: out[row, n] = hid[row, :] . W_d[n, :] for the item's BM rows and 64
// output columns n; routed rows -> y_perm (bf16), shared rows -> y_shared (f32).
template <int BM>
__global__ __launch_bounds__(256) void k_down(Groups gs, int d, int h, int hs, const uint16_t* __restrict__ hid,
                                              const uint16_t* __restrict__ hid_shared,
                                              const uint16_t* __restrict__ w_down,
                                              const uint16_t* __restrict__ ws_down, uint16_t* __restrict__ y_perm,
                                              float* __restrict__ y_shared) {
  __shared__ int ip[kMaxGroups + 1];
  __shared__ int wsum[4];
  constexpr int MB = BM / 16;
  const int items = item_prefix<BM>(ip, wsum, gs, d / 64, d / 64);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int r16 = lane & 15, kq = lane >> 4;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int w = xcd_contiguous(blockIdx.x, gridDim.x); w < items; w += gridDim.x) {
    const Item it = decode_item(ip, gs, BM, w);
    const int H = it.shared ? hs : h;
    const int n = it.nt * 64 + wave * 16 + r16;
    const uint16_t* pb = (it.shared ? ws_down : w_down + (size_t)it.group * d * h) + (size_t)n * H + kq * 8;
    const uint16_t* src = it.shared ? hid_shared : hid;
    const uint16_t* pa[MB];
    bool va[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = it.m0 + mb * 16 + r16;
      va[mb] = r < it.nrows;
      pa[mb] = src + (size_t)(it.row0 + (va[mb] ? r : 0)) * H + kq * 8;
    }
    f32x4 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    int kk = 0;
    for (; kk + 32 * kUnroll <= H; kk += 32 * kUnroll) {
      u32x4 b[kUnroll], a[MB][kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) b[u] = load16(pb + kk + 32 * u);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) a[mb][u] = va[mb] ? load16(pa[mb] + kk + 32 * u) : zero;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[mb] = mfma_16x16x32(a[mb][u], b[u], acc[mb]);
    }
    for (; kk < H; kk += 32) {
      const u32x4 b = load16(pb + kk);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const u32x4 a = va[mb] ? load16(pa[mb] + kk) : zero;
        acc[mb] = mfma_16x16x32(a, b, acc[mb]);
      }
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = it.m0 + mb * 16 + kq * 4 + i;
        if (r < it.nrows) {
          const size_t o = (size_t)(it.row0 + r) * d + n;
          if (it.shared) y_shared[o] = acc[mb][i];
          else y_perm[o] = (uint16_t)f32_to_bf16(acc[mb][i]);
        }
      }
    }
  }
}

namespace {

constexpr int kMaxDevices = 64;

// Persistent grid: as many blocks as can be resident at once on the current
// device (occupancy x compute units), so that no block starts late and every
// block strides over its share of the items.  Cached per kernel and device.
template <class Kernel>
int persistent_grid(Kernel kernel) {
  static int cache[kMaxDevices] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  if (cache[dev] == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0) != hipSuccess || per_cu < 1)
      per_cu = 1;
    cache[dev] = cus * per_cu;
  }
  return cache[dev];
}

int pick_bm(int T, int k, int E) {
  // Average rows per routed group decides the M-tile: 16 for decode-sized
  // batches.
  const long rows = (long)T * k;
  return rows <= 16L * E ? 16 : 32;
}

template <int BM>
hipError_t gate_up_bm(const uint16_t* x, const Groups& gs, int d, int h, int hs, const uint16_t* w_gu,
                      const uint16_t* ws_gu, uint16_t* hid, uint16_t* hid_shared, hipStream_t stream) {
  const auto kern = k_gate_up<BM>;
  hipLaunchKernelGGL(kern, dim3(persistent_grid(kern)), dim3(256), 0, stream, x, gs, d, h, hs, w_gu, ws_gu, hid,
                     hid_shared);
  return hipGetLastError();
}

template <int BM>
hipError_t down_bm(const Groups& gs, int d, int h, int hs, const uint16_t* hid, const uint16_t* hid_shared,
                   const uint16_t* w_down, const uint16_t* ws_down, uint16_t* y_perm, float* y_shared,
                   hipStream_t stream) {
  const auto kern = k_down<BM>;
  hipLaunchKernelGGL(kern, dim3(persistent_grid(kern)), dim3(256), 0, stream, gs, d, h, hs, hid, hid_shared, w_down,
                     ws_down, y_perm, y_shared);
  return hipGetLastError();
}

Groups make_groups(int T, int E, int k, const int32_t* offsets, const int32_t* perm, bool shared) {
  Groups gs;
  gs.offsets = offsets;
  gs.perm = perm;
  gs.E = E;
  gs.k = k;
  gs.T = T;
  gs.shared = shared;
  return gs;
}

}  // namespace

hipError_t launch_gate_up(int T, int d, int E, int k, int h, int hs, const uint16_t* x, const int32_t* offsets,
                          const int32_t* perm, const uint16_t* w_gu, const uint16_t* ws_gu, uint16_t* hid,
                          uint16_t* hid_shared, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const Groups gs = make_groups(T, E, k, offsets, perm, ws_gu != nullptr);
  if (pick_bm(T, k, offsets ? E : 1) == 16)
    return gate_up_bm<16>(x, gs, d, h, hs, w_gu, ws_gu, hid, hid_shared, stream);
  return gate_up_bm<32>(x, gs, d, h, hs, w_gu, ws_gu, hid, hid_shared, stream);
}

hipError_t launch_down(int T, int d, int E, int k, int h, int hs, const int32_t* offsets, const uint16_t* hid,
                       const uint16_t* hid_shared, const uint16_t* w_down, const uint16_t* ws_down, uint16_t* y_perm,
                       float* y_shared, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const Groups gs = make_groups(T, E, k, offsets, nullptr, ws_down != nullptr);
  if (pick_bm(T, k, offsets ? E : 1) == 16)
    return down_bm<16>(gs, d, h, hs, hid, hid_shared, w_down, ws_down, y_perm, y_shared, stream);
  return down_bm<32>(gs, d, h, hs, hid, hid_shared, w_down, ws_down, y_perm, y_shared, stream);
}

size_t expert_hid_bytes(int T, int k, int h) { return ((size_t)T * k * h * sizeof(uint16_t) + 255) / 256 * 256; }
size_t shared_hid_bytes(int T, int hs) { return ((size_t)T * hs * sizeof(uint16_t) + 255) / 256 * 256; }

}  // namespace moe
