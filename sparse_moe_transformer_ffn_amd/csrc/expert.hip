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

// tp[g] = sum_{g' < g} ceil(rows(g') / BM), tp[G] = total, in LDS.  256
// threads, G <= 1024 (four groups per thread).  Returns the total.
template <int BM>
__device__ int tile_prefix(int* tp, int* wsum, const int32_t* __restrict__ offsets, int G, int T) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  int cnt[4], local = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int g = tid * 4 + q;
    int rows = 0;
    if (g < G) rows = offsets ? offsets[g + 1] - offsets[g] : T;
    cnt[q] = (rows + BM - 1) / BM;
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
  for (int q = 0; q < 4; ++q) {
    const int g = tid * 4 + q;
    if (g < G) tp[g] = run;
    run += cnt[q];
  }
  if (tid == 0) tp[G] = total;
  __syncthreads();
  return total;
}

struct Item {
  int group, nt, m0, row0, nrows;
};

// Item w -> (group, N-tile, first row).  Groups with no tile are skipped by
// taking the largest g with tp[g] <= w / NT.
__device__ __forceinline__ Item decode_item(const int* tp, int G, int NT, int BM, int w,
                                            const int32_t* __restrict__ offsets, int T) {
  const int q = w / NT;
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tp[mid] <= q) lo = mid;
    else hi = mid - 1;
  }
  Item it;
  it.group = lo;
  const int tiles = tp[lo + 1] - tp[lo];
  const int wl = w - NT * tp[lo];
  it.nt = wl / tiles;
  it.m0 = (wl - it.nt * tiles) * BM;
  it.row0 = offsets ? offsets[lo] : 0;
  it.nrows = offsets ? offsets[lo + 1] - it.row0 : T;
  return it;
}

}  // namespace

// Phase 1.  GATHER: rows are permuted pairs (token = perm_pairs[row] / k);
// otherwise row r is token r (shared expert, one group).
template <int BM, bool GATHER>
__global__ __launch_bounds__(256) void k_gate_up(const uint16_t* __restrict__ x, const int32_t* __restrict__ offsets,
                                                 const int32_t* __restrict__ perm, int G, int T, int d, int h,
                                                 int k_top, const uint16_t* __restrict__ w_gu,
                                                 uint16_t* __restrict__ hid) {
  __shared__ int tp[1025];
  __shared__ int wsum[4];
  constexpr int MB = BM / 16;
  const int total_m = tile_prefix<BM>(tp, wsum, offsets, G, T);
  const int NT = h / 64;
  const int items = total_m * NT;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int r16 = lane & 15, kq = lane >> 4;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int w = xcd_contiguous(blockIdx.x, gridDim.x); w < items; w += gridDim.x) {
    const Item it = decode_item(tp, G, NT, BM, w, offsets, T);
    const int j = it.nt * 64 + wave * 16 + r16;
    const uint16_t* wbase = w_gu + (size_t)it.group * 2 * h * d;
    const uint16_t* pg = wbase + (size_t)j * d + kq * 8;
    const uint16_t* pu = wbase + (size_t)(h + j) * d + kq * 8;
    const uint16_t* pa[MB];
    bool va[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = it.m0 + mb * 16 + r16;
      va[mb] = r < it.nrows;
      int tok = 0;
      if (va[mb]) tok = GATHER ? perm[it.row0 + r] / k_top : r;
      pa[mb] = x + (size_t)tok * d + kq * 8;
    }
    f32x4 ag[MB], au[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      ag[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
      au[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll 4
    for (int kk = 0; kk < d; kk += 32) {
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
          hid[(size_t)(it.row0 + r) * h + j] = (uint16_t)f32_to_bf16(silu(g) * u);
        }
      }
    }
  }
}

// Phase 2: out[row, n] = sum_j hid[row, j] * w_down[group][n, j].
template <int BM, bool OUT_F32>
__global__ __launch_bounds__(256) void k_down(const int32_t* __restrict__ offsets, int G, int T, int d, int h,
                                              const uint16_t* __restrict__ hid, const uint16_t* __restrict__ w_down,
                                              void* __restrict__ out) {
  __shared__ int tp[1025];
  __shared__ int wsum[4];
  constexpr int MB = BM / 16;
  const int total_m = tile_prefix<BM>(tp, wsum, offsets, G, T);
  const int NT = d / 64;
  const int items = total_m * NT;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int r16 = lane & 15, kq = lane >> 4;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int w = xcd_contiguous(blockIdx.x, gridDim.x); w < items; w += gridDim.x) {
    const Item it = decode_item(tp, G, NT, BM, w, offsets, T);
    const int n = it.nt * 64 + wave * 16 + r16;
    const uint16_t* pb = w_down + (size_t)it.group * d * h + (size_t)n * h + kq * 8;
    const uint16_t* pa[MB];
    bool va[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = it.m0 + mb * 16 + r16;
      va[mb] = r < it.nrows;
      pa[mb] = hid + (size_t)(it.row0 + (va[mb] ? r : 0)) * h + kq * 8;
    }
    f32x4 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int kk = 0; kk < h; kk += 32) {
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
          if (OUT_F32) static_cast<float*>(out)[o] = acc[mb][i];
          else static_cast<uint16_t*>(out)[o] = (uint16_t)f32_to_bf16(acc[mb][i]);
        }
      }
    }
  }
}

namespace {

constexpr int kPersistentBlocks = 1024;  // 256 CUs x 4 resident blocks

int pick_bm(int T, int k, int G) {
  // Average rows per group decides the M-tile: 16 for decode-sized batches.
  const long rows = (long)T * k;
  return rows <= 16L * G ? 16 : 32;
}

}  // namespace

hipError_t launch_gate_up(int T, int d, int E, int k, int h, const uint16_t* x, const int32_t* offsets,
                          const int32_t* perm, const uint16_t* w_gu, uint16_t* hid, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 grid(kPersistentBlocks), block(256);
  if (pick_bm(T, k, E) == 16)
    hipLaunchKernelGGL((k_gate_up<16, true>), grid, block, 0, stream, x, offsets, perm, E, T, d, h, k, w_gu, hid);
  else
    hipLaunchKernelGGL((k_gate_up<32, true>), grid, block, 0, stream, x, offsets, perm, E, T, d, h, k, w_gu, hid);
  return hipGetLastError();
}

hipError_t launch_down(int T, int d, int E, int k, int h, const int32_t* offsets, const uint16_t* hid,
                       const uint16_t* w_down, uint16_t* y_perm, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 grid(kPersistentBlocks), block(256);
  if (pick_bm(T, k, E) == 16)
    hipLaunchKernelGGL((k_down<16, false>), grid, block, 0, stream, offsets, E, T, d, h, hid, w_down, y_perm);
  else
    hipLaunchKernelGGL((k_down<32, false>), grid, block, 0, stream, offsets, E, T, d, h, hid, w_down, y_perm);
  return hipGetLastError();
}

hipError_t launch_shared(int T, int d, int hs, const uint16_t* x, const uint16_t* ws_gu, const uint16_t* ws_d,
                         float* y_shared, uint16_t* hid, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 grid(kPersistentBlocks), block(256);
  if (T <= 16) {
    hipLaunchKernelGGL((k_gate_up<16, false>), grid, block, 0, stream, x, nullptr, nullptr, 1, T, d, hs, 1, ws_gu,
                       hid);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((k_down<16, true>), grid, block, 0, stream, nullptr, 1, T, d, hs, hid, ws_d, y_shared);
  } else {
    hipLaunchKernelGGL((k_gate_up<32, false>), grid, block, 0, stream, x, nullptr, nullptr, 1, T, d, hs, 1, ws_gu,
                       hid);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((k_down<32, true>), grid, block, 0, stream, nullptr, 1, T, d, hs, hid, ws_d, y_shared);
  }
  return hipGetLastError();
}

size_t expert_workspace_bytes(int T, int k, int h) { return (size_t)T * k * h * sizeof(uint16_t); }
size_t shared_workspace_bytes(int T, int hs) { return (size_t)T * hs * sizeof(uint16_t); }

}  // namespace moe
