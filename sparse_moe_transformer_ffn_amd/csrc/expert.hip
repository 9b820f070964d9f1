// expert.hip -- grouped SwiGLU expert GEMMs on bf16 MFMA (gfx950).
//
// Layer definition: [Digest] "Step 3.5 Flash 技术论文深度解读" architecture
// table (routed experts of hidden 1,280) and activation-explosion cause 3
// (SwiGLU gate and up projection branches); the grouped layout follows
// [Blog] "Step 3.5 Flash: Open Frontier-Level Intelligence with 11B Active
// Parameters" §3.2.4 (fused MoE gather/scatter with grouped GEMM).
//
// These are the streaming-regime kernels (under 11 rows per expert on
// average, 10 for down: decode-sized and small batches; the dense FFN up to
// 64 tokens), where the weights are read once and the MFMA work is small:
// every wave loads its operands straight from HBM/L2 into registers, keeping
// a batch of 2 to 8 K-steps of weight rows in flight (6 at decode: the batch
// length trades bytes in flight per wave against waves per SIMD).  The item
// decomposition is in grouped.h.
//
// Phase 1 (gate/up): item = BM rows x 64 CPW hidden units (16 CPW with the
// reduction split over the four waves); each wave computes both
// G = X W_g[j]^T and U = X W_u[j]^T for its units j so that SwiGLU
// (SiLU(G) * U) is applied in registers before the bf16 store.
// Phase 2 (down): item = BM rows x 64 CPW output columns (CPW groups of 16
// per wave), reduction over h.
#include "common.h"
#include "grouped.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kUnroll = 8;  // K steps (of 32) per batch of loads

// Blocks launched per resident block slot.  Item w goes to block w % grid and
// block b runs on XCD b % 8, so every round of items is spread over all eight
// XCDs (an XCD-contiguous order left the last, partial round on the first few
// XCDs); with eight blocks per slot the dispatcher hands the remaining blocks
// to whichever CU of an XCD frees first, which evens out the tail (decode
// gate/up with 2, 4, 8, 16 blocks per slot: 481, 476, 470, 469 us; down 251,
// 246, 245, 250 us).  Items of these kernels share no weights across XCDs,
// so nothing is lost in L2.
constexpr int kOversubscribe = 8;

// Weight rows are read as whole 128-byte lines with non-temporal loads: lane
// l reads 16 bytes of row l >> 3 (rows 8.. for `hi`) at segment l & 7 of a
// 64-wide K block, so one load covers 8 rows x 128 B and the 16 rows of a
// wave's operand take two loads per block.  The MFMA lane layout (row l & 15,
// 32 bytes per row per step) would split every line over two loads; with
// whole lines a plain read of this chip reaches 6.5-6.8 TB/s instead of
// 6.0-6.1, and gate/up at decode took 480 us instead of 543.  The lanes then
// trade data (ds_bpermute) into the MFMA layout; the weights are read once,
// so the non-temporal hint costs no reuse.
struct Lines {
  u32x4 lo, hi;  // rows 0-7 and 8-15 of one 64-wide K block
};

__device__ __forceinline__ Lines load_lines(const uint16_t* p8, size_t hi_off) {
  Lines L;
  L.lo = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p8));
  L.hi = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p8 + hi_off));
  return L;
}

// MFMA operand of K step s of the block (elements 32 s .. 32 s + 31): lane l
// gets row l & 15, elements 8 (l >> 4) .. +7 of the step, from lane
// ((l & 7) << 3) | ((l >> 4) + 4 s) of `lo` or `hi`.  addr = 4 x that lane;
// hi = (l & 15) >= 8.
__device__ __forceinline__ u32x4 lines_operand(const Lines& L, int addr, bool hi) {
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int v0 = __builtin_amdgcn_ds_bpermute(addr, (int)L.lo[q]);
    const int v1 = __builtin_amdgcn_ds_bpermute(addr, (int)L.hi[q]);
    o[q] = (uint32_t)(hi ? v1 : v0);
  }
  return o;
}

}  // namespace

// Phase 1: hid[row, j] = SiLU(x_row . W_g[j]) * (x_row . W_u[j]).  Routed
// rows gather their token via perm_pairs; shared rows are tokens in order.
// KW = 1: an item is BM rows x 64 CPW hidden units, wave w owns CPW groups of
//         16 units over the whole reduction.
// KW = 4: an item is BM rows x 16 CPW hidden units and wave w owns the w-th
//         quarter of the reduction; the four partial sums meet in LDS and are
//         added in wave order (a fixed order: results do not depend on the
//         schedule).  Items are four times smaller, so the last items of the
//         launch, which run alone, take a quarter of the time.
// UNR: K steps per batch of loads.
// CPW: groups of 16 hidden units per wave (their gate and up rows share each
//      load of token rows: with 64-row items the token operand would
//      otherwise be twice the weight bytes per wave).
template <int BM, int KW, bool CLAMP = false, int UNR = kUnroll, int CPW = 1>
__global__ __launch_bounds__(256) void k_gate_up(const uint16_t* __restrict__ x, Groups gs, int d, int h, int hs,
                                                 const uint16_t* __restrict__ w_gu,
                                                 const uint16_t* __restrict__ ws_gu, uint16_t* __restrict__ hid,
                                                 uint16_t* __restrict__ hid_shared, float clamp) {
  __shared__ int ip[kMaxGroups + 1];
  __shared__ int wsum[4];
  constexpr int MB = BM / 16;
  constexpr int UNITS = 64 * CPW / KW;  // hidden units per item
  __shared__ float red[KW > 1 ? KW - 1 : 1][2 * CPW * MB * 4][kWave];
  const int items = item_prefix<BM>(ip, wsum, gs, h / UNITS, hs / UNITS);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int r16 = lane & 15, kq = lane >> 4;
  const int klen = d / KW, kbeg = KW > 1 ? wave * klen : 0;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int w = (int)blockIdx.x; w < items; w += gridDim.x) {
    const Item it = decode_item_xcd(ip, gs, BM, h / UNITS, hs / UNITS, w);
    const int H = it.shared ? hs : h;
    // Unit of this lane in its first group; group c adds 16 c.
    const int j = it.nt * UNITS + (KW > 1 ? 0 : wave * 16 * CPW) + r16;
    const uint16_t* wbase = it.shared ? ws_gu : w_gu + (size_t)it.group * 2 * h * d;
    uint16_t* out = it.shared ? hid_shared : hid;
    const uint16_t* pg = wbase + (size_t)j * d + kbeg + kq * 8;
    const uint16_t* pu = wbase + (size_t)(H + j) * d + kbeg + kq * 8;
    // Whole-line loads of the same 16 gate and up rows (see load_lines).
    const int j8 = j - r16 + (lane >> 3);
    const uint16_t* pg8 = wbase + (size_t)j8 * d + kbeg + (lane & 7) * 8;
    const uint16_t* pu8 = wbase + (size_t)(H + j8) * d + kbeg + (lane & 7) * 8;
    const uint16_t* pa[MB];
    bool va[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = it.m0 + mb * 16 + r16;
      va[mb] = r < it.nrows;
      int tok = 0;
      if (va[mb]) tok = it.shared ? r : gs.perm[it.row0 + r] / gs.k;
      pa[mb] = x + (size_t)tok * d + kbeg + kq * 8;
    }
    f32x4 ag[CPW][MB], au[CPW][MB];
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        ag[c][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
        au[c][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    const int addr0 = 4 * (((lane & 7) << 3) | kq), addr1 = addr0 + 16;
    const bool hirow = r16 >= 8;
    // K in batches of UNR steps: every load of a batch is issued before
    // its MFMAs, so each wave keeps UNR weight rows' worth of requests in
    // flight (the streaming regime is latency x bandwidth bound).  A batch of
    // `steps` < UNR (an even count) takes the whole-line pairs left at the end.
    auto batch = [&](int kk, int steps) {
      Lines lg[CPW][UNR / 2], lu[CPW][UNR / 2];
#pragma unroll
      for (int b2 = 0; b2 < UNR / 2; ++b2)
        if (2 * b2 < steps) {
#pragma unroll
          for (int c = 0; c < CPW; ++c) {
            lg[c][b2] = load_lines(pg8 + (size_t)c * 16 * d + kk + 64 * b2, (size_t)8 * d);
            lu[c][b2] = load_lines(pu8 + (size_t)c * 16 * d + kk + 64 * b2, (size_t)8 * d);
          }
        }
      u32x4 a[MB][UNR];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int u = 0; u < UNR; ++u)
          if (u < steps) a[mb][u] = va[mb] ? load16(pa[mb] + kk + 32 * u) : zero;
#pragma unroll
      for (int u = 0; u < UNR; ++u)
        if (u < steps) {
#pragma unroll
          for (int c = 0; c < CPW; ++c) {
            const u32x4 bg = lines_operand(lg[c][u / 2], u % 2 ? addr1 : addr0, hirow);
            const u32x4 bu = lines_operand(lu[c][u / 2], u % 2 ? addr1 : addr0, hirow);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
              ag[c][mb] = mfma_16x16x32(a[mb][u], bg, ag[c][mb]);
              au[c][mb] = mfma_16x16x32(a[mb][u], bu, au[c][mb]);
            }
          }
        }
    };
    int kk = 0;
    for (; kk + 32 * UNR <= klen; kk += 32 * UNR) batch(kk, UNR);
    if (const int rest = (klen - kk) / 64 * 2) {
      batch(kk, rest);
      kk += 32 * rest;
    }
    for (; kk < klen; kk += 32) {
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        const u32x4 bg = load16(pg + (size_t)c * 16 * d + kk);
        const u32x4 bu = load16(pu + (size_t)c * 16 * d + kk);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const u32x4 a = va[mb] ? load16(pa[mb] + kk) : zero;
          ag[c][mb] = mfma_16x16x32(a, bg, ag[c][mb]);
          au[c][mb] = mfma_16x16x32(a, bu, au[c][mb]);
        }
      }
    }
    if (KW > 1) {
      // Waves 1..KW-1 hand their partial sums to wave 0.
      if (wave > 0) {
#pragma unroll
        for (int c = 0; c < CPW; ++c)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              red[wave - 1][(c * MB + mb) * 8 + i][lane] = ag[c][mb][i];
              red[wave - 1][(c * MB + mb) * 8 + 4 + i][lane] = au[c][mb][i];
            }
      }
      __syncthreads();
      if (wave == 0) {
#pragma unroll
        for (int q = 0; q < KW - 1; ++q)
#pragma unroll
          for (int c = 0; c < CPW; ++c)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                ag[c][mb][i] += red[q][(c * MB + mb) * 8 + i][lane];
                au[c][mb][i] += red[q][(c * MB + mb) * 8 + 4 + i][lane];
              }
      }
      __syncthreads();  // red[] free for the next item
      if (wave > 0) continue;
    }
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = it.m0 + mb * 16 + kq * 4 + i;
          if (r < it.nrows) {
            const float g = ag[c][mb][i], u = au[c][mb][i];
            out[(size_t)(it.row0 + r) * H + j + 16 * c] = (uint16_t)f32_to_bf16(swiglu(g, u, CLAMP ? clamp : 0.f));
          }
        }
      }
  }
}

// Phase 2: out[row, n] = hid[row, :] . W_d[n, :]; routed rows -> y_perm
// (bf16), shared rows -> y_shared (f32).
// KW = 1: an item is BM rows x 64·CPW output columns, wave w owns CPW groups
//         of 16 columns over the whole reduction (the routed experts' 1,280);
//         with CPW = 2 each wave keeps 16 weight rows' loads in flight per
//         batch, as the gate/up waves do (292 vs 300 µs at decode).
// KW = 4: an item is BM rows x 16·CPW columns and wave w owns the w-th
//         quarter of the reduction, the partial sums added in LDS in wave
//         order: for a long reduction (the dense FFN's 11,264) with few rows,
//         four times as many items keep enough waves streaming.
// KS > 1 (the shared group alone): the reduction is also split over KS
//         items, each writing its partial sums to partial[ks][row][d] (f32);
//         k_sum_partials adds them in ks order into y_shared.
// UNR: K steps per batch of loads (fewer keep a 32-row item at four waves
//         per SIMD).
template <int BM, int KW, int KS = 1, int CPW = 1, int UNR = kUnroll>
__global__ __launch_bounds__(256) void k_down(Groups gs, int d, int h, int hs, const uint16_t* __restrict__ hid,
                                              const uint16_t* __restrict__ hid_shared,
                                              const uint16_t* __restrict__ w_down,
                                              const uint16_t* __restrict__ ws_down, uint16_t* __restrict__ y_perm,
                                              float* __restrict__ y_shared, float* __restrict__ partial) {
  __shared__ int ip[kMaxGroups + 1];
  __shared__ int wsum[4];
  constexpr int MB = BM / 16;
  constexpr int COLS = 64 * CPW / KW;  // output columns per item
  __shared__ float red[KW > 1 ? KW - 1 : 1][CPW * MB * 4][kWave];
  const int ncol = d / COLS;
  const int items = item_prefix<BM>(ip, wsum, gs, ncol, ncol * KS);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int r16 = lane & 15, kq = lane >> 4;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int w = (int)blockIdx.x; w < items; w += gridDim.x) {
    const Item it = decode_item_xcd(ip, gs, BM, ncol, ncol * KS, w);
    const int H = it.shared ? hs : h;
    const int ks = KS > 1 ? it.nt / ncol : 0, cg = KS > 1 ? it.nt % ncol : it.nt;
    const int klen = H / (KW * KS), kbeg = (ks * KW + (KW > 1 ? wave : 0)) * klen;
    // Column of this lane in its first 16-column group; group c adds 16c.
    const int n = cg * COLS + (KW > 1 ? 0 : wave * 16 * CPW) + r16;
    const uint16_t* pb =
        (it.shared ? ws_down : w_down + (size_t)it.group * d * h) + (size_t)n * H + kbeg + kq * 8;
    const uint16_t* src = it.shared ? hid_shared : hid;
    const uint16_t* pa[MB];
    bool va[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = it.m0 + mb * 16 + r16;
      va[mb] = r < it.nrows;
      pa[mb] = src + (size_t)(it.row0 + (va[mb] ? r : 0)) * H + kbeg + kq * 8;
    }
    f32x4 acc[CPW][MB];
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[c][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Whole-line loads of the same 16-row groups (see load_lines).
    static_assert(UNR % 2 == 0, "whole-line loads cover two K steps");
    const uint16_t* pb8 = pb - (size_t)r16 * H - kq * 8 + (size_t)(lane >> 3) * H + (lane & 7) * 8;
    const int addr0 = 4 * (((lane & 7) << 3) | kq), addr1 = addr0 + 16;
    const bool hirow = r16 >= 8;
    // Batches as in phase 1; the steps left at the end go one by one (a
    // shorter whole-line batch there measured slower at decode: 252 vs
    // 247 us).
    auto batch = [&](int kk, int steps) {
      Lines lb[CPW][UNR / 2];
#pragma unroll
      for (int b2 = 0; b2 < UNR / 2; ++b2)
        if (2 * b2 < steps) {
#pragma unroll
          for (int c = 0; c < CPW; ++c)
            lb[c][b2] = load_lines(pb8 + (size_t)c * 16 * H + kk + 64 * b2, (size_t)8 * H);
        }
      u32x4 a[MB][UNR];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int u = 0; u < UNR; ++u)
          if (u < steps) a[mb][u] = va[mb] ? load16(pa[mb] + kk + 32 * u) : zero;
#pragma unroll
      for (int u = 0; u < UNR; ++u)
        if (u < steps) {
#pragma unroll
          for (int c = 0; c < CPW; ++c) {
            const u32x4 b = lines_operand(lb[c][u / 2], u % 2 ? addr1 : addr0, hirow);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) acc[c][mb] = mfma_16x16x32(a[mb][u], b, acc[c][mb]);
          }
        }
    };
    int kk = 0;
    for (; kk + 32 * UNR <= klen; kk += 32 * UNR) batch(kk, UNR);
    for (; kk < klen; kk += 32) {
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        const u32x4 b = load16(pb + (size_t)c * 16 * H + kk);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const u32x4 a = va[mb] ? load16(pa[mb] + kk) : zero;
          acc[c][mb] = mfma_16x16x32(a, b, acc[c][mb]);
        }
      }
    }
    if (KW > 1) {
      if (wave > 0) {
#pragma unroll
        for (int c = 0; c < CPW; ++c)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[wave - 1][(c * MB + mb) * 4 + i][lane] = acc[c][mb][i];
      }
      __syncthreads();
      if (wave == 0) {
#pragma unroll
        for (int q = 0; q < KW - 1; ++q)
#pragma unroll
          for (int c = 0; c < CPW; ++c)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[c][mb][i] += red[q][(c * MB + mb) * 4 + i][lane];
      }
      __syncthreads();  // red[] free for the next item
      if (wave > 0) continue;
    }
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = it.m0 + mb * 16 + kq * 4 + i;
          if (r < it.nrows) {
            const size_t o = (size_t)(it.row0 + r) * d + n + c * 16;
            if (KS > 1) partial[(size_t)ks * gs.T * d + o] = acc[c][mb][i];
            else if (it.shared) y_shared[o] = acc[c][mb][i];
            else y_perm[o] = (uint16_t)f32_to_bf16(acc[c][mb][i]);
          }
        }
      }
  }
}

// y[i] = sum over k = 0..KS-1 of partial[k][i], in k order (n elements, n a
// multiple of 4).
template <int KS>
__global__ __launch_bounds__(256) void k_sum_partials(const float* __restrict__ partial, size_t n,
                                                      float* __restrict__ y) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n / 4; i += (size_t)gridDim.x * 256) {
    float4 s = reinterpret_cast<const float4*>(partial)[i];
#pragma unroll
    for (int k = 1; k < KS; ++k) {
      const float4 v = reinterpret_cast<const float4*>(partial + (size_t)k * n)[i];
      s.x += v.x;
      s.y += v.y;
      s.z += v.z;
      s.w += v.w;
    }
    reinterpret_cast<float4*>(y)[i] = s;
  }
}

namespace {

// Which regime a phase runs in (crossovers measured on the 288-expert layer,
// d = 4,096, and on the dense FFN of hidden 11,264):
// - routed gate/up: the LDS-tiled kernels from 11 rows per routed group on
//   average; from 2 to 11 the streaming kernels with 32-row items (one M-tile
//   for nearly every group, so each weight row is read once; with 16-row
//   items a group of 17-32 rows reads its weights twice) in batches of 2 K
//   steps, two groups of 16 units per wave; below 2, 16-row items.  Gate/up
//   per launch, the previous rule (16-row streaming items below 5 rows per
//   group, tiled from 5) -> this one: 2.7 rows per group 0.558 -> 0.541 ms,
//   3.6: 0.615 -> 0.591, 4.4: 0.659 -> 0.610, 5.3: 0.710 -> 0.627, 7.1:
//   0.716 -> 0.633, 8.9: 0.786 -> 0.708, 10.7: 0.792 -> 0.767; at 12.4 the
//   32-row items lose (0.826 vs 0.793), at 1.8 (decode) they tie.  Batches
//   of 4 or 8 steps, or one group per wave, hold more registers per wave and
//   ran 7-12% slower at 7.1 rows per group.
// - routed down: tiled from 10 rows per group; from 4 to 10 it streams
//   32-row items (one M-tile for most groups) in batches of 2 K steps with
//   four groups of 16 columns per wave (8.0 rows per group: 424 vs 496 us
//   tiled in batches of 4 with two groups; 10.7: 500 vs 505; 12.4: 566 vs
//   513; four groups in batches of 2 against two in batches of 4: 7.1 rows
//   per group 0.372 vs 0.381 ms, 8.9: 0.421 vs 0.438), below 4 16-row items
//   (at decode two groups in batches of 6 beat four groups in batches of 2
//   or 6: 0.248 vs 0.254 and 0.274 ms).
// - the shared group alone (the dense FFN): the tiled kernels above 64
//   tokens.  Up to 256 tokens (one M-tile) they need the caller's split
//   scratch, which spreads each weight tile's reduction over several items
//   (gate/up 88 tiles x 4 splits, down 16 x 22 at hidden 11,264); without
//   it down stays on the streaming kernels, whose own split covers its long
//   reduction.  Dense FFN per call, streaming (32-row items) -> tiled with
//   splits: 0.229 -> 0.139 ms at 128 tokens, 0.355 -> 0.182 ms at 256; up to
//   64 tokens the streaming kernels with one M-tile win (64 tokens: 0.092 vs
//   0.122 ms; 80 to 128 tokens: within 3% of the tiled ones).
bool use_tiled(int T, int k, int E, const int32_t* offsets, bool down, bool split_scratch) {
  if (offsets) return (long)T * k >= (down ? 10L : 11L) * E;
  if (T <= 64) return false;
  return down ? T > 256 || split_scratch : true;
}

int pick_bm(int T, int k, int E) {
  // Average rows per group decides the M-tile: 16 up to 16 rows, else 32
  // (the shared group alone from 17 tokens).  Routed launches take 32-row
  // items earlier, in launch_gate_up from 2 rows per group and in
  // launch_down from 4.
  const long rows = (long)T * k;
  return rows <= 16L * E ? 16 : 32;
}

template <int BM, int KW, int UNR = kUnroll, int CPW = 1>
hipError_t gate_up_bm(const uint16_t* x, const Groups& gs, int d, int h, int hs, const uint16_t* w_gu,
                      const uint16_t* ws_gu, uint16_t* hid, uint16_t* hid_shared, float clamp, hipStream_t stream) {
  const auto kern = clamp > 0.f ? k_gate_up<BM, KW, true, UNR, CPW> : k_gate_up<BM, KW, false, UNR, CPW>;
  hipLaunchKernelGGL(kern, dim3(persistent_grid(kern) * kOversubscribe), dim3(256), 0, stream, x, gs, d, h, hs, w_gu, ws_gu, hid,
                     hid_shared, clamp);
  return hipGetLastError();
}

template <int BM, int KW, int UNR = kUnroll>
hipError_t down_bm(const Groups& gs, int d, int h, int hs, const uint16_t* hid, const uint16_t* hid_shared,
                   const uint16_t* w_down, const uint16_t* ws_down, uint16_t* y_perm, float* y_shared,
                   hipStream_t stream) {
  // Two 16-column groups per wave where the item width (128 columns) divides d.
  const auto kern =
      (KW == 1 && d % 128 == 0) ? k_down<BM, KW, 1, KW == 1 ? 2 : 1, UNR> : k_down<BM, KW, 1, 1, UNR>;
  hipLaunchKernelGGL(kern, dim3(persistent_grid(kern) * kOversubscribe), dim3(256), 0, stream, gs, d, h, hs, hid, hid_shared, w_down,
                     ws_down, y_perm, y_shared, nullptr);
  return hipGetLastError();
}

// The shared group alone with its reduction also split over items.
template <int BM, int UNR = kUnroll, int CPW = 1>
hipError_t down_bm_split(const Groups& gs, int d, int hs, const uint16_t* hid_shared, const uint16_t* ws_down,
                         float* y_shared, float* partial, hipStream_t stream) {
  const auto kern = k_down<BM, 4, kDownSplits, CPW, UNR>;
  hipLaunchKernelGGL(kern, dim3(persistent_grid(kern) * kOversubscribe), dim3(256), 0, stream, gs, d, 0, hs, nullptr, hid_shared,
                     nullptr, ws_down, nullptr, nullptr, partial);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const size_t n = (size_t)gs.T * d;
  const size_t blocks = (n / 4 + 255) / 256;
  hipLaunchKernelGGL(k_sum_partials<kDownSplits>, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0,
                     stream, partial, n, y_shared);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up(int T, int d, int E, int k, int h, int hs, const uint16_t* x, const int32_t* offsets,
                          const int32_t* perm, const uint16_t* w_gu, const uint16_t* ws_gu, uint16_t* hid,
                          uint16_t* hid_shared, int32_t* queue, hipStream_t stream, int e_total, float act_clamp,
                          float* partial) {
  if (T == 0) return hipSuccess;
  const int et = e_total > 0 ? e_total : E;
  // The tiled gate/up item covers 128 hidden units of each group.
  if (use_tiled(T, k, et, offsets, false, partial != nullptr) && h % 128 == 0 && hs % 128 == 0)
    return launch_gate_up_tiled(T, d, E, k, h, hs, x, offsets, perm, w_gu, ws_gu, hid, hid_shared, queue, stream,
                                act_clamp, partial);
  const Groups gs = make_groups(T, E, k, offsets, perm, ws_gu != nullptr);
  // Reduction split over the waves when every quarter is whole 32-wide steps.
  const bool split = d % 128 == 0;
  // The shared group alone up to 64 tokens: one M-tile, so every weight row
  // is read once, in short batches so that one round of blocks covers all
  // items.  From 17 rows each wave takes two groups of 16 units, whose four
  // weight row sets share each load of token rows.  Dense FFN of hidden 11,264
  // per call against batches of 8 steps, 32-row M-tiles and one group per
  // wave (tiled kernels at 64 tokens): 8 tokens 0.062 -> 0.055 ms, 16: 0.072
  // -> 0.061, 32: 0.093 -> 0.075, 48: 0.157 -> 0.082, 64: 0.122 -> 0.092.
  if (!offsets && split && T <= 16)
    return gate_up_bm<16, 4, 4>(x, gs, d, h, hs, w_gu, ws_gu, hid, hid_shared, act_clamp, stream);
  // Routed groups of 2 to 11 rows on average (below the tiled kernels'
  // threshold): 32-row items, batches of 2 steps, two 16-unit groups per wave.
  if (offsets && split && (long)T * k >= 2L * et)
    return gate_up_bm<32, 4, 2, 2>(x, gs, d, h, hs, w_gu, ws_gu, hid, hid_shared, act_clamp, stream);
  // 16-row items in batches of 6 steps (three waves per SIMD): 483 -> 477 us
  // at decode against batches of 8.
  if (pick_bm(T, k, offsets ? et : 1) == 16) {
    if (split) return gate_up_bm<16, 4, 6>(x, gs, d, h, hs, w_gu, ws_gu, hid, hid_shared, act_clamp, stream);
    return gate_up_bm<16, 1>(x, gs, d, h, hs, w_gu, ws_gu, hid, hid_shared, act_clamp, stream);
  }
  if (!offsets && split && T <= 32)
    return gate_up_bm<32, 4, 2, 2>(x, gs, d, h, hs, w_gu, ws_gu, hid, hid_shared, act_clamp, stream);
  if (!offsets && split && T <= 64)
    return gate_up_bm<64, 4, 2, 2>(x, gs, d, h, hs, w_gu, ws_gu, hid, hid_shared, act_clamp, stream);
  if (split) return gate_up_bm<32, 4>(x, gs, d, h, hs, w_gu, ws_gu, hid, hid_shared, act_clamp, stream);
  return gate_up_bm<32, 1>(x, gs, d, h, hs, w_gu, ws_gu, hid, hid_shared, act_clamp, stream);
}

hipError_t launch_down(int T, int d, int E, int k, int h, int hs, const int32_t* offsets, const uint16_t* hid,
                       const uint16_t* hid_shared, const uint16_t* w_down, const uint16_t* ws_down, uint16_t* y_perm,
                       float* y_shared, int32_t* queue, hipStream_t stream, int e_total, float* partial) {
  if (T == 0) return hipSuccess;
  const int et = e_total > 0 ? e_total : E;
  // The tiled down item covers 256 output columns.
  if (use_tiled(T, k, et, offsets, true, partial != nullptr) && d % 256 == 0)
    return launch_down_tiled(T, d, E, k, h, hs, offsets, hid, hid_shared, w_down, ws_down, y_perm, y_shared, queue,
                             stream, partial);
  const Groups gs = make_groups(T, E, k, offsets, nullptr, ws_down != nullptr);
  // The routed experts' reduction (1,280) is short enough already: quarters
  // of it are too few steps to keep loads in flight.  A long reduction of the
  // shared group alone (the dense FFN) is split over the waves.
  const bool split = !offsets && hs >= 4096 && hs % 128 == 0 && d % 16 == 0;
  // With few rows that still leaves too few items: split the reduction over
  // items too, into the caller's partial-sum buffer.
  // Up to 64 tokens one M-tile, as in gate/up; from 17 rows each wave takes
  // four groups of 16 columns (d is a multiple of 64), which share each load
  // of hidden rows.
  if (split && partial && T <= kDownSplitMaxTokens && hs % (128 * kDownSplits) == 0) {
    if (T <= 16) return down_bm_split<16, 4>(gs, d, hs, hid_shared, ws_down, y_shared, partial, stream);
    if (T <= 32) return down_bm_split<32, 4, 4>(gs, d, hs, hid_shared, ws_down, y_shared, partial, stream);
    if (T <= 64) return down_bm_split<64, 2, 4>(gs, d, hs, hid_shared, ws_down, y_shared, partial, stream);
    return down_bm_split<32>(gs, d, hs, hid_shared, ws_down, y_shared, partial, stream);
  }
  // Routed groups of 4 to 10 rows on average: 32-row items, batches of 2
  // steps, four 16-column groups per wave where the item width (256 columns)
  // divides d, else two in batches of 4.
  if (offsets && (long)T * k >= 4L * et) {
    if (d % 256 == 0) {
      const auto kern = k_down<32, 1, 1, 4, 2>;
      hipLaunchKernelGGL(kern, dim3(persistent_grid(kern) * kOversubscribe), dim3(256), 0, stream, gs, d, h, hs, hid,
                         hid_shared, w_down, ws_down, y_perm, y_shared, nullptr);
      return hipGetLastError();
    }
    return down_bm<32, 1, 4>(gs, d, h, hs, hid, hid_shared, w_down, ws_down, y_perm, y_shared, stream);
  }
  if (pick_bm(T, k, offsets ? et : 1) == 16) {
    if (split) return down_bm<16, 4>(gs, d, h, hs, hid, hid_shared, w_down, ws_down, y_perm, y_shared, stream);
    // Batches of 6 steps, four waves per SIMD: 256 -> 247 us at decode
    // against batches of 8 at three waves.
    return down_bm<16, 1, 6>(gs, d, h, hs, hid, hid_shared, w_down, ws_down, y_perm, y_shared, stream);
  }
  if (split) return down_bm<32, 4>(gs, d, h, hs, hid, hid_shared, w_down, ws_down, y_perm, y_shared, stream);
  return down_bm<32, 1>(gs, d, h, hs, hid, hid_shared, w_down, ws_down, y_perm, y_shared, stream);
}

size_t split_partial_bytes(int T, int d, int hs) {
  const size_t streaming =
      T <= kDownSplitMaxTokens ? ((size_t)kDownSplits * T * d * sizeof(float) + 255) / 256 * 256 : 0;
  const size_t tiled = tiled_split_bytes(T, d, hs);
  return streaming > tiled ? streaming : tiled;
}

size_t expert_hid_bytes(int T, int k, int h) { return ((size_t)T * k * h * sizeof(uint16_t) + 255) / 256 * 256; }
size_t shared_hid_bytes(int T, int hs) { return ((size_t)T * hs * sizeof(uint16_t) + 255) / 256 * 256; }

}  // namespace moe
