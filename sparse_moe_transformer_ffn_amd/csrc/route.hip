// route.hip -- router: logits (thin bf16 GEMM on MFMA), sigmoid scores,
// biased top-k selection per token on one wavefront, weights, gap, counts.
//
// Layer definition: [Blog] "Step 3.5 Flash: Open Frontier-Level Intelligence
// with 11B Active Parameters" §2.2.2 (routing probabilities, top-K set and
// mask); the selection-only bias is the loss-free balancing of [Digest]
// "Step 3.5 Flash 技术论文深度解读" (note under the architecture table).
#include "common.h"
#include "kernels.h"

namespace moe {

// Partial logits z_part[ks][t][e] = sum over the ks-th reduction chunk of
// x[t,:] . w_router[e,:].  One wave computes a 16-token x 16-expert tile; a
// block of four waves covers 64 experts.  Grid: (ceil(E/64), ceil(T/16), ks).
// Block (0,0,0) also clears expert_counts for the selection kernel.
//
// NORM: x is the un-normalised stream h.  The block first forms the sum of
// squares of its 16 rows exactly as k_rmsnorm does (thread tid: columns
// 8 tid + 2048 j in order, a butterfly over the wave, the four waves in
// order), then normalises each 16-byte slice of x as it loads it, rounding
// to bf16 as k_rmsnorm does; the blocks of the first expert column also store
// their slices to x_out, so x_out matches moe_rmsnorm bit for bit.
template <bool NORM>
__global__ __launch_bounds__(256) void k_route_logits(const uint16_t* __restrict__ x,
                                                      const uint16_t* __restrict__ w_router, int T, int d, int E,
                                                      int kchunk, float* __restrict__ partial,
                                                      int32_t* __restrict__ counts, const float* __restrict__ gamma,
                                                      float eps, uint16_t* __restrict__ x_out) {
  const int tid = threadIdx.x;
  if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0)
    for (int e = tid; e < E; e += 256) counts[e] = 0;
  const int wave = tid / kWave, lane = tid % kWave;
  const int r16 = lane & 15, kq = lane >> 4;
  const int t0 = blockIdx.y * 16;
  float inv = 1.f;
  if constexpr (NORM) {
    __shared__ float part[16][4];
    __shared__ float inv_s[16];
    float ss[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) ss[r] = 0.f;
    for (int c = tid * 8; c < d; c += 256 * 8) {
      u32x4 v[16];
#pragma unroll
      for (int r = 0; r < 16; ++r)
        v[r] = t0 + r < T ? load16(x + (size_t)(t0 + r) * d + c) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float f[8];
        unpack8(v[r], f);
#pragma unroll
        for (int q = 0; q < 8; ++q) ss[r] = fmaf(f[q], f[q], ss[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float v = ss[r];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
      if (lane == 0) part[r][wave] = v;
    }
    __syncthreads();
    if (tid < 16) inv_s[tid] = rms_inv((part[tid][0] + part[tid][1]) + (part[tid][2] + part[tid][3]), d, eps);
    __syncthreads();
    inv = inv_s[r16];
  }
  const int e0 = blockIdx.x * 64 + wave * 16;
  if (e0 >= E) return;
  const int k_begin = blockIdx.z * kchunk;
  const int k_end = min(d, k_begin + kchunk);
  const int ta = t0 + r16, eb = e0 + r16;
  const bool va = ta < T, vb = eb < E;
  const uint16_t* pa = x + (size_t)(va ? ta : 0) * d + kq * 8;
  const uint16_t* pb = w_router + (size_t)(vb ? eb : 0) * d + kq * 8;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const bool store_x = NORM && va && blockIdx.x == 0 && wave == 0;
  // One 32-wide K step on loaded slices (normalising x first under NORM).
  auto step = [&](u32x4 a, u32x4 b, int kk) {
    if constexpr (NORM) {
      const int c = kk + kq * 8;
      float f[8];
      unpack8(a, f);
#pragma unroll
      for (int q = 0; q < 8; ++q) f[q] = rms_scale(f[q], inv, gamma, c + q);
      a = va ? pack8(f) : zero;
      if (store_x) *reinterpret_cast<u32x4*>(x_out + (size_t)ta * d + c) = a;
    }
    acc = mfma_16x16x32(a, b, acc);
  };
  // Four steps' loads issued before their MFMAs, then the remaining steps.
  int kk = k_begin;
  for (; kk + 4 * 32 <= k_end; kk += 4 * 32) {
    u32x4 a[4], b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a[u] = va ? load16(pa + kk + 32 * u) : zero;
      b[u] = vb ? load16(pb + kk + 32 * u) : zero;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) step(a[u], b[u], kk + 32 * u);
  }
  for (; kk < k_end; kk += 32) step(va ? load16(pa + kk) : zero, vb ? load16(pb + kk) : zero, kk);
  const int e = e0 + r16;
  if (e < E) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + kq * 4 + i;
      if (t < T) partial[((size_t)blockIdx.z * T + t) * E + e] = acc[i];
    }
  }
}

// Large batches: the same partial logits from an LDS-staged GEMM.  A block
// covers 128 tokens x all E experts (E a multiple of 32, at most 288) over one
// reduction chunk [k0, k0 + kchunk).  Operands go HBM/L2 -> LDS with direct
// loads (global_load_lds_dwordx4) through three stages of 64-wide K slices;
// wave w multiplies tokens [32 w, 32 w + 32) by every expert with MFMA
// 32x32x16 (E/32 accumulator tiles), so each router slice read from LDS
// serves 32 tokens and each token slice E experts.  Rows of a slice are eight
// 16-byte segments stored at slot seg ^ ((row >> 1) & 7) (conflict-free
// reads of one segment of 32 consecutive rows).
namespace {

constexpr int kRtM = 128;                    // tokens per block
constexpr int kRtMaxE = 288;                 // experts held per stage
constexpr int kRtChunk = 64;                 // K elements per stage
constexpr int kRtStageA = kRtM * kRtChunk;   // bf16 elements
constexpr int kRtStage = kRtStageA + kRtMaxE * kRtChunk;  // 52 KiB
constexpr int kRtLoadsA = kRtM / 8 / 4;      // direct loads per thread per chunk (8 rows each)
constexpr int kRtLoadsB = kRtMaxE / 8 / 4;
// s_waitcnt vmcnt(one chunk's loads), lgkmcnt and expcnt not waited on.
constexpr int kRtWaitChunk = 0x0F70 | (kRtLoadsA + kRtLoadsB);
static_assert(kRtLoadsA + kRtLoadsB < 16, "vmcnt field");

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int rt_swz(int row) { return (row >> 1) & 7; }

// Direct loads of one chunk: A regions q*4 + wave (q < kRtLoadsA), then B
// regions q*4 + wave (q < kRtLoadsB); region r covers rows 8r .. 8r+7 of the
// stage.  Every thread issues the same number of loads whatever T and E:
// token rows past T re-read row T-1 and router rows past E re-read row E-1
// (into stage rows nobody reads), so the in-flight count is a constant.
__device__ __forceinline__ void rt_issue(const uint16_t* x, const uint16_t* w_router, int T, int d, int E, int t0,
                                         int kk, uint16_t* stage, int wave, int lane) {
  const int seg_row = lane / 8, slot = lane % 8;
#pragma unroll
  for (int q = 0; q < kRtLoadsA; ++q) {
    const int row = (q * 4 + wave) * 8 + seg_row;
    const int t = min(t0 + row, T - 1);
    const int seg = slot ^ rt_swz(row);
    __builtin_amdgcn_global_load_lds(x + (size_t)t * d + kk + seg * 8, stage + (q * 4 + wave) * 8 * kRtChunk, 16,
                                     0, 0);
  }
#pragma unroll
  for (int q = 0; q < kRtLoadsB; ++q) {
    const int r = q * 4 + wave;
    const int row = r * 8 + seg_row;
    const int seg = slot ^ rt_swz(row);
    __builtin_amdgcn_global_load_lds(w_router + (size_t)min(row, E - 1) * d + kk + seg * 8,
                                     stage + kRtStageA + r * 8 * kRtChunk, 16, 0, 0);
  }
}

}  // namespace

namespace {

// Per-thread constants of the LDS-staged router kernel.
struct RtLane {
  const uint16_t* x;
  const uint16_t* w_router;
  int T, d, E, t0, k0, nch, wave, lane;
  int arow;  // LDS row of this lane's token fragment
  int lhi;   // lane / 32: which 8 of a 16-wide K step
  int f;     // rt_swz of every row this lane reads
  int ntile; // E / 32
};

// Chunk c (in `cur`): chunk c has landed for this thread once only the next
// chunk's loads remain; the barrier (a bare s_barrier: a release fence would
// drain the loads in flight) makes it visible to all and guarantees nobody
// still reads `ahead`, the stage of chunk c-1, which chunk c+2 goes into.
// Past the last chunk the loads repeat the last chunk into a stage nobody
// reads, so the count of loads in flight stays the same.
__device__ __forceinline__ void rt_chunk(const RtLane& ln, const uint16_t* cur, uint16_t* ahead, int c,
                                         f32x16 (&acc)[kRtMaxE / 32]) {
  __builtin_amdgcn_s_waitcnt(kRtWaitChunk);
  __builtin_amdgcn_s_barrier();
  rt_issue(ln.x, ln.w_router, ln.T, ln.d, ln.E, ln.t0, ln.k0 + min(c + 2, ln.nch - 1) * kRtChunk, ahead, ln.wave,
           ln.lane);
#pragma unroll
  for (int s = 0; s < kRtChunk / 16; ++s) {
    const int slot = ((2 * s + ln.lhi) ^ ln.f) * 8;
    const u32x4 a = *reinterpret_cast<const u32x4*>(&cur[ln.arow * kRtChunk + slot]);
#pragma unroll
    for (int j = 0; j < kRtMaxE / 32; ++j) {
      if (j < ln.ntile) {
        const u32x4 b = *reinterpret_cast<const u32x4*>(&cur[kRtStageA + (j * 32 + (ln.lane & 31)) * kRtChunk + slot]);
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                         acc[j], 0, 0, 0);
      }
    }
  }
}

}  // namespace

__global__ __launch_bounds__(256) void k_route_logits_tiled(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ w_router, int T, int d,
                                                            int E, int kchunk, float* __restrict__ partial,
                                                            int32_t* __restrict__ counts) {
  __shared__ __attribute__((aligned(16))) uint16_t st0[kRtStage];
  __shared__ __attribute__((aligned(16))) uint16_t st1[kRtStage];
  __shared__ __attribute__((aligned(16))) uint16_t st2[kRtStage];
  const int tid = threadIdx.x;
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int e = tid; e < E; e += 256) counts[e] = 0;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int l32 = lane & 31, lhi = lane >> 5;
  const int t0 = blockIdx.x * kRtM;
  const int k0 = blockIdx.y * kchunk;
  const int nch = (min(d, k0 + kchunk) - k0) / kRtChunk;  // the last split may be shorter
  const int ntile = E / 32;
  f32x16 acc[kRtMaxE / 32];
#pragma unroll
  for (int j = 0; j < kRtMaxE / 32; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[j][i] = 0.f;
  rt_issue(x, w_router, T, d, E, t0, k0, st0, wave, lane);
  rt_issue(x, w_router, T, d, E, t0, k0 + min(1, nch - 1) * kRtChunk, st1, wave, lane);
  const RtLane ln{x, w_router, T, d, E, t0, k0, nch, wave, lane, wave * 32 + l32, lhi, rt_swz(l32), E / 32};
  int c = 0;
  for (; c + 3 <= nch; c += 3) {
    rt_chunk(ln, st0, st2, c, acc);
    rt_chunk(ln, st1, st0, c + 1, acc);
    rt_chunk(ln, st2, st1, c + 2, acc);
  }
  if (c < nch) {
    rt_chunk(ln, st0, st2, c, acc);
    if (c + 1 < nch) rt_chunk(ln, st1, st0, c + 1, acc);
  }
  // No direct load may still be writing this block's LDS when it exits.
  __builtin_amdgcn_s_waitcnt(0x0F70);
  // acc[j] element i: token 32 w + 8 (i/4) + 4 lhi + (i%4), expert 32 j + l32.
#pragma unroll
  for (int j = 0; j < kRtMaxE / 32; ++j) {
    if (j >= ntile) continue;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int t = t0 + wave * 32 + 8 * (i / 4) + 4 * lhi + (i % 4);
      if (t < T) partial[((size_t)blockIdx.y * T + t) * E + j * 32 + l32] = acc[j][i];
    }
  }
}

namespace {

// Order-preserving map of a float to uint32 (larger float -> larger key).
// -0 is first folded onto +0 so that equal floats get equal keys.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t b = __float_as_uint(f + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// Number of keys >= tau over the wave (EPL keys per lane; invalid slots hold 0).
template <int EPL>
__device__ __forceinline__ int count_at_least(const uint32_t (&key)[EPL], uint32_t tau) {
  int c = 0;
#pragma unroll
  for (int j = 0; j < EPL; ++j) c += __popcll(__ballot(key[j] >= tau));
  return c;
}

// Largest tau with at least `need` keys >= tau: the need-th largest key.
// Largest key strictly below tau over the wave (0 if none).
template <int EPL>
__device__ __forceinline__ uint32_t max_below(const uint32_t (&key)[EPL], uint32_t tau) {
  uint32_t m = 0u;
#pragma unroll
  for (int j = 0; j < EPL; ++j) m = (key[j] < tau && key[j] > m) ? key[j] : m;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)m, off, kWave);
    m = o > m ? o : m;
  }
  return m;
}

template <int EPL>
__device__ __forceinline__ uint32_t kth_largest(const uint32_t (&key)[EPL], int need) {
  uint32_t tau = 0u;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = tau | (1u << b);
    if (count_at_least<EPL>(key, cand) >= need) tau = cand;
  }
  return tau;
}

}  // namespace

// Per-token selection.  A wave handles tpw consecutive tokens, one at a time;
// lane l owns experts l, l+64, ... (EPL = experts per lane, E <= 64*EPL).
// The k-th largest biased score is found exactly by a 32-step radix search on
// order-preserving keys, counting with wave ballots (no cross-lane data
// movement); the chosen set is every expert above it plus, among those equal
// to it, the lowest indices.  A block of four waves aggregates the expert
// histogram of its 4 * tpw tokens in LDS before one global atomic add per
// touched expert (integer atomics: order-independent).
//
// DIAG: also the routing probabilities p_{t,e} = s_{t,e} / sum_e' s_{t,e'}
// ([Blog] §2.2.2) summed over the wave's tokens, and the probability mass of
// each token's chosen set ([Blog] §5.2.3, routing confidence), written as
// wave partials diag[e * nw + w] (row E: the mass) for w < nw = ceil(T/tpw);
// fixed summation order, so the result is deterministic.
template <int EPL, bool DIAG>
__global__ __launch_bounds__(256) void k_route_select(const float* __restrict__ partial, int ksplit, int T, int E,
                                                      int k, int tpw, const float* __restrict__ sel_bias,
                                                      const float* __restrict__ logit_bias,
                                                      int32_t* __restrict__ topk_ids,
                                                      float* __restrict__ topk_weights, float* __restrict__ topk_gap,
                                                      int32_t* __restrict__ counts, float* __restrict__ diag,
                                                      int nw) {
  __shared__ int hist[1024];
  __shared__ float chosen_s[4][16];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int wave = tid / kWave, lane = tid % kWave;
  float p_acc[EPL], mass_acc = 0.f;
#pragma unroll
  for (int j = 0; j < EPL; ++j) p_acc[j] = 0.f;
  for (int tw = 0; tw < tpw; ++tw) {  // wave-uniform; no block barrier inside
    const int t = (blockIdx.x * 4 + wave) * tpw + tw;
    if (t >= T) break;
    // Logit = sum of the split-K partials in chunk order; loads are issued
    // four chunks at a time so their latencies overlap.
    float z[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) z[j] = 0.f;
    const size_t stride = (size_t)T * E;
    const float* base = partial + (size_t)t * E + lane;
    int ks = 0;
    for (; ks + 4 <= ksplit; ks += 4) {
      float v[4][EPL];
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < EPL; ++j)
          v[q][j] = (lane + kWave * j < E) ? base[(ks + q) * stride + kWave * j] : 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < EPL; ++j) z[j] += v[q][j];
    }
    for (; ks < ksplit; ++ks)
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        if (lane + kWave * j < E) z[j] += base[ks * stride + kWave * j];
    float score[EPL];
    uint32_t key[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane + kWave * j;
      score[j] = 0.f;
      key[j] = 0u;  // below every real key: never chosen
      if (e < E) {
        const float zz = logit_bias ? z[j] + logit_bias[e] : z[j];
        score[j] = 1.0f / (1.0f + __expf(-zz));
        const float beta = score[j] + sel_bias[e];
        // A NaN score sorts below every number; +1 keeps it above the padding.
        key[j] = (beta == beta) ? order_key(beta) : 1u;
      }
    }
    const uint32_t tau = kth_largest<EPL>(key, k);
    // Chosen: keys > tau, then the lowest-index experts with key == tau.
    const unsigned long long below = (1ull << lane) - 1ull;
    int above = 0;
#pragma unroll
    for (int j = 0; j < EPL; ++j) above += __popcll(__ballot(key[j] > tau));
    int ties_left = k - above;
    unsigned long long chosen[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      unsigned long long m = __ballot(key[j] > tau);
      unsigned long long tie = __ballot(key[j] == tau);
      while (ties_left > 0 && tie) {  // wave-uniform: masks are scalars
        const unsigned long long low = tie & (~tie + 1ull);
        m |= low;
        tie ^= low;
        --ties_left;
      }
      chosen[j] = m;
    }
    // Gap to the (k+1)-th largest key: tau again if at least k+1 keys reach
    // tau (a tie; gap zero), else the largest key below tau.
    float gap = __builtin_huge_valf();
    if (k < E) {
      const uint32_t tau2 = count_at_least<EPL>(key, tau) > k ? tau : max_below<EPL>(key, tau);
      gap = key_value(tau) - key_value(tau2);
    }
    // Rank of each chosen expert in ascending expert order (j major, then
    // lane), its weight from the unbiased scores summed in that order.
    int before = 0;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      if ((chosen[j] >> lane) & 1ull) chosen_s[wave][before + __popcll(chosen[j] & below)] = score[j];
      before += __popcll(chosen[j]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float total = 0.f;
    for (int q = 0; q < k; ++q) total += chosen_s[wave][q];
    if constexpr (DIAG) {
      // Butterfly sum: every lane ends with the same bits.
      float all = 0.f;
#pragma unroll
      for (int j = 0; j < EPL; ++j) all += score[j];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) all += __shfl_xor(all, off);
#pragma unroll
      for (int j = 0; j < EPL; ++j) p_acc[j] += score[j] / all;
      mass_acc += total / all;
    }
    before = 0;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      if ((chosen[j] >> lane) & 1ull) {
        const int rank = before + __popcll(chosen[j] & below);
        const int e = lane + kWave * j;
        topk_ids[(size_t)t * k + rank] = e;
        topk_weights[(size_t)t * k + rank] = score[j] / total;
        atomicAdd(&hist[e], 1);
      }
      before += __popcll(chosen[j]);
    }
    if (lane == 0 && topk_gap) topk_gap[t] = gap;
    __builtin_amdgcn_wave_barrier();  // chosen_s is reused by the next token
  }
  if constexpr (DIAG) {
    const int w = blockIdx.x * 4 + wave;
    if (w < nw) {
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        if (lane + kWave * j < E) diag[(size_t)(lane + kWave * j) * nw + w] = p_acc[j];
      if (lane == 0) diag[(size_t)E * nw + w] = mass_acc;
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256)
    if (hist[e]) atomicAdd(&counts[e], hist[e]);
}

// Column sums of the wave partials: block e adds diag[e * nw + w] over w in
// a fixed order (thread-strided with four loads in flight, then a tree), in
// double.
__global__ __launch_bounds__(256) void k_diag_columns(const float* __restrict__ diag, int nw,
                                                      double* __restrict__ col) {
  __shared__ double red[256];
  const int e = blockIdx.x, tid = threadIdx.x;
  double s = 0.0;
  for (int w0 = 0; w0 < nw; w0 += 1024) {
    float v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int w = w0 + q * 256 + tid;
      v[q] = w < nw ? diag[(size_t)e * nw + w] : 0.f;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) s += (double)v[q];
  }
  red[tid] = s;
  __syncthreads();
  for (int half = 128; half >= 1; half >>= 1) {
    if (tid < half) red[tid] += red[tid + half];
    __syncthreads();
  }
  if (tid == 0) col[e] = red[0];
}

// p_e = (sum_t p_{t,e}) / T, f_e = counts_e / (T k); over G contiguous groups
// of E/G experts, L_EP = G * sum_g f_g p_g ([Blog] §2.2.2); confidence =
// (sum_t mass_t) / T ([Blog] §5.2.3).  T = 0 writes zeros.  One block.
__global__ __launch_bounds__(256) void k_diag_finish(const double* __restrict__ col,
                                                     const int32_t* __restrict__ counts, int T, int E, int k, int G,
                                                     float* __restrict__ p_e, float* __restrict__ f_e,
                                                     float* __restrict__ summary) {
  __shared__ double pd[1024], fd[1024], prod[1024];
  const int tid = threadIdx.x;
  if (T == 0) {
    for (int e = tid; e < E; e += 256) p_e[e] = f_e[e] = 0.f;
    if (tid == 0) summary[0] = summary[1] = 0.f;
    return;
  }
  for (int e = tid; e < E; e += 256) {
    pd[e] = col[e] / (double)T;
    fd[e] = (double)counts[e] / ((double)T * k);
    p_e[e] = (float)pd[e];
    f_e[e] = (float)fd[e];
  }
  __syncthreads();
  const int per = E / G;
  for (int g = tid; g < G; g += 256) {
    double pg = 0.0, fg = 0.0;
    for (int e = g * per; e < (g + 1) * per; ++e) {
      pg += pd[e];
      fg += fd[e];
    }
    prod[g] = fg * pg;
  }
  __syncthreads();
  if (tid == 0) {
    double l = 0.0;
    for (int g = 0; g < G; ++g) l += prod[g];
    summary[0] = (float)(G * l);
    summary[1] = (float)(col[E] / (double)T);
  }
}

__global__ void k_zero_i32(int32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

RouteSplit route_split(int T, int d, int E) {
  if (T >= 1024 && E % 32 == 0 && E <= kRtMaxE && d % kRtChunk == 0) {
    // LDS-staged kernel: split the reduction until there are >= 256 blocks,
    // keeping chunks whole 64-wide slices.
    const int mblocks = (T + kRtM - 1) / kRtM;
    int ks = (256 + mblocks - 1) / mblocks;
    ks = ks > 8 ? 8 : ks;
    ks = ks > d / kRtChunk ? d / kRtChunk : ks;
    ks = ks < 1 ? 1 : ks;
    int kchunk = (d / kRtChunk + ks - 1) / ks * kRtChunk;
    ks = (d + kchunk - 1) / kchunk;
    return RouteSplit{ks, kchunk, true};
  }
  const int base = ((E + 63) / 64) * ((T + 15) / 16);
  int ks = 512 / (base > 0 ? base : 1);
  ks = ks < 1 ? 1 : ks;
  ks = ks > d / 256 ? d / 256 : ks;
  ks = ks > 8 ? 8 : ks;
  ks = ks < 1 ? 1 : ks;
  int kchunk = (d + ks - 1) / ks;
  kchunk = (kchunk + 31) / 32 * 32;
  ks = (d + kchunk - 1) / kchunk;
  return RouteSplit{ks, kchunk, false};
}

namespace {

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

// Tokens per wave of the selection: one below 2,048 tokens (latency), two up
// to 8,191, four from 8,192 (whole router at 8,192 tokens: 73 us with 4, 76
// with 2, 84 with 8; at 4,096 tokens 53 us with 2, 58 with 4).
int select_tpw(int T) { return T >= 8192 ? 4 : T >= 2048 ? 2 : 1; }

size_t logits_bytes(int T, int d, int E) {
  return round256((size_t)route_split(T, d, E).ksplit * (size_t)T * (size_t)E * sizeof(float));
}

}  // namespace

hipError_t launch_route(int T, int d, int E, int k, const uint16_t* x, const uint16_t* w_router,
                        const float* sel_bias, const float* logit_bias, int32_t* topk_ids, float* topk_weights,
                        int32_t* counts, float* topk_gap, const RouteDiag* diag, void* workspace,
                        hipStream_t stream, const RouteNorm* norm) {
  if (T == 0) {
    hipLaunchKernelGGL(k_zero_i32, dim3((E + 255) / 256), dim3(256), 0, stream, counts, E);
    if (diag)
      hipLaunchKernelGGL(k_diag_finish, dim3(1), dim3(256), 0, stream, nullptr, counts, 0, E, k, diag->groups,
                         diag->p_e, diag->f_e, diag->summary);
    return hipGetLastError();
  }
  const RouteSplit rs = route_split(T, d, E);
  float* partial = static_cast<float*>(workspace);
  hipError_t err;
  if (rs.tiled) {
    // The staged kernel loads x straight into LDS, so the normalised rows
    // are formed first and routed from x_out.
    if (norm) {
      if ((err = launch_rmsnorm(T, d, x, norm->gamma, norm->eps, norm->x_out, stream)) != hipSuccess) return err;
      x = norm->x_out;
    }
    hipLaunchKernelGGL(k_route_logits_tiled, dim3((T + kRtM - 1) / kRtM, rs.ksplit), dim3(256), 0, stream, x,
                       w_router, T, d, E, rs.kchunk, partial, counts);
  } else if (norm) {
    hipLaunchKernelGGL(k_route_logits<true>, dim3((E + 63) / 64, (T + 15) / 16, rs.ksplit), dim3(256), 0, stream,
                       x, w_router, T, d, E, rs.kchunk, partial, counts, norm->gamma, norm->eps, norm->x_out);
  } else {
    hipLaunchKernelGGL(k_route_logits<false>, dim3((E + 63) / 64, (T + 15) / 16, rs.ksplit), dim3(256), 0, stream,
                       x, w_router, T, d, E, rs.kchunk, partial, counts, nullptr, 0.f, nullptr);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const int tpw = select_tpw(T);
  const int nw = (T + tpw - 1) / tpw;
  char* diag_base = static_cast<char*>(workspace) + logits_bytes(T, d, E);
  float* wave_part = reinterpret_cast<float*>(diag_base);
  double* col = reinterpret_cast<double*>(diag_base + round256((size_t)(E + 1) * nw * sizeof(float)));
  const dim3 grid((T + 4 * tpw - 1) / (4 * tpw)), block(256);
  const int epl = (E + 63) / 64;
#define MOE_SELECT(N)                                                                                          \
  do {                                                                                                         \
    if (diag)                                                                                                  \
      hipLaunchKernelGGL((k_route_select<N, true>), grid, block, 0, stream, partial, rs.ksplit, T, E, k, tpw,  \
                         sel_bias, logit_bias, topk_ids, topk_weights, topk_gap, counts, wave_part, nw);       \
    else                                                                                                       \
      hipLaunchKernelGGL((k_route_select<N, false>), grid, block, 0, stream, partial, rs.ksplit, T, E, k, tpw, \
                         sel_bias, logit_bias, topk_ids, topk_weights, topk_gap, counts, nullptr, 0);          \
  } while (0)
  if (epl <= 1) MOE_SELECT(1);
  else if (epl <= 2) MOE_SELECT(2);
  else if (epl <= 4) MOE_SELECT(4);
  else if (epl <= 5) MOE_SELECT(5);
  else if (epl <= 8) MOE_SELECT(8);
  else MOE_SELECT(16);
#undef MOE_SELECT
  if (!diag) return hipGetLastError();
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(k_diag_columns, dim3(E + 1), dim3(256), 0, stream, wave_part, nw, col);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(k_diag_finish, dim3(1), dim3(256), 0, stream, col, counts, T, E, k, diag->groups, diag->p_e,
                     diag->f_e, diag->summary);
  return hipGetLastError();
}

// Logits partials, then (for the diagnostics) the wave partials [E+1][nw] f32
// and the column sums [E+1] f64.
size_t route_workspace_bytes(int T, int d, int E) {
  const int tpw = select_tpw(T);
  const size_t nw = (size_t)(T + tpw - 1) / tpw;
  return logits_bytes(T, d, E) + round256((size_t)(E + 1) * nw * sizeof(float)) +
         round256((size_t)(E + 1) * sizeof(double));
}

}  // namespace moe
