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
__global__ __launch_bounds__(256) void k_route_logits(const uint16_t* __restrict__ x,
                                                      const uint16_t* __restrict__ w_router, int T, int d, int E,
                                                      int kchunk, float* __restrict__ partial,
                                                      int32_t* __restrict__ counts) {
  const int tid = threadIdx.x;
  if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0)
    for (int e = tid; e < E; e += 256) counts[e] = 0;
  const int wave = tid / kWave, lane = tid % kWave;
  const int r16 = lane & 15, kq = lane >> 4;
  const int t0 = blockIdx.y * 16;
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
#pragma unroll 4
  for (int kk = k_begin; kk < k_end; kk += 32) {
    const u32x4 a = va ? load16(pa + kk) : zero;
    const u32x4 b = vb ? load16(pb + kk) : zero;
    acc = mfma_16x16x32(a, b, acc);
  }
  const int e = e0 + r16;
  if (e < E) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + kq * 4 + i;
      if (t < T) partial[((size_t)blockIdx.z * T + t) * E + e] = acc[i];
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

// Per-token selection.  One wave per token; lane l owns experts l, l+64, ...
// (EPL = experts per lane, E <= 64*EPL).  The k-th largest biased score is
// found exactly by a 32-step radix search on order-preserving keys, counting
// with wave ballots (no cross-lane data movement); the chosen set is every
// expert above it plus, among those equal to it, the lowest indices.  A block
// of four waves handles four tokens and aggregates the expert histogram in LDS
// before one global atomic add per touched expert (integer atomics:
// order-independent).
template <int EPL>
__global__ __launch_bounds__(256) void k_route_select(const float* __restrict__ partial, int ksplit, int T, int E,
                                                      int k, const float* __restrict__ sel_bias,
                                                      const float* __restrict__ logit_bias,
                                                      int32_t* __restrict__ topk_ids,
                                                      float* __restrict__ topk_weights, float* __restrict__ topk_gap,
                                                      int32_t* __restrict__ counts) {
  __shared__ int hist[1024];
  __shared__ float chosen_s[4][16];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int wave = tid / kWave, lane = tid % kWave;
  const int t = blockIdx.x * 4 + wave;
  if (t < T) {  // wave-uniform; no block barrier inside
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
    // Gap to the (k+1)-th largest: zero if a tied expert was left out.
    float gap = __builtin_huge_valf();
    if (k < E) {
      const uint32_t tau2 = kth_largest<EPL>(key, k + 1);
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
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256)
    if (hist[e]) atomicAdd(&counts[e], hist[e]);
}

__global__ void k_zero_i32(int32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

RouteSplit route_split(int T, int d, int E) {
  const int base = ((E + 63) / 64) * ((T + 15) / 16);
  int ks = 512 / (base > 0 ? base : 1);
  ks = ks < 1 ? 1 : ks;
  ks = ks > d / 256 ? d / 256 : ks;
  ks = ks > 8 ? 8 : ks;
  ks = ks < 1 ? 1 : ks;
  int kchunk = (d + ks - 1) / ks;
  kchunk = (kchunk + 31) / 32 * 32;
  ks = (d + kchunk - 1) / kchunk;
  return RouteSplit{ks, kchunk};
}

hipError_t launch_route(int T, int d, int E, int k, const uint16_t* x, const uint16_t* w_router,
                        const float* sel_bias, const float* logit_bias, int32_t* topk_ids, float* topk_weights,
                        int32_t* counts, float* topk_gap, void* workspace, hipStream_t stream) {
  if (T == 0) {
    hipLaunchKernelGGL(k_zero_i32, dim3((E + 255) / 256), dim3(256), 0, stream, counts, E);
    return hipGetLastError();
  }
  const RouteSplit rs = route_split(T, d, E);
  float* partial = static_cast<float*>(workspace);
  hipLaunchKernelGGL(k_route_logits, dim3((E + 63) / 64, (T + 15) / 16, rs.ksplit), dim3(256), 0, stream, x,
                     w_router, T, d, E, rs.kchunk, partial, counts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const dim3 grid((T + 3) / 4), block(256);
  const int epl = (E + 63) / 64;
#define MOE_SELECT(N)                                                                                             \
  hipLaunchKernelGGL(k_route_select<N>, grid, block, 0, stream, partial, rs.ksplit, T, E, k, sel_bias, logit_bias, \
                     topk_ids, topk_weights, topk_gap, counts)
  if (epl <= 1) MOE_SELECT(1);
  else if (epl <= 2) MOE_SELECT(2);
  else if (epl <= 4) MOE_SELECT(4);
  else if (epl <= 5) MOE_SELECT(5);
  else if (epl <= 8) MOE_SELECT(8);
  else MOE_SELECT(16);
#undef MOE_SELECT
  return hipGetLastError();
}

size_t route_workspace_bytes(int T, int d, int E) {
  const RouteSplit rs = route_split(T, d, E);
  return (size_t)rs.ksplit * (size_t)T * (size_t)E * sizeof(float);
}

}  // namespace moe
