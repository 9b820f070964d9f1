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

// (score, expert) ordering of the selection: higher biased score first, equal
// scores go to the lower expert index.
__device__ __forceinline__ bool better(float b1, int e1, float b2, int e2) {
  return b1 > b2 || (b1 == b2 && e1 < e2);
}

}  // namespace

// Per-token selection.  One wave per token; lane l owns experts l, l+64, ...
// (EPL = experts per lane, E <= 64*EPL).  A block of four waves handles 16
// tokens and aggregates the expert histogram in LDS before one global atomic
// add per touched expert (integer atomics: order-independent).
template <int EPL>
__global__ __launch_bounds__(256) void k_route_select(const float* __restrict__ partial, int ksplit, int T, int E,
                                                      int k, const float* __restrict__ sel_bias,
                                                      const float* __restrict__ logit_bias,
                                                      int32_t* __restrict__ topk_ids,
                                                      float* __restrict__ topk_weights, float* __restrict__ topk_gap,
                                                      int32_t* __restrict__ counts) {
  __shared__ int hist[1024];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int wave = tid / kWave, lane = tid % kWave;
  const float neg_inf = -__builtin_huge_valf();
  for (int it = 0; it < 4; ++it) {
    const int t = blockIdx.x * 16 + it * 4 + wave;
    if (t >= T) continue;  // wave-uniform; no barrier inside the loop
    float beta[EPL], score[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane + kWave * j;
      if (e < E) {
        float z = 0.f;
        for (int ks = 0; ks < ksplit; ++ks) z += partial[((size_t)ks * T + t) * E + e];
        if (logit_bias) z += logit_bias[e];
        score[j] = 1.0f / (1.0f + __expf(-z));
        beta[j] = score[j] + sel_bias[e];
        if (beta[j] != beta[j]) beta[j] = neg_inf;  // NaN input: never preferred
      } else {
        score[j] = 0.f;
        beta[j] = neg_inf;
      }
    }
    // Selection rounds: the wave-wide best untaken expert each round.  Only
    // real experts (e < E) that are not yet taken are candidates, so the k ids
    // are always distinct and in range.
    unsigned taken = 0u;
    int my_id = 0;
    float my_s = 0.f, kth = 0.f, next = neg_inf;
    const int rounds = k < E ? k + 1 : k;
    for (int r = 0; r < rounds; ++r) {
      float bb = neg_inf, bs = 0.f;
      int be = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        const int e = lane + kWave * j;
        if (e < E && !((taken >> j) & 1u) && better(beta[j], e, bb, be)) {
          bb = beta[j];
          be = e;
          bs = score[j];
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ob = __shfl_xor(bb, off);
        const int oe = __shfl_xor(be, off);
        const float os = __shfl_xor(bs, off);
        if (better(ob, oe, bb, be)) {
          bb = ob;
          be = oe;
          bs = os;
        }
      }
      if (r < k) {
        if (lane == r) {
          my_id = be;
          my_s = bs;
        }
        if (be < E && (be & (kWave - 1)) == lane) taken |= 1u << (be >> 6);
        kth = bb;
      } else {
        next = bb;
      }
    }
    // Ascending expert order: rank of my id among the k chosen.
    int rank = 0;
    for (int q = 0; q < k; ++q) rank += (__shfl(my_id, q) < my_id) ? 1 : 0;
    float total = 0.f;
    for (int q = 0; q < k; ++q) {
      const unsigned long long m = __ballot(lane < k && rank == q);
      total += __shfl(my_s, __ffsll((long long)m) - 1);
    }
    if (lane < k) {
      topk_ids[(size_t)t * k + rank] = my_id;
      topk_weights[(size_t)t * k + rank] = my_s / total;
      atomicAdd(&hist[my_id], 1);
    }
    if (lane == 0 && topk_gap) topk_gap[t] = k < E ? kth - next : __builtin_huge_valf();
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
  const dim3 grid((T + 15) / 16), block(256);
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
