// combine.hip -- weighted scatter-combine of the routed expert outputs plus
// the shared expert ([Blog] "Step 3.5 Flash: Open Frontier-Level Intelligence
// with 11B Active Parameters" §2.2: one always-on shared expert; §4.1.2:
// routed-expert aggregation is explicitly scaled), and the zero-centred
// RMSNorm used in front of FFN sub-layers ([Blog] §2.2, Figure 2 caption).
#include "common.h"
#include "kernels.h"

namespace moe {

// One block per token; each thread owns 8 consecutive columns per step.  The
// k contributions are summed in slot order (ascending expert id), in f32;
// the k rows' loads of a step are all issued before the sums, so a step waits
// on one memory latency rather than k.  KMAX >= k bounds the rows held in
// registers (8 or kMaxTopK), which sets the occupancy.
//
// residual (NULL: none): the pre-norm block's skip connection, added to the
// f32 result before its one rounding to bf16.  It may alias y (neither is
// declared restrict): each thread reads its 16 bytes before writing them.
//
// DIAG: the rows are already in registers, so the block also forms each
// row's sum of squares (f32: per thread in column order, then a butterfly
// over the wave and the four waves in order) and stores it by permuted row,
// row_ss[pair_pos[t*k+j]], and for the shared expert's row, shared_ss[t].
// NT: non-temporal loads of the routed and shared rows and non-temporal
// stores of y, for large batches where nothing of them is read again soon
// (k = 8, d = 4,096, 8,192 tokens: 145 -> 125 us; at 64 tokens the plain
// policy is 0.2-0.5 us faster).
template <int KMAX, bool DIAG, bool NT>
__global__ __launch_bounds__(256) void k_combine(const uint16_t* __restrict__ y_perm,
                                                 const int32_t* __restrict__ pair_pos,
                                                 const float* __restrict__ topk_weights,
                                                 const float* __restrict__ y_shared,
                                                 const uint16_t* residual, float routed_scale, int d, int k,
                                                 uint16_t* y, float* __restrict__ row_ss,
                                                 float* __restrict__ shared_ss) {
  __shared__ int pos[KMAX];
  __shared__ float wt[KMAX];
  __shared__ float ss_part[DIAG ? 4 : 1][KMAX + 1];
  const int t = blockIdx.x, tid = threadIdx.x;
  if (tid < k) {
    pos[tid] = pair_pos[(size_t)t * k + tid];
    wt[tid] = topk_weights[(size_t)t * k + tid];
  }
  __syncthreads();
  float ss[KMAX + 1];
#pragma unroll
  for (int j = 0; j <= KMAX; ++j) ss[j] = 0.f;
  for (int c = tid * 8; c < d; c += 256 * 8) {
    u32x4 rows[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (j < k)
        rows[j] = NT ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(y_perm + (size_t)pos[j] * d + c))
                     : load16(y_perm + (size_t)pos[j] * d + c);
    float4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    if (y_shared) {
      const float4* s = reinterpret_cast<const float4*>(y_shared + (size_t)t * d + c);
      if constexpr (NT) {
        const f32x4* sv = reinterpret_cast<const f32x4*>(s);
        const f32x4 a0 = __builtin_nontemporal_load(sv), a1 = __builtin_nontemporal_load(sv + 1);
        s0 = make_float4(a0[0], a0[1], a0[2], a0[3]);
        s1 = make_float4(a1[0], a1[1], a1[2], a1[3]);
      } else {
        s0 = s[0];
        s1 = s[1];
      }
    }
    const u32x4 res = residual ? load16(residual + (size_t)t * d + c) : u32x4{0u, 0u, 0u, 0u};
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j < k) {
        float v[8];
        unpack8(rows[j], v);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = fmaf(wt[j], v[q], acc[q]);
        if constexpr (DIAG) {
#pragma unroll
          for (int q = 0; q < 8; ++q) ss[j] = fmaf(v[q], v[q], ss[j]);
        }
      }
    }
    float o[8];
    if (y_shared) {
      const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int q = 0; q < 8; ++q) o[q] = fmaf(routed_scale, acc[q], sv[q]);
      if constexpr (DIAG) {
#pragma unroll
        for (int q = 0; q < 8; ++q) ss[KMAX] = fmaf(sv[q], sv[q], ss[KMAX]);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) o[q] = routed_scale * acc[q];
    }
    if (residual) {
      float rv[8];
      unpack8(res, rv);
#pragma unroll
      for (int q = 0; q < 8; ++q) o[q] = rv[q] + o[q];
    }
    if constexpr (NT) __builtin_nontemporal_store(pack8(o), reinterpret_cast<u32x4*>(y + (size_t)t * d + c));
    else *reinterpret_cast<u32x4*>(y + (size_t)t * d + c) = pack8(o);
  }
  if constexpr (DIAG) {
    const int wave = tid / kWave, lane = tid % kWave;
#pragma unroll
    for (int j = 0; j <= KMAX; ++j) {
      if (j < k || (j == KMAX && y_shared)) {
        float v = ss[j];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
        if (lane == 0) ss_part[wave][j < k ? j : k] = v;
      }
    }
    __syncthreads();
    if (tid <= k) {
      const float v = (ss_part[0][tid] + ss_part[1][tid]) + (ss_part[2][tid] + ss_part[3][tid]);
      if (tid < k) row_ss[pos[tid]] = v;
      else if (y_shared) shared_ss[t] = v;
    }
  }
}

// Per-expert activation RMS from the row sums of squares: block e adds the
// rows of expert e (entry E: the shared expert's T rows) in double, in a
// fixed order (thread-strided with four loads in flight, then a tree), and
// takes sqrt(sum / (rows * d)); no rows gives 0.
__global__ __launch_bounds__(256) void k_expert_rms(const float* __restrict__ row_ss,
                                                    const float* __restrict__ shared_ss,
                                                    const int32_t* __restrict__ offsets, int T, int E, int d,
                                                    float* __restrict__ rms) {
  __shared__ double red[256];
  const int e = blockIdx.x, tid = threadIdx.x;
  const float* src;
  int n;
  if (e < E) {
    src = row_ss + offsets[e];
    n = offsets[e + 1] - offsets[e];
  } else {
    src = shared_ss;
    n = shared_ss ? T : 0;
  }
  double s = 0.0;
  for (int r0 = 0; r0 < n; r0 += 1024) {
    float v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = r0 + q * 256 + tid;
      v[q] = r < n ? src[r] : 0.f;
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
  if (tid == 0) rms[e] = n > 0 ? (float)sqrt(red[0] / ((double)n * d)) : 0.f;
}

// Spread of the routed experts' RMS ([Blog] §4.1.3, Figure 4: maximum against
// median expert output norm; [Digest] expert collapse: min against median):
// over the experts that received rows, ratio = (min, max) / median, the
// median of an even count being the mean of the two middle values.  No such
// expert, or a zero median, gives (0, 0).  One block; order statistics by
// rank counting (ties broken by expert index) over keys that are the RMS of
// the experts with rows and +inf for the others and the padding.
__global__ __launch_bounds__(1024) void k_rms_ratio(const float* __restrict__ rms,
                                                    const int32_t* __restrict__ offsets, int E,
                                                    float* __restrict__ ratio) {
  __shared__ __attribute__((aligned(16))) float key[1024];
  __shared__ float sorted[1024];
  __shared__ int used;
  const int tid = threadIdx.x;
  const int E4 = (E + 3) / 4 * 4;
  if (tid == 0) used = 0;
  __syncthreads();
  if (tid < E4) {
    const bool has = tid < E && offsets[tid + 1] > offsets[tid];
    key[tid] = has ? rms[tid] : __builtin_huge_valf();
    if (has) atomicAdd(&used, 1);
  }
  __syncthreads();
  const int m = used;
  if (tid < E && key[tid] != __builtin_huge_valf()) {
    const float ke = key[tid];
    int rank = 0;
#pragma unroll 4
    for (int j4 = 0; j4 < E4; j4 += 4) {
      const float4 kj = *reinterpret_cast<const float4*>(&key[j4]);
      rank += (kj.x < ke || (kj.x == ke && j4 < tid)) + (kj.y < ke || (kj.y == ke && j4 + 1 < tid)) +
              (kj.z < ke || (kj.z == ke && j4 + 2 < tid)) + (kj.w < ke || (kj.w == ke && j4 + 3 < tid));
    }
    sorted[rank] = ke;
  }
  __syncthreads();
  if (tid == 0) {
    const double med = m == 0 ? 0.0 : 0.5 * ((double)sorted[(m - 1) / 2] + (double)sorted[m / 2]);
    if (m == 0 || !(med > 0.0)) {
      ratio[0] = ratio[1] = 0.f;
    } else {
      ratio[0] = (float)((double)sorted[0] / med);
      ratio[1] = (float)((double)sorted[m - 1] / med);
    }
  }
}

// One block per row: sum of squares in f32, then scale and round to bf16.
__global__ __launch_bounds__(256) void k_rmsnorm(const uint16_t* __restrict__ in, const float* __restrict__ gamma,
                                                 float eps, int cols, uint16_t* __restrict__ out) {
  __shared__ float part[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  const uint16_t* src = in + (size_t)row * cols;
  float ss = 0.f;
  for (int c = tid * 8; c < cols; c += 256 * 8) {
    float v[8];
    unpack8(load16(src + c), v);
#pragma unroll
    for (int q = 0; q < 8; ++q) ss = fmaf(v[q], v[q], ss);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  if (tid % kWave == 0) part[tid / kWave] = ss;
  __syncthreads();
  const float inv = rms_inv((part[0] + part[1]) + (part[2] + part[3]), cols, eps);
  for (int c = tid * 8; c < cols; c += 256 * 8) {
    float v[8];
    unpack8(load16(src + c), v);
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = rms_scale(v[q], inv, gamma, c + q);
    *reinterpret_cast<u32x4*>(out + (size_t)row * cols + c) = pack8(v);
  }
}

hipError_t launch_combine(int T, int d, int k, const uint16_t* y_perm, const int32_t* pair_pos,
                          const float* topk_weights, const float* y_shared, const uint16_t* residual,
                          float routed_scale, uint16_t* y, const CombineDiag* diag, void* workspace,
                          hipStream_t stream) {
  float* row_ss = diag ? static_cast<float*>(workspace) : nullptr;
  float* shared_ss = diag && y_shared ? row_ss + (size_t)T * k : nullptr;
  hipError_t err;
  if (T > 0) {
    // Non-temporal from 64 MB of routed rows.
    const bool nt = (size_t)T * k * d * sizeof(uint16_t) >= ((size_t)64 << 20);
#define MOE_COMBINE(KMAX, DIAG)                                                                                    \
  do {                                                                                                             \
    if (nt)                                                                                                        \
      hipLaunchKernelGGL((k_combine<KMAX, DIAG, true>), dim3(T), dim3(256), 0, stream, y_perm, pair_pos,           \
                         topk_weights, y_shared, residual, routed_scale, d, k, y, row_ss, shared_ss);              \
    else                                                                                                           \
      hipLaunchKernelGGL((k_combine<KMAX, DIAG, false>), dim3(T), dim3(256), 0, stream, y_perm, pair_pos,          \
                         topk_weights, y_shared, residual, routed_scale, d, k, y, row_ss, shared_ss);              \
  } while (0)
    if (k <= 8) {
      if (diag) MOE_COMBINE(8, true);
      else MOE_COMBINE(8, false);
    } else {
      if (diag) MOE_COMBINE(kMaxTopK, true);
      else MOE_COMBINE(kMaxTopK, false);
    }
#undef MOE_COMBINE
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (!diag) return hipSuccess;
  hipLaunchKernelGGL(k_expert_rms, dim3(diag->E + 1), dim3(256), 0, stream, row_ss, shared_ss, diag->offsets, T,
                     diag->E, d, diag->rms);
  if ((err = hipGetLastError()) != hipSuccess || !diag->ratio) return err;
  hipLaunchKernelGGL(k_rms_ratio, dim3(1), dim3(1024), 0, stream, diag->rms, diag->offsets, diag->E, diag->ratio);
  return hipGetLastError();
}

// Row sums of squares: T*k routed rows, then T shared rows.
size_t combine_diag_workspace_bytes(int T, int k) { return (size_t)T * (k + 1) * sizeof(float); }

hipError_t launch_rmsnorm(int rows, int cols, const uint16_t* in, const float* gamma, float eps, uint16_t* out,
                          hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(k_rmsnorm, dim3(rows), dim3(256), 0, stream, in, gamma, eps, cols, out);
  return hipGetLastError();
}

}  // namespace moe
