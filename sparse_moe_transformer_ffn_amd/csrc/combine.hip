// combine.hip -- weighted scatter-combine of the routed expert outputs plus
// the shared expert ([Blog] "Step 3.5 Flash: Open Frontier-Level Intelligence
// with 11B Active Parameters" §2.2: one always-on shared expert; §4.1.2:
// routed-expert aggregation is explicitly scaled), and the zero-centred
// RMSNorm used in front of FFN sub-layers ([Blog] §2.2, Figure 2 caption).
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

__device__ __forceinline__ void unpack8(u32x4 v, float* f) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f[2 * q] = __uint_as_float(v[q] << 16);
    f[2 * q + 1] = __uint_as_float(v[q] & 0xffff0000u);
  }
}

__device__ __forceinline__ u32x4 pack8(const float* f) {
  u32x4 v;
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = f32_to_bf16(f[2 * q]) | (f32_to_bf16(f[2 * q + 1]) << 16);
  return v;
}

}  // namespace

// One block per token; each thread owns 8 consecutive columns per step.  The
// k contributions are summed in slot order (ascending expert id), in f32;
// the k rows' loads of a step are all issued before the sums, so a step waits
// on one memory latency rather than k.
__global__ __launch_bounds__(256) void k_combine(const uint16_t* __restrict__ y_perm,
                                                 const int32_t* __restrict__ pair_pos,
                                                 const float* __restrict__ topk_weights,
                                                 const float* __restrict__ y_shared, float routed_scale, int d,
                                                 int k, uint16_t* __restrict__ y) {
  __shared__ int pos[kMaxTopK];
  __shared__ float wt[kMaxTopK];
  const int t = blockIdx.x, tid = threadIdx.x;
  if (tid < k) {
    pos[tid] = pair_pos[(size_t)t * k + tid];
    wt[tid] = topk_weights[(size_t)t * k + tid];
  }
  __syncthreads();
  for (int c = tid * 8; c < d; c += 256 * 8) {
    u32x4 rows[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
      if (j < k) rows[j] = load16(y_perm + (size_t)pos[j] * d + c);
    float4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    if (y_shared) {
      const float4* s = reinterpret_cast<const float4*>(y_shared + (size_t)t * d + c);
      s0 = s[0];
      s1 = s[1];
    }
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < k) {
        float v[8];
        unpack8(rows[j], v);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = fmaf(wt[j], v[q], acc[q]);
      }
    }
    float o[8];
    if (y_shared) {
      const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int q = 0; q < 8; ++q) o[q] = fmaf(routed_scale, acc[q], sv[q]);
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) o[q] = routed_scale * acc[q];
    }
    *reinterpret_cast<u32x4*>(y + (size_t)t * d + c) = pack8(o);
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
  const float total = (part[0] + part[1]) + (part[2] + part[3]);
  const float inv = 1.0f / sqrtf(total / (float)cols + eps);
  for (int c = tid * 8; c < cols; c += 256 * 8) {
    float v[8];
    unpack8(load16(src + c), v);
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = v[q] * inv * (gamma ? 1.0f + gamma[c + q] : 1.0f);
    *reinterpret_cast<u32x4*>(out + (size_t)row * cols + c) = pack8(v);
  }
}

hipError_t launch_combine(int T, int d, int k, const uint16_t* y_perm, const int32_t* pair_pos,
                          const float* topk_weights, const float* y_shared, float routed_scale, uint16_t* y,
                          hipStream_t stream) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(k_combine, dim3(T), dim3(256), 0, stream, y_perm, pair_pos, topk_weights, y_shared,
                     routed_scale, d, k, y);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(int rows, int cols, const uint16_t* in, const float* gamma, float eps, uint16_t* out,
                          hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(k_rmsnorm, dim3(rows), dim3(256), 0, stream, in, gamma, eps, cols, out);
  return hipGetLastError();
}

}  // namespace moe
