// common.h -- device helpers shared by libmoe's gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, one L2 each

__device__ __forceinline__ float bf16_to_f32(uint32_t v16) { return __uint_as_float(v16 << 16); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// float -> bf16, round to nearest even; NaN stays NaN (one
// v_cvt_pk_bf16_f32, gfx950's conversion instruction).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two floats -> two bf16 in one word, lo in bits 15:0 (one conversion).
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// 16x16x32 bf16 MFMA, f32 accumulate.  Operand lanes: lane l supplies row
// (l % 16) of A (and column (l % 16) of B) for the 8 reduction elements
// 8*(l/16) .. 8*(l/16)+7; any fixed assignment of reduction elements works as
// long as A and B use the same one.  Result: lane l holds D[4*(l/16)+i][l%16]
// for i = 0..3.
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ u32x4 load16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ float silu(float v) { return v / (1.0f + __expf(-v)); }

// SwiGLU hidden activation SiLU(g) * u, clipped to [-clamp, clamp] when
// clamp > 0 (activation clipping; off when clamp <= 0).
__device__ __forceinline__ float swiglu(float g, float u, float clamp) {
  const float v = silu(g) * u;
  return clamp > 0.f ? fminf(fmaxf(v, -clamp), clamp) : v;
}

// Eight bf16 values (one 16-byte load) <-> eight floats.
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
  for (int q = 0; q < 4; ++q) v[q] = pack2_bf16(f[2 * q], f[2 * q + 1]);
  return v;
}

// Zero-centred RMSNorm pieces, shared by every kernel that normalises rows
// so that they all produce the same bits: the inverse RMS from a row's sum
// of squares, and one normalised element v / rms * (1 + gamma_i).
__device__ __forceinline__ float rms_inv(float sum_sq, int cols, float eps) {
  return 1.0f / sqrtf(sum_sq / (float)cols + eps);
}

__device__ __forceinline__ float rms_scale(float v, float inv, const float* gamma, int i) {
  return v * inv * (gamma ? 1.0f + gamma[i] : 1.0f);
}

}  // namespace moe
