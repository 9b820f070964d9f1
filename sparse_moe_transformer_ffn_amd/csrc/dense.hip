// dense.hip -- the SwiGLU FFN of one group holding every token (the dense FFN
// of [Digest] "Step 3.5 Flash 技术论文深度解读" architecture table, hidden
// 11,264) at up to 64 tokens, bf16 MFMA 16x16x32 (gfx950).
//
// At this size both projections stream their weights once from HBM (a
// 64-token batch does 64 flops per weight element), so each CU should read a
// fixed share of the weights and little else.  One block (4 waves, one per
// SIMD, each with the SIMD's 512 registers) per CU:
// - gate/up: block b owns hidden units [U b, U b + U) (U = 4G: 44 at hidden
//   11,264 on 256 CUs), i.e. 2U weight rows; its waves split the d-long
//   reduction four ways, so each token element is read once per CU.  The
//   four sums meet in LDS, SwiGLU is applied and the hidden rows stored.
// - down: block (c, q) owns output columns [64 c, 64 c + 64) over the q-th
//   of kDenseDownSplits ranges of the hidden-long reduction (64 column groups
//   x 4 = 256 blocks at d = 4,096), the waves splitting that range again; the
//   ranges' f32 sums are added in range order by a third small launch.
// Inside a block the waves' sums meet in LDS in a fixed tree (w += w + 2,
// then w += w + 1), so results do not depend on the schedule.
//
// One cooperative launch of both phases with a grid barrier in between
// measured slower (83 vs 68 us at 64 tokens): every block's device-scope
// release and acquire writes back and invalidates its XCD's L2, which costs
// more than the launch boundaries it replaces.
#include "common.h"
#include "grouped.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kDenseWaves = 4;  // one per SIMD: each wave may hold 512 registers
constexpr int kDenseThreads = kDenseWaves * kWave;
constexpr int kRedPad = 4;      // floats of padding per LDS row of partial sums

// Range [b0, b1) of part p when n items are split into `parts` contiguous
// ranges as evenly as possible (the first n % parts ranges one longer).
__device__ __forceinline__ void split_range(int n, int parts, int p, int& b0, int& b1) {
  const int q = n / parts, r = n % parts;
  b0 = p * q + (p < r ? p : r);
  b1 = b0 + q + (p < r ? 1 : 0);
}

// Partial sums in LDS, column-major: red[w][column][token], so that a lane's
// four consecutive tokens of one column (element i of acc[t][mb]: token
// 16 mb + 4 (lane / 16) + i, column 16 t + lane % 16) are one 16-byte access,
// and 16 lanes of consecutive columns (rows 4 (MB 16 + kRedPad) bytes apart)
// cover all banks.
template <int MB, int NT>
using Red = float[NT * 16][MB * 16 + kRedPad];

template <int MB, int NT>
__device__ __forceinline__ f32x4* red_at(Red<MB, NT>* red, int w, int t, int mb, int lane) {
  return reinterpret_cast<f32x4*>(&red[w][16 * t + (lane & 15)][16 * mb + 4 * (lane >> 4)]);
}

// Sum of the four waves' accumulators in a fixed order (w += w + 2, then
// w += w + 1): wave 0's acc holds the block's sums afterwards, and with
// STORE also red[0].
template <int MB, int NT, bool STORE>
__device__ __forceinline__ void tree_sum(f32x4 (&acc)[NT][MB], Red<MB, NT>* red, int wave, int lane) {
#pragma unroll
  for (int half = kDenseWaves / 2; half >= 1; half /= 2) {
    if (wave >= half && wave < 2 * half) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) *red_at<MB, NT>(red, wave - half, t, mb, lane) = acc[t][mb];
    }
    __syncthreads();
    if (wave < half) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[t][mb] += *red_at<MB, NT>(red, wave, t, mb, lane);
    }
    __syncthreads();
  }
  if (STORE) {
    if (wave == 0) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) *red_at<MB, NT>(red, 0, t, mb, lane) = acc[t][mb];
    }
    __syncthreads();
  }
}

// One wave's reduction over K blocks kb0 .. kb0 + n - 1 (64 elements each):
// G groups of 8 weight rows times MB tiles of 16 token rows, into acc[t][mb]
// for weight tiles t = groups 2t, 2t + 1.
// - Weights: whole 128-byte lines into registers, lane l holding row l / 8
//   of a group at 16-byte segment (l % 8) ^ (l / 8) of the block; wsrc[g] is
//   the lane's source for block 0.  Before its multiplies a block's lines
//   are written to this wave's LDS patch (lane l at bytes 16 l .. of the
//   group's KiB, so the XOR spreads a column of 8 rows over all banks) and
//   read back in the MFMA layout, one 16-byte read per tile and step.
// - Token rows: registers in the MFMA layout, lane l holding row l % 16 of a
//   tile at elements 8 (l / 16) .. +7 of each 32-wide step; xsrc[mb] is the
//   lane's source for block 0.
// The registers form rings: weights kRingW blocks deep, token rows kRingX;
// block j's slots are reloaded with blocks j + kRingW / j + kRingX right
// after its multiplies have read them, so each wave keeps about 33 KiB of
// weights in flight (one wave per SIMD has 512 registers for it).  Every
// load is unconditional (lanes without a row or token read a valid one whose
// results are never stored), and scheduling barriers keep each block's loads
// behind its reads, so the compiler's wait for block j counts exactly the
// loads issued after it.
constexpr int kRingW = 3, kRingX = 2, kPeriod = 6;  // kPeriod = lcm(kRingW, kRingX)

template <int MB, int G>
struct Stream {
  static constexpr int NT = (G + 1) / 2;
  const uint16_t* wsrc[G];
  const uint16_t* xsrc[MB];
  uint16_t* patch;  // this wave's 2 NT KiB of LDS
  int wr;           // lane's LDS element offset of its line writes (group 0)
  int rd[2];        // lane's LDS element offset of its B operand, per step (tile 0)
  bool zero_hi;     // lane reads the missing upper group of the last tile (odd G)
  u32x4 L[kRingW][G];
  u32x4 A[kRingX][MB][2];

  template <int SW>
  __device__ __forceinline__ void issue_w(int kb) {
#pragma unroll
    for (int g = 0; g < G; ++g)
      L[SW][g] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wsrc[g] + 64 * kb));
    __builtin_amdgcn_sched_barrier(0);
  }
  template <int SX>
  __device__ __forceinline__ void issue_x(int kb) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int s = 0; s < 2; ++s) A[SX][mb][s] = load16(xsrc[mb] + 64 * kb + 32 * s);
    __builtin_amdgcn_sched_barrier(0);
  }

  template <int SW, int SX>
  __device__ __forceinline__ void compute(f32x4 (&acc)[NT][MB]) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int g = 0; g < G; ++g) *reinterpret_cast<u32x4*>(patch + wr + 512 * g) = L[SW][g];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4 b[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) b[t] = *reinterpret_cast<const u32x4*>(patch + rd[s] + 1024 * t);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const u32x4 bt = 2 * t + 1 == G && zero_hi ? zero : b[t];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[t][mb] = mfma_16x16x32(A[SX][mb][s], bt, acc[t][mb]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // Block j = j0 + R (R = j % kPeriod), then the reloads it frees.
  template <int R>
  __device__ __forceinline__ void step(int kb0, int n, int j0, bool guard, f32x4 (&acc)[NT][MB]) {
    const int j = j0 + R;
    if (guard && j >= n) return;
    compute<R % kRingW, R % kRingX>(acc);
    if (!guard || j + kRingW < n) issue_w<R % kRingW>(kb0 + j + kRingW);
    if (!guard || j + kRingX < n) issue_x<R % kRingX>(kb0 + j + kRingX);
  }

  template <int R = 0>
  __device__ __forceinline__ void period(int kb0, int n, int j0, bool guard, f32x4 (&acc)[NT][MB]) {
    if constexpr (R < kPeriod) {
      step<R>(kb0, n, j0, guard, acc);
      period<R + 1>(kb0, n, j0, guard, acc);
    }
  }

  // The reduction over n blocks.
  __device__ __forceinline__ void run(int kb0, int n, f32x4 (&acc)[NT][MB]) {
    if (n < kRingW) {  // too short for the ring: one block at a time
      for (int j = 0; j < n; ++j) {
        issue_w<0>(kb0 + j);
        issue_x<0>(kb0 + j);
        compute<0, 0>(acc);
      }
      return;
    }
    issue_w<0>(kb0);
    issue_w<1>(kb0 + 1);
    issue_w<2>(kb0 + 2);
    issue_x<0>(kb0);
    issue_x<1>(kb0 + 1);
    int j0 = 0;
    // Whole periods whose every step reloads both rings.
    for (; j0 + kPeriod + kRingW <= n; j0 += kPeriod) period(kb0, n, j0, false, acc);
    for (; j0 < n; j0 += kPeriod) period(kb0, n, j0, true, acc);
  }
};

// Lane constants of a Stream: weight row of group g = row(g, lane / 8) (row
// length K), token row of tile mb = 16 mb + lane % 16 (clamped to row 0 from
// T on), and the LDS offsets.
template <int MB, int G, typename RowOf>
__device__ __forceinline__ void stream_setup(Stream<MB, G>& st, const uint16_t* w, int K, RowOf row,
                                             const uint16_t* xs, int T, uint16_t* patch) {
  const int lane = threadIdx.x % kWave;
  const int r8 = lane >> 3, sl = lane & 7;
#pragma unroll
  for (int g = 0; g < G; ++g) st.wsrc[g] = w + (size_t)row(g, r8) * K + 8 * (sl ^ r8);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int t = 16 * mb + (lane & 15);
    st.xsrc[mb] = xs + (size_t)(t < T ? t : 0) * K + 8 * (lane >> 4);
  }
  st.patch = patch;
  st.wr = 8 * lane;
  const int c = lane & 15, rr = c & 7;
#pragma unroll
  for (int s = 0; s < 2; ++s) st.rd[s] = (c >> 3) * 512 + rr * 64 + (((4 * s + (lane >> 4)) ^ rr) * 8);
  st.zero_hi = c >= 8;
}

// LDS of a kernel: each wave's patch of 2 NT KiB (G rounded up to even: the
// B reads of an odd G's last tile cover the missing group's KiB too, whose
// values are replaced by zeros; 8 KiB for down), the same memory holding the
// partial sums of tree_sum afterwards.
template <int MB, int G>
struct DenseLds {
  static constexpr int NT = (G + 1) / 2;
  static constexpr int kPatchPerWave = 2 * NT * 512;                                    // uint16 elements
  static constexpr int kPatch = kDenseWaves * (2 * NT > 8 ? 2 * NT : 8) * 512;          // uint16 elements
  static constexpr int kRedGu = (kDenseWaves / 2) * NT * 16 * (MB * 16 + kRedPad) * 2;  // uint16 elements
  static constexpr int kRedDown = (kDenseWaves / 2) * 4 * 16 * (MB * 16 + kRedPad) * 2;
  static constexpr int kSize = kPatch > kRedGu ? (kPatch > kRedDown ? kPatch : kRedDown)
                                               : (kRedGu > kRedDown ? kRedGu : kRedDown);
};

// Gate/up: hid[t][u] = SwiGLU(x_t . W[u], x_t . W[H + u]) for the block's
// units u in [U b, U b + U) ∩ [0, H), U = 4G.  Column (slot) s of the block's
// 8G columns is gate row U b + s for s < U and up row H + U b + s - U for
// s >= U (slots of units past H read row 0 and are never stored).
template <int MB, int G>
__global__ __launch_bounds__(kDenseThreads, 1) void k_dense_gate_up(const uint16_t* __restrict__ x, int T, int d,
                                                                    int H, const uint16_t* __restrict__ w_gu,
                                                                    uint16_t* __restrict__ hid, float clamp) {
  constexpr int U = 4 * G;
  using Lds = DenseLds<MB, G>;
  constexpr int NT = Lds::NT;
  __shared__ __attribute__((aligned(16))) uint16_t lds[Lds::kSize];
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int u0 = blockIdx.x * U, nu = min(U, H - u0);
  int b0, b1;
  split_range(d / 64, kDenseWaves, wave, b0, b1);
  Stream<MB, G> st;
  stream_setup(st, w_gu, d,
               [&](int g, int r8) {
                 const int s = 8 * g + r8;
                 const int u = s < U ? s : s - U;
                 return u < nu ? (s < U ? u0 + u : H + u0 + u) : 0;
               },
               x, T, lds + wave * Lds::kPatchPerWave);
  f32x4 acc[NT][MB];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[t][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.run(b0, b1 - b0, acc);
  __syncthreads();  // the patches become the partial sums
  auto red = reinterpret_cast<Red<MB, NT>*>(lds);
  tree_sum<MB, NT, true>(acc, red, wave, lane);
  // Lane u < nu of each wave: unit u0 + u of tokens wave, wave + 4, ...
  if (lane < nu) {
#pragma unroll 4
    for (int t = wave; t < T; t += kDenseWaves)
      hid[(size_t)t * H + u0 + lane] = (uint16_t)f32_to_bf16(swiglu(red[0][lane][t], red[0][U + lane][t], clamp));
  }
}

// Down: block (c, q) = (blockIdx / KQ, blockIdx % KQ) sums hid[t] . W_d[n]
// for columns n in [64 c, 64 c + 64) over the q-th of KQ ranges of the H / 64
// K blocks into out[q][t][n] (f32, row stride d).  Blocks b and b + 8 run on
// the same XCD, so with KQ dividing 8 an XCD's blocks share one range of the
// hidden rows in its L2.
template <int MB>
__global__ __launch_bounds__(kDenseThreads, 1) void k_dense_down(const uint16_t* __restrict__ hid, int T, int d,
                                                                 int H, int KQ, const uint16_t* __restrict__ w_d,
                                                                 float* __restrict__ out) {
  using Lds = DenseLds<MB, 8>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[Lds::kSize];
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int q = blockIdx.x % KQ, n0 = (blockIdx.x / KQ) * 64;
  int r0, r1, b0, b1;
  split_range(H / 64, KQ, q, r0, r1);
  split_range(r1 - r0, kDenseWaves, wave, b0, b1);
  Stream<MB, 8> st;
  stream_setup(st, w_d, H, [&](int g, int r8) { return n0 + 8 * g + r8; }, hid, T, lds + wave * 8 * 512);
  f32x4 acc[4][MB];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[t][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.run(r0 + b0, b1 - b0, acc);
  __syncthreads();
  auto red = reinterpret_cast<Red<MB, 4>*>(lds);
  tree_sum<MB, 4, false>(acc, red, wave, lane);
  // Wave 0 stores the block's sums straight from its accumulators.
  if (wave == 0) {
    float* o = out + (size_t)q * T * d + n0 + (lane & 15);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = 16 * mb + 4 * (lane >> 4) + i;
          if (tok < T) o[(size_t)tok * d + 16 * t] = acc[t][mb][i];
        }
  }
}

// y[i] = sum over q < KQ of P[q][i], in q order (n a multiple of 4).
__global__ __launch_bounds__(256) void k_dense_sum(const float* __restrict__ P, int KQ, size_t n,
                                                   float* __restrict__ y) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n / 4; i += (size_t)gridDim.x * 256) {
    float4 s = reinterpret_cast<const float4*>(P)[i];
    for (int q = 1; q < KQ; ++q) {
      const float4 v = reinterpret_cast<const float4*>(P + q * n)[i];
      s.x += v.x, s.y += v.y, s.z += v.z, s.w += v.w;
    }
    reinterpret_cast<float4*>(y)[i] = s;
  }
}

// Line groups (of 8 rows) per gate/up block: the smallest of kGroupChoices
// whose 4G units per block cover the hidden size on `blocks` blocks; 0 if
// none does.
constexpr int kGroupChoices[] = {4, 6, 8, 10, 11};

int dense_groups(int H, int blocks) {
  for (int G : kGroupChoices)
    if ((long)4 * G * blocks >= H) return G;
  return 0;
}

int dense_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 1;
    cus[dev] = n;
  }
  return cus[dev];
}

template <int MB, int G>
hipError_t launch_g(int T, int d, int H, const uint16_t* x, const uint16_t* w_gu, uint16_t* hid, float clamp,
                    hipStream_t stream) {
  hipLaunchKernelGGL((k_dense_gate_up<MB, G>), dim3((H + 4 * G - 1) / (4 * G)), dim3(kDenseThreads), 0, stream, x, T,
                     d, H, w_gu, hid, clamp);
  return hipGetLastError();
}

template <int MB>
hipError_t launch_mb(int T, int d, int H, const uint16_t* x, const uint16_t* w_gu, const uint16_t* w_d, uint16_t* hid,
                     float* partial, float* y, float clamp, hipStream_t stream) {
  hipError_t err;
  switch (dense_groups(H, dense_cus())) {
    case 4: err = launch_g<MB, 4>(T, d, H, x, w_gu, hid, clamp, stream); break;
    case 6: err = launch_g<MB, 6>(T, d, H, x, w_gu, hid, clamp, stream); break;
    case 8: err = launch_g<MB, 8>(T, d, H, x, w_gu, hid, clamp, stream); break;
    case 10: err = launch_g<MB, 10>(T, d, H, x, w_gu, hid, clamp, stream); break;
    default: err = launch_g<MB, 11>(T, d, H, x, w_gu, hid, clamp, stream); break;
  }
  if (err != hipSuccess) return err;
  const int KQ = kDenseDownSplits;
  hipLaunchKernelGGL(k_dense_down<MB>, dim3(d / 64 * KQ), dim3(kDenseThreads), 0, stream, hid, T, d, H, KQ, w_d,
                     partial);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const size_t n = (size_t)T * d, blocks = (n / 4 + 255) / 256;
  hipLaunchKernelGGL(k_dense_sum, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, stream, partial, KQ,
                     n, y);
  return hipGetLastError();
}

}  // namespace

bool dense_ffn_fits(int T, int d, int H) {
  if (T < 1 || T > kDenseMaxTokens || d % 64 || H % 64) return false;
  const int cus = dense_cus();
  // At least 16 units per CU (else the token rows outweigh the weights) and a
  // down range of at least one K block per wave.
  return dense_groups(H, cus) > 0 && (long)16 * cus <= H && H / 64 >= kDenseWaves * kDenseDownSplits;
}

hipError_t launch_dense_ffn(int T, int d, int H, const uint16_t* x, const uint16_t* w_gu, const uint16_t* w_d,
                            uint16_t* hid, float* partial, float* y, float clamp, hipStream_t stream) {
  if (T <= 16) return launch_mb<1>(T, d, H, x, w_gu, w_d, hid, partial, y, clamp, stream);
  if (T <= 32) return launch_mb<2>(T, d, H, x, w_gu, w_d, hid, partial, y, clamp, stream);
  if (T <= 48) return launch_mb<3>(T, d, H, x, w_gu, w_d, hid, partial, y, clamp, stream);
  return launch_mb<4>(T, d, H, x, w_gu, w_d, hid, partial, y, clamp, stream);
}

}  // namespace moe
