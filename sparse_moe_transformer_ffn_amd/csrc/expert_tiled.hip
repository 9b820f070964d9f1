// expert_tiled.hip -- grouped SwiGLU expert GEMMs for the compute regime
// (hundreds of rows per expert: prefill-sized batches), bf16 MFMA 32x32x16.
//
// Layer definition as in expert.hip ([Digest] "Step 3.5 Flash 技术论文深度解读"
// architecture table and activation-explosion cause 3; grouped layout after
// [Blog] "Step 3.5 Flash: Open Frontier-Level Intelligence with 11B Active
// Parameters" §3.2.4).
//
// Block = 4 waves; item = 128 token rows x 256 weight rows:
//   gate/up: 128 gate rows j0.. and the 128 matching up rows h+j0.. of W_gu;
//   down:    256 rows n0.. of W_d.
// Wave (wm, wn) = (wave % 2, wave / 2) owns rows [64 wm, 64 wm + 64) of the
// M-tile and 128 of the columns: gate/up units [64 wn, 64 wn + 64) of both
// halves (so SiLU(G) * U pairs sit in the same lane), or down columns
// [128 wn, 128 wn + 128).  That is 2 x 4 MFMA 32x32x16 tiles, 128 f32
// accumulators per lane, 0.75 KiB of LDS reads per MFMA.
//
// Work order (grouped.h): M-tiles fastest in bands of up to 4, so the blocks
// that run side by side on one XCD share a weight slab (one HBM read, the
// band's other M-tiles hit L2) while the token rows they touch stay within a
// few MiB of the XCD's 4 MiB L2.
//
// Operand staging.  Both operands go from HBM/L2 straight into LDS with the
// gfx950 direct-to-LDS load (global_load_lds_dwordx4: lane l of a wave writes
// its 16 bytes at LDS base + 16*l), through a ring of three stages of 64-wide
// K chunks (A 128x64 + B 256x64 bf16 = 48 KiB per stage), so two chunks are in
// flight while the third is multiplied, with no register staging.  A row of
// 64 elements is 8 16-byte segments; segment s of row r is stored at slot
// s ^ ((r >> 1) & 7), so a wave's 16-byte reads of one segment of 16
// consecutive rows hit 16 distinct bank groups.  The direct loads choose
// their source segment to produce that layout.  Each thread issues 12 direct
// loads per chunk (4 for A, 8 for B); before a stage is read each thread waits
// until only the newer chunk's 12 are outstanding, then the block barrier
// makes every thread's part visible (a bare s_barrier: no release fence,
// which would drain the loads in flight).  The three stages are distinct LDS
// arrays and the K loop is unrolled by three so the compiler sees which stage
// each read uses.  Token rows past the group's end load the group's first
// row (their results are never stored); waves whose 64 rows all lie past the
// end skip their MFMAs but still issue their share of the loads and join the
// barriers.
//
// MFMA 32x32x16 operands: lane l supplies row (l % 32) of A / column (l % 32)
// of B for the 8 reduction elements 8*(l/32) .. +7 of the 16; result element
// i of lane l is D[8*(i/4) + 4*(l/32) + (i%4)][l % 32].
#include "common.h"
#include "grouped.h"
#include "kernels.h"

namespace moe {

typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

constexpr int kThreads = 256;
constexpr int kTileM = 128;
constexpr int kTileN = 256;                  // weight rows per item
constexpr int kBand = 4;                     // M-tiles per band of the work order
constexpr int kChunk = 64;                   // K elements per stage
constexpr int kSegs = kChunk / 8;            // 16-byte segments per row
constexpr int kStageA = kTileM * kChunk;     // bf16 elements
constexpr int kStageB = kTileN * kChunk;
constexpr int kStage = kStageA + kStageB;    // 48 KiB
constexpr int kRegionRows = 64 / kSegs;      // rows written by one wave-wide direct load
constexpr int kLoadsA = kTileM / kRegionRows / 4;  // per thread per chunk
constexpr int kLoadsB = kTileN / kRegionRows / 4;
constexpr int kLoadsPerChunk = kLoadsA + kLoadsB;  // 12

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4 and lgkmcnt 11:8 left at their maxima).
constexpr int kWaitNextChunk = 0x0F70 | kLoadsPerChunk;
constexpr int kWaitAll = 0x0F70;  // vmcnt(0)

// Cache policy of the direct loads: the default for both operands.  Token rows
// are re-read by every N-tile of their M-tile and weight rows by every M-tile
// of their band, both through L2 (a non-temporal hint on the weight rows
// measured slower: it defeats the sharing within a band).
constexpr int kPolicyReuse = 0;
constexpr int kPolicyStream = 0;

__device__ __forceinline__ f32x16 mfma_32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

enum Phase { kGateUp = 0, kDown = 1 };

struct Pipe {
  const uint16_t* src[kLoadsPerChunk];  // per-thread source of each direct load (chunk 0)
  int lds_off[kLoadsPerChunk];          // wave-uniform LDS element offset inside a stage
};

__device__ __forceinline__ void issue_chunk(const Pipe& p, uint16_t* stage, int c) {
#pragma unroll
  for (int q = 0; q < kLoadsA; ++q)
    __builtin_amdgcn_global_load_lds(p.src[q] + c * kChunk, stage + p.lds_off[q], 16, 0, kPolicyReuse);
#pragma unroll
  for (int q = kLoadsA; q < kLoadsPerChunk; ++q)
    __builtin_amdgcn_global_load_lds(p.src[q] + c * kChunk, stage + p.lds_off[q], 16, 0, kPolicyStream);
}

// LDS rows this lane reads: A rows of its two M-subtiles, B rows of its four
// N-subtiles (all with swz(row) = swz(l32)).
struct ReadMap {
  int a_row[2], b_row[4];
};

// Fragments of one 16-wide K step.
struct Frags {
  u32x4 a[2], b[4];
};

__device__ __forceinline__ void read_frags(const uint16_t* stage, const ReadMap& m, int s, int lhi, int f,
                                           Frags& fr) {
  const int slot = ((2 * s + lhi) ^ f) * 8;
#pragma unroll
  for (int ms = 0; ms < 2; ++ms) fr.a[ms] = *reinterpret_cast<const u32x4*>(&stage[m.a_row[ms] * kChunk + slot]);
#pragma unroll
  for (int ns = 0; ns < 4; ++ns)
    fr.b[ns] = *reinterpret_cast<const u32x4*>(&stage[kStageA + m.b_row[ns] * kChunk + slot]);
}

// One 64-wide K chunk (four MFMA steps) from `stage` into the accumulators.
// The fragments of step s+1 are read before the MFMAs of step s are issued,
// so the LDS latency hides behind eight MFMAs instead of stalling them.
__device__ __forceinline__ void mma_chunk(const uint16_t* stage, const ReadMap& m, int lhi, int f,
                                          f32x16 (&acc)[2][4]) {
  Frags fr[2];
  read_frags(stage, m, 0, lhi, f, fr[0]);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (s + 1 < 4) read_frags(stage, m, s + 1, lhi, f, fr[(s + 1) & 1]);
    // Keep the reads above the MFMAs (the scheduler would otherwise sink them
    // and reuse one register set).
    __builtin_amdgcn_sched_barrier(0);
    const Frags& c = fr[s & 1];
#pragma unroll
    for (int ms = 0; ms < 2; ++ms)
#pragma unroll
      for (int ns = 0; ns < 4; ++ns) acc[ms][ns] = mfma_32x32x16(c.a[ms], c.b[ns], acc[ms][ns]);
  }
}

// Chunk c (already in `cur`): refill the stage of chunk c-1 with chunk c+2,
// multiply, then wait until chunk c+1 has landed for every thread.  Past the
// last chunk the refill repeats the last chunk (an L2 hit into a stage nobody
// reads), so every step issues and waits the same way: no branch lets the
// compiler think a stage about to be read still has loads in flight, and it
// adds no draining wait of its own.
__device__ __forceinline__ void pipe_step(const Pipe& p, const uint16_t* cur, uint16_t* ahead, int c, int nch,
                                          const ReadMap& m, int lhi, int f, f32x16 (&acc)[2][4]) {
  issue_chunk(p, ahead, min(c + 2, nch - 1));
  mma_chunk(cur, m, lhi, f, acc);
  __builtin_amdgcn_s_waitcnt(kWaitNextChunk);
  __builtin_amdgcn_s_barrier();
}

}  // namespace

// PHASE kGateUp: A = x rows (gathered), B rows = gate/up rows, K = d,
//                out = SiLU(G) * U -> hid / hid_shared (bf16, row stride H).
// PHASE kDown:   A = hid rows, B rows = W_d rows, K = H,
//                out -> y_perm (bf16) / y_shared (f32), row stride d.
template <int PHASE>
__global__ __launch_bounds__(kThreads) void k_expert_tiled(const uint16_t* __restrict__ a_src,
                                                           const uint16_t* __restrict__ a_src_shared, Groups gs, int d,
                                                           int h, int hs, const uint16_t* __restrict__ w,
                                                           const uint16_t* __restrict__ ws,
                                                           uint16_t* __restrict__ out, void* __restrict__ out_shared,
                                                           int* __restrict__ queue) {
  __shared__ int ip[kMaxGroups + 1];
  __shared__ int next_item;
  __shared__ int wsum[kThreads / kWave];
  __shared__ __attribute__((aligned(16))) uint16_t stage0[kStage];
  __shared__ __attribute__((aligned(16))) uint16_t stage1[kStage];
  __shared__ __attribute__((aligned(16))) uint16_t stage2[kStage];
  const int nt_routed = PHASE == kGateUp ? h / (kTileN / 2) : d / kTileN;
  const int nt_shared = PHASE == kGateUp ? hs / (kTileN / 2) : d / kTileN;
  const int items = item_prefix<kTileM, kThreads>(ip, wsum, gs, nt_routed, nt_shared);
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform per wave
  const int wm = wave % 2, wn = wave / 2;
  const int l32 = lane & 31, lhi = lane >> 5;
  const int f = swz(l32);
  ReadMap m;
#pragma unroll
  for (int ms = 0; ms < 2; ++ms) m.a_row[ms] = wm * 64 + ms * 32 + l32;
#pragma unroll
  for (int ns = 0; ns < 4; ++ns) {
    if (PHASE == kGateUp) m.b_row[ns] = (ns < 2 ? 0 : kTileN / 2) + wn * 64 + (ns % 2) * 32 + l32;
    else m.b_row[ns] = wn * 128 + ns * 32 + l32;
  }

  // Dynamic work queue per XCD: XCD x owns items [lo, hi) and its blocks take
  // them in order, one atomic per item, so the items in flight on an XCD are
  // always a contiguous window of the work order (the L2 sharing above relies
  // on it).  Every block exits once its XCD's range is exhausted.
  const int xcd = blockIdx.x % kNumXcd;
  const int lo = (int)((long long)items * xcd / kNumXcd);
  const int hi = (int)((long long)items * (xcd + 1) / kNumXcd);
  for (;;) {
    if (tid == 0) next_item = lo + atomicAdd(&queue[xcd], 1);
    __syncthreads();
    const int wi = next_item;
    if (wi >= hi) break;  // uniform across the block
    const Item it = decode_item<kBand>(ip, gs, kTileM, nt_routed, nt_shared, wi);
    const int H = it.shared ? hs : h;
    const int K = PHASE == kGateUp ? d : H;
    const int nch = K / kChunk;
    const uint16_t* wmat;
    int b_lo, b_hi;  // weight-matrix row of tile row r: b_lo + r (r < 128), b_hi + r (r >= 128)
    if (PHASE == kGateUp) {
      wmat = it.shared ? ws : w + (size_t)it.group * 2 * h * d;
      b_lo = it.nt * (kTileN / 2);
      b_hi = H + it.nt * (kTileN / 2) - kTileN / 2;
    } else {
      wmat = it.shared ? ws : w + (size_t)it.group * d * h;
      b_lo = it.nt * kTileN;
      b_hi = it.nt * kTileN;
    }
    // Direct-load plan.  Load q of wave `wave` fills one 1 KiB region (8 rows
    // x 8 slots) of the A (q < kLoadsA) or B part of a stage: region
    // q' * 4 + wave, lane l -> row 8*region + l/8, slot l%8 = segment ^
    // swz(row).
    Pipe p;
    const uint16_t* abase = it.shared ? a_src_shared : a_src;
    const int astride = PHASE == kGateUp ? d : H;
    size_t arow[kLoadsA];
#pragma unroll
    for (int q = 0; q < kLoadsA; ++q) {
      const int r = it.m0 + (q * 4 + wave) * kRegionRows + lane / kSegs;
      arow[q] = (size_t)(it.row0 + (r < it.nrows ? r : 0));
    }
    if (PHASE == kGateUp) {
      if (it.shared) {
#pragma unroll
        for (int q = 0; q < kLoadsA; ++q) arow[q] -= (size_t)it.row0;
      } else {
        int tok[kLoadsA];
#pragma unroll
        for (int q = 0; q < kLoadsA; ++q) tok[q] = gs.perm[arow[q]];
#pragma unroll
        for (int q = 0; q < kLoadsA; ++q) arow[q] = (size_t)(tok[q] / gs.k);
      }
    }
#pragma unroll
    for (int q = 0; q < kLoadsPerChunk; ++q) {
      const bool is_a = q < kLoadsA;
      const int region = (is_a ? q : q - kLoadsA) * 4 + wave;
      const int row = region * kRegionRows + lane / kSegs;
      const int seg = (lane % kSegs) ^ swz(row);
      p.lds_off[q] = (is_a ? 0 : kStageA) + region * kRegionRows * kChunk;
      if (is_a) {
        p.src[q] = abase + arow[q] * astride + seg * 8;
      } else {
        const int grow = row < kTileN / 2 ? b_lo + row : b_hi + row;
        p.src[q] = wmat + (size_t)grow * K + seg * 8;
      }
    }
    // Every wave multiplies, also on rows past the group's end: items then
    // cost the same, so the blocks sharing operands through L2 stay in step.
    const int wave_row0 = it.m0 + wm * 64;

    f32x16 acc[2][4];
#pragma unroll
    for (int ms = 0; ms < 2; ++ms)
#pragma unroll
      for (int ns = 0; ns < 4; ++ns)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[ms][ns][i] = 0.f;

    // Every wave is past the previous item's reads and stores.
    __builtin_amdgcn_s_waitcnt(kWaitAll);
    __builtin_amdgcn_s_barrier();
    issue_chunk(p, stage0, 0);
    issue_chunk(p, stage1, min(1, nch - 1));
    __builtin_amdgcn_s_waitcnt(kWaitNextChunk);
    __builtin_amdgcn_s_barrier();
    int c = 0;
    for (; c + 3 <= nch; c += 3) {
      pipe_step(p, stage0, stage2, c, nch, m, lhi, f, acc);
      pipe_step(p, stage1, stage0, c + 1, nch, m, lhi, f, acc);
      pipe_step(p, stage2, stage1, c + 2, nch, m, lhi, f, acc);
    }
    if (c < nch) {
      pipe_step(p, stage0, stage2, c, nch, m, lhi, f, acc);
      if (c + 1 < nch) pipe_step(p, stage1, stage0, c + 1, nch, m, lhi, f, acc);
    }

    // Epilogue.  Element i of acc[ms][ns] is row 8*(i/4) + 4*lhi + (i%4) of
    // M-subtile ms, column l32 of N-subtile ns.
#pragma unroll
    for (int ms = 0; ms < 2; ++ms) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = wave_row0 + ms * 32 + 8 * (i / 4) + 4 * lhi + (i % 4);
        if (r >= it.nrows) continue;
        const size_t grow = (size_t)(it.row0 + r);
        if (PHASE == kGateUp) {
          uint16_t* o = it.shared ? static_cast<uint16_t*>(out_shared) : out;
#pragma unroll
          for (int ns = 0; ns < 2; ++ns) {
            const float g = acc[ms][ns][i], u = acc[ms][ns + 2][i];
            o[grow * H + it.nt * (kTileN / 2) + wn * 64 + ns * 32 + l32] = (uint16_t)f32_to_bf16(silu(g) * u);
          }
        } else {
#pragma unroll
          for (int ns = 0; ns < 4; ++ns) {
            const size_t o = grow * d + it.nt * kTileN + wn * 128 + ns * 32 + l32;
            if (it.shared) static_cast<float*>(out_shared)[o] = acc[ms][ns][i];
            else out[o] = (uint16_t)f32_to_bf16(acc[ms][ns][i]);
          }
        }
      }
    }
  }
}

namespace {

__global__ void k_clear_queue(int* queue) {
  if (threadIdx.x < kNumXcd) queue[threadIdx.x] = 0;
}

}  // namespace

hipError_t launch_gate_up_tiled(int T, int d, int E, int k, int h, int hs, const uint16_t* x, const int32_t* offsets,
                                const int32_t* perm, const uint16_t* w_gu, const uint16_t* ws_gu, uint16_t* hid,
                                uint16_t* hid_shared, int32_t* queue, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const Groups gs = make_groups(T, E, k, offsets, perm, ws_gu != nullptr);
  hipLaunchKernelGGL(k_clear_queue, dim3(1), dim3(64), 0, stream, queue);
  const auto kern = k_expert_tiled<kGateUp>;
  hipLaunchKernelGGL(kern, dim3(persistent_grid(kern, kThreads)), dim3(kThreads), 0, stream, x, x, gs, d, h, hs,
                     w_gu, ws_gu, hid, static_cast<void*>(hid_shared), queue);
  return hipGetLastError();
}

hipError_t launch_down_tiled(int T, int d, int E, int k, int h, int hs, const int32_t* offsets, const uint16_t* hid,
                             const uint16_t* hid_shared, const uint16_t* w_down, const uint16_t* ws_down,
                             uint16_t* y_perm, float* y_shared, int32_t* queue, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const Groups gs = make_groups(T, E, k, offsets, nullptr, ws_down != nullptr);
  hipLaunchKernelGGL(k_clear_queue, dim3(1), dim3(64), 0, stream, queue);
  const auto kern = k_expert_tiled<kDown>;
  hipLaunchKernelGGL(kern, dim3(persistent_grid(kern, kThreads)), dim3(kThreads), 0, stream, hid, hid_shared, gs, d,
                     h, hs, w_down, ws_down, y_perm, static_cast<void*>(y_shared), queue);
  return hipGetLastError();
}

}  // namespace moe
