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
// few MiB of the XCD's 4 MiB L2.  Blocks take items from a per-XCD queue.
//
// Operand staging.  Both operands go from HBM/L2 straight into LDS with the
// gfx950 direct-to-LDS load (global_load_lds_dwordx4: lane l of a wave writes
// its 16 bytes at LDS base + 16*l) through a ring of three stages of K chunks
// (Cfg: 64 wide for gate/up, one block per CU; 32 wide for down, two blocks
// per CU), with no register staging.  A row of a chunk is kSegs 16-byte
// segments; segment s of row r is stored at slot s ^ swz(r), so a wave's
// 16-byte reads of one segment of 16 consecutive rows cover all LDS banks.
// The direct loads choose their source segment to produce that layout.
//
// Software pipeline (pipe_chunk): each 16-wide K step issues its eight
// MFMAs one by one, and after each one the next step's fragment read from
// LDS and a share of the direct loads of the chunk two ahead, in a pinned
// order, so LDS and memory latency hide behind the matrix pipe.  One block
// barrier per chunk, before its last step, after each thread has waited for
// its own loads of the next chunk (vmcnt) and its reads of this one
// (lgkmcnt): a bare s_barrier, no release fence, which would drain the loads
// in flight.  The three stages are distinct LDS arrays and the chunk loop is
// unrolled by three so the compiler sees which stage each access uses.  Token
// rows past the group's end load the group's first row (their results are
// never stored); every wave multiplies, so items cost the same.
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
// Chunk geometry per phase.  Gate/up (K = d, long items) uses 64-wide chunks:
// every direct load moves whole 128-byte lines, three 48 KiB stages, one block
// of four waves per CU.  Down (K = hidden, items a third as long) uses 32-wide
// chunks: three 24 KiB stages, so two blocks share a CU and each one's
// barrier waits and item start-up are covered by the other's multiplies.
template <int PHASE>
struct Cfg {
  static constexpr int kChunk = PHASE == 0 ? 64 : 32;          // K elements per stage
  static constexpr int kBlocksPerCU = 64 / kChunk;
  static constexpr int kSegs = kChunk / 8;                     // 16-byte segments per row
  static constexpr int kStageA = kTileM * kChunk;              // bf16 elements
  static constexpr int kStageB = kTileN * kChunk;
  static constexpr int kStage = kStageA + kStageB;
  static constexpr int kSteps = kChunk / 16;                   // MFMA K steps per chunk
  static constexpr int kRegionRows = 64 / kSegs;               // rows written by one wave-wide direct load
  static constexpr int kLoadsA = kTileM / kRegionRows / 4;     // per thread per chunk
  static constexpr int kLoadsB = kTileN / kRegionRows / 4;
  static constexpr int kLoadsPerChunk = kLoadsA + kLoadsB;
  // K steps over which a chunk's direct loads are spread: gate/up (one wave
  // per SIMD) spreads them over the whole chunk to keep the issue slots of
  // each step light; down (two waves per SIMD, latency-bound) sends them all
  // in the first step.
  static constexpr int kLoadSteps = PHASE == 0 ? kSteps : 1;
  static constexpr int kLoadsPerStep = kLoadsPerChunk / kLoadSteps;
  // Loads of chunk c+2 issued before the wait that precedes the last step.
  static constexpr int kLoadsBeforeWait = kLoadSteps < kSteps ? kLoadsPerChunk : (kSteps - 1) * kLoadsPerStep;  // s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
  // 6:4, lgkmcnt 11:8).  kWaitChunk0: vmcnt(kLoadsPerChunk) -- an item's
  // first chunk landed while its second is in flight; kWaitNextChunk: only
  // the loads of chunk c+2 issued so far may remain, and lgkmcnt(0)
  // (pipe_chunk).
  static constexpr int kWaitChunk0 = 0x0F70 | kLoadsPerChunk;
  static constexpr int kWaitNextChunk = 0x0070 | kLoadsBeforeWait;
  // Rows sharing one 256-byte window of the 64 LDS banks.
  static constexpr int kRowsPerWindow = 256 / (2 * kChunk);
  static_assert(kSteps % 2 == 0 && kLoadsPerChunk < 16 && kLoadsPerStep * kLoadSteps == kLoadsPerChunk,
                "pipeline shape, vmcnt field");
  // Slot of 16-byte segment `seg` of LDS row `row`: the rows of a window get
  // distinct XOR masks, so a wave's reads of one segment of 16 consecutive
  // rows cover all banks.
  __device__ static __forceinline__ int swz(int row) { return (row / kRowsPerWindow) & (kSegs - 1); }
};
constexpr int kWaitAll = 0x0F70;  // vmcnt(0)

// Cache policy of the direct loads: the default for both operands.  Token rows
// are re-read by every N-tile of their M-tile and weight rows by every M-tile
// of their band, both through L2 (a non-temporal hint on the weight rows
// measured slower: it defeats the sharing within a band).
constexpr int kPolicy = 0;

__device__ __forceinline__ f32x16 mfma_32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

enum Phase { kGateUp = 0, kDown = 1 };

template <int PHASE>
struct Pipe {
  const uint16_t* src[Cfg<PHASE>::kLoadsPerChunk];  // per-thread source of each direct load (chunk 0)
  int lds_off[Cfg<PHASE>::kLoadsPerChunk];          // wave-uniform LDS element offset inside a stage
};

template <int PHASE>
__device__ __forceinline__ void issue_chunk(const Pipe<PHASE>& p, uint16_t* stage, int c) {
  using C = Cfg<PHASE>;
#pragma unroll
  for (int q = 0; q < C::kLoadsPerChunk; ++q)
    __builtin_amdgcn_global_load_lds(p.src[q] + c * C::kChunk, stage + p.lds_off[q], 16, 0, kPolicy);
}

// LDS element offsets of this lane's fragment reads inside a stage, per K
// step s: A row 64 wm + l32 (M-subtile 0; subtile 1 is 32 rows further) and
// B row b_first + l32 (N-subtile 0; the others at kBDelta rows further), each
// at the step's swizzled slot.  All rows a lane reads have swz(row) = swz(l32).
template <int PHASE>
struct ReadMap {
  int a[Cfg<PHASE>::kSteps], b[Cfg<PHASE>::kSteps];
};

// Row offsets of the N-subtiles within the 256-row B tile.  Gate/up: wave wn
// owns units [64 wn, 64 wn + 64) of the gate half (tile rows 0..127) and the
// same units of the up half (rows 128..255).  Down: columns [128 wn, +128).
template <int PHASE>
__device__ __forceinline__ constexpr int b_delta(int ns) {
  return PHASE == 0 ? (ns < 2 ? 0 : kTileN / 2) + (ns % 2) * 32 : ns * 32;
}

// Fragments of one 16-wide K step: v[0..1] = A of M-subtiles 0..1,
// v[2..5] = B of N-subtiles 0..3.
struct Frags {
  u32x4 v[6];
};

template <int PHASE>
__device__ __forceinline__ u32x4 read_frag(const uint16_t* stage, const ReadMap<PHASE>& m, int s, int q) {
  constexpr int kc = Cfg<PHASE>::kChunk;
  const int off = q < 2 ? m.a[s] + q * 32 * kc : m.b[s] + b_delta<PHASE>(q - 2) * kc;
  return *reinterpret_cast<const u32x4*>(&stage[off]);
}

// One K step: the eight MFMAs of `cur`, each followed by one of the six LDS
// reads of the next step's fragments (step `s` of `stage`, into `nxt`) and by
// its share of direct loads q0 .. q0+nq-1 of chunk `cload` into `ahead`.
// The order is pinned (sched_barrier): while an MFMA occupies the matrix pipe
// the wave issues the next read and loads.
template <int PHASE>
__device__ __forceinline__ void mma_step(const Frags& cur, Frags& nxt, const uint16_t* stage,
                                         const ReadMap<PHASE>& m, int s, const Pipe<PHASE>& p, uint16_t* ahead,
                                         int cload, int q0, int nq, f32x16 (&acc)[2][4]) {
  using C = Cfg<PHASE>;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    acc[i / 4][i % 4] = mfma_32x32x16(cur.v[i / 4], cur.v[2 + i % 4], acc[i / 4][i % 4]);
    __builtin_amdgcn_sched_barrier(0);
    if (i < 6) {
      nxt.v[i] = read_frag<PHASE>(stage, m, s, i);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int q = q0 + i * nq / 8; q < q0 + (i + 1) * nq / 8; ++q) {
      __builtin_amdgcn_global_load_lds(p.src[q] + cload * C::kChunk, ahead + p.lds_off[q], 16, 0, kPolicy);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Chunk c of an item, whose step-0 fragments are already in fr[0] (read from
// `cur`).  The first kLoadSteps steps issue chunk c+2's direct loads into
// `ahead` (the stage of chunk c-1, which every wave finished reading before
// the previous barrier).  Steps 0 .. S-2 multiply and read steps 1 .. S-1 of
// `cur`.  Before the last step: wait until this thread's loads of chunk c+1
// have landed (only chunk c+2's may remain) and its reads of chunk c are
// done, then the block barrier -- chunk c+1 is now visible to all and nobody
// reads chunk c any more.  The last step multiplies and reads step 0 of chunk
// c+1 from `next` into fr[0].  Past the last chunk the loads repeat the last
// chunk (an L2 hit into a stage nobody reads) and the final step-0 reads
// fetch unused data, so every chunk issues and waits the same way.
template <int PHASE>
__device__ __forceinline__ void pipe_chunk(const Pipe<PHASE>& p, const uint16_t* cur, const uint16_t* next,
                                           uint16_t* ahead, int c, int nch, const ReadMap<PHASE>& m,
                                           Frags (&fr)[2], f32x16 (&acc)[2][4]) {
  using C = Cfg<PHASE>;
  const int cl = min(c + 2, nch - 1);
#pragma unroll
  for (int st = 0; st + 1 < C::kSteps; ++st)
    mma_step<PHASE>(fr[st & 1], fr[(st + 1) & 1], cur, m, st + 1, p, ahead, cl, st * C::kLoadsPerStep,
                    st < C::kLoadSteps ? C::kLoadsPerStep : 0, acc);
  __builtin_amdgcn_s_waitcnt(C::kWaitNextChunk);
  __builtin_amdgcn_s_barrier();
  constexpr int last = C::kSteps - 1;
  mma_step<PHASE>(fr[1], fr[0], next, m, 0, p, ahead, cl, last * C::kLoadsPerStep,
                  last < C::kLoadSteps ? C::kLoadsPerStep : 0, acc);
}

}  // namespace

// PHASE kGateUp: A = x rows (gathered), B rows = gate/up rows, K = d,
//                out = SiLU(G) * U -> hid / hid_shared (bf16, row stride H).
// PHASE kDown:   A = hid rows, B rows = W_d rows, K = H,
//                out -> y_perm (bf16) / y_shared (f32), row stride d.
template <int PHASE>
__global__ __launch_bounds__(kThreads, Cfg<PHASE>::kBlocksPerCU) void k_expert_tiled(const uint16_t* __restrict__ a_src,
                                                           const uint16_t* __restrict__ a_src_shared, Groups gs, int d,
                                                           int h, int hs, const uint16_t* __restrict__ w,
                                                           const uint16_t* __restrict__ ws,
                                                           uint16_t* __restrict__ out, void* __restrict__ out_shared,
                                                           int* __restrict__ queue) {
  using C = Cfg<PHASE>;
  __shared__ int ip[kMaxGroups + 1];
  __shared__ int next_item;
  __shared__ int wsum[kThreads / kWave];
  __shared__ __attribute__((aligned(16))) uint16_t stage0[C::kStage];
  __shared__ __attribute__((aligned(16))) uint16_t stage1[C::kStage];
  __shared__ __attribute__((aligned(16))) uint16_t stage2[C::kStage];
  const int nt_routed = PHASE == kGateUp ? h / (kTileN / 2) : d / kTileN;
  const int nt_shared = PHASE == kGateUp ? hs / (kTileN / 2) : d / kTileN;
  const int items = item_prefix<kTileM, kThreads>(ip, wsum, gs, nt_routed, nt_shared);
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform per wave
  const int wm = wave % 2, wn = wave / 2;
  const int l32 = lane & 31, lhi = lane >> 5;
  const int f = C::swz(l32);
  ReadMap<PHASE> m;
#pragma unroll
  for (int st = 0; st < C::kSteps; ++st) {
    const int slot = ((2 * st + lhi) ^ f) * 8;
    m.a[st] = (wm * 64 + l32) * C::kChunk + slot;
    m.b[st] = C::kStageA + ((PHASE == kGateUp ? wn * 64 : wn * 128) + l32) * C::kChunk + slot;
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
    const int nch = K / C::kChunk;
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
    // Direct-load plan.  Load q of wave `wave` fills one 1 KiB region
    // (kRegionRows rows x kSegs slots) of the A (q < kLoadsA) or B part of a
    // stage: region q' * 4 + wave, lane l -> row kRegionRows * region +
    // l / kSegs, slot l % kSegs = segment ^ swz(row).
    Pipe<PHASE> p;
    const uint16_t* abase = it.shared ? a_src_shared : a_src;
    const int astride = PHASE == kGateUp ? d : H;
    size_t arow[C::kLoadsA];
#pragma unroll
    for (int q = 0; q < C::kLoadsA; ++q) {
      const int r = it.m0 + (q * 4 + wave) * C::kRegionRows + lane / C::kSegs;
      arow[q] = (size_t)(it.row0 + (r < it.nrows ? r : 0));
    }
    if (PHASE == kGateUp) {
      if (it.shared) {
#pragma unroll
        for (int q = 0; q < C::kLoadsA; ++q) arow[q] -= (size_t)it.row0;
      } else {
        int tok[C::kLoadsA];
#pragma unroll
        for (int q = 0; q < C::kLoadsA; ++q) tok[q] = gs.perm[arow[q]];
#pragma unroll
        for (int q = 0; q < C::kLoadsA; ++q) arow[q] = (size_t)(tok[q] / gs.k);
      }
    }
#pragma unroll
    for (int q = 0; q < C::kLoadsPerChunk; ++q) {
      const bool is_a = q < C::kLoadsA;
      const int region = (is_a ? q : q - C::kLoadsA) * 4 + wave;
      const int row = region * C::kRegionRows + lane / C::kSegs;
      const int seg = (lane % C::kSegs) ^ C::swz(row);
      p.lds_off[q] = (is_a ? 0 : C::kStageA) + region * C::kRegionRows * C::kChunk;
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
    issue_chunk<PHASE>(p, stage0, 0);
    issue_chunk<PHASE>(p, stage1, min(1, nch - 1));
    __builtin_amdgcn_s_waitcnt(C::kWaitChunk0);
    __builtin_amdgcn_s_barrier();
    Frags fr[2];
#pragma unroll
    for (int q = 0; q < 6; ++q) fr[0].v[q] = read_frag<PHASE>(stage0, m, 0, q);
    int c = 0;
    for (; c + 3 <= nch; c += 3) {
      pipe_chunk<PHASE>(p, stage0, stage1, stage2, c, nch, m, fr, acc);
      pipe_chunk<PHASE>(p, stage1, stage2, stage0, c + 1, nch, m, fr, acc);
      pipe_chunk<PHASE>(p, stage2, stage0, stage1, c + 2, nch, m, fr, acc);
    }
    if (c < nch) {
      pipe_chunk<PHASE>(p, stage0, stage1, stage2, c, nch, m, fr, acc);
      if (c + 1 < nch) pipe_chunk<PHASE>(p, stage1, stage2, stage0, c + 1, nch, m, fr, acc);
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
