// expert_tiled.hip -- grouped SwiGLU expert GEMMs for the compute regime
// (from 11 rows per expert on average, 10 for down, up to prefill-sized
// batches; the dense FFN above 64 tokens), bf16 MFMA 32x32x16.
//
// Layer definition as in expert.hip ([Digest] "Step 3.5 Flash 技术论文深度解读"
// architecture table and activation-explosion cause 3; grouped layout after
// [Blog] "Step 3.5 Flash: Open Frontier-Level Intelligence with 11B Active
// Parameters" §3.2.4).
//
// Block = 8 waves (two per SIMD); item = up to 256 token rows x 256 weight
// rows of one group:
//   gate/up: 128 gate rows j0.. and the 128 matching up rows h+j0.. of W_gu;
//   down:    256 rows n0.. of W_d.
// Per 64-wide K chunk the block moves 64 KiB from L2 into LDS for 8.4 MFLOP:
// the operand traffic per flop is what bounds these kernels (the L2 -> CU
// path delivers ~16.5 TB/s on this chip), and a 256 x 256 item needs a third
// less of it than a 128 x 256 one.  A group's last M-tile may hold fewer
// rows: it loads and multiplies only its 64-row slices, so its cost follows
// its rows.
//
// Wave w = (wm, wn) = (w / 2, w % 2) owns rows [64 wm, 64 wm + 64) of the
// M-tile and 128 weight rows: gate/up units [64 wn, 64 wn + 64) of both halves
// (so SiLU(G) * U pairs sit in the same lane), or down columns
// [128 wn, 128 wn + 128).  That is 2 x 4 MFMA 32x32x16 tiles, 128 f32
// accumulators per lane, 0.75 KiB of LDS reads per MFMA.  SIMD s runs waves s
// and s + 4, whose M-slices are s / 2 and s / 2 + 2: in an item of at most
// 128 rows waves 4..7 skip their multiplies and every SIMD still has one wave
// multiplying.
//
// Work order (grouped.h): M-tiles fastest in bands of up to 4; blocks take
// items from a per-XCD queue, so the items in flight on an XCD are a window of
// consecutive items sharing their groups' token rows and weights through L2;
// a block whose queue is empty takes from the other XCDs' queues.
//
// Operand staging.  Both operands go from HBM/L2 straight into LDS with the
// gfx950 direct-to-LDS load (global_load_lds_dwordx4: lane l of a wave writes
// its 16 bytes at LDS base + 16*l), whole 128-byte rows per 64-wide chunk
// (half rows cost a third of the L2 throughput), through two stages of
// A 256x64 + B 256x64 bf16 = 64 KiB each, with no register staging (items of
// one 64-row slice: a ring of three 40 KiB slots instead, see
// run_item_small).  Segment s
// of row r is stored at slot s ^ ((r >> 1) & 7), so a wave's 16-byte reads of
// one segment of 16 consecutive rows cover all LDS banks.  The direct loads
// choose their source segment to produce that layout.
//
// Software pipeline (pipe_chunk): chunk c's first K step issues all of chunk
// c+1's direct loads into the other stage, one after each MFMA; steps 0-2
// each follow every MFMA with one LDS read of the next step's fragments.
// After step 3 each thread waits for its loads of chunk c+1, then the block
// barrier (a bare s_barrier: no release fence, which would drain the loads in
// flight) makes chunk c+1 visible; reading its first fragments is the only
// exposed LDS latency per chunk, which the SIMD's other wave covers.  Token
// rows past the group's end load the group's first row (their results are
// never stored).
//
// MFMA 32x32x16 operands: lane l supplies row (l % 32) of A / column (l % 32)
// of B for the 8 reduction elements 8*(l/32) .. +7 of the 16; result element
// i of lane l is D[8*(i/4) + 4*(l/32) + (i%4)][l % 32].  The kernels pass the
// weight fragment as A and the token fragment as B, so D is the transposed
// output tile: four adjacent output columns of one token row per lane.
#include "common.h"
#include "grouped.h"
#include "kernels.h"

namespace moe {

typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * kWave;
constexpr int kTileM = 256;                       // token rows of a full item
constexpr int kTileN = 256;                       // weight rows per item
constexpr int kBand = 4;                          // M-tiles per band of the work order
constexpr int kChunk = 64;                        // K elements per stage
constexpr int kSegs = kChunk / 8;                 // 16-byte segments per row
constexpr int kStageA = kTileM * kChunk;          // bf16 elements
constexpr int kStageB = kTileN * kChunk;
constexpr int kSteps = kChunk / 16;               // MFMA K steps per chunk
constexpr int kRegionRows = 64 / kSegs;           // rows written by one wave-wide direct load
constexpr int kLoadsA = kTileM / kRegionRows / kWaves;  // per thread per chunk
constexpr int kLoadsB = kTileN / kRegionRows / kWaves;
constexpr int kLoads = kLoadsA + kLoadsB;         // 8: one after each MFMA of a step
static_assert(kLoads == 8 && kSteps == 4, "pipeline shape");

// s_waitcnt vmcnt(0) (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4 and lgkmcnt 11:8 not waited on).
constexpr int kWaitAll = 0x0F70;

constexpr int kPolicy = 0;       // default cache policy of the direct loads
constexpr int kNonTemporal = 2;  // the loads' nt bit (gfx950 cache-policy operand)

__device__ __forceinline__ f32x16 mfma_32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ int swz(int row) { return (row >> 1) & (kSegs - 1); }

// Orders one wave's LDS accesses across its lanes (writes before the reads
// that follow, reads before the writes that follow).
__device__ __forceinline__ void wave_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// LDS byte address of a pointer into this block's shared memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// The lane's index, computed where it is called: values derived from it are
// not hoisted out of the item loop to sit in registers across the K loop.
__device__ __forceinline__ int lane_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// The epilogue stages through a buffer that no direct load in flight writes.
// Written as plain C++ its LDS accesses would each wait for every outstanding
// global load and store first, because the compiler cannot tell the direct
// loads' target buffers apart; these two do their own waiting instead.  One
// wave's LDS accesses execute in order, so a write needs no wait before a
// later read, and each read waits for itself.  `off` must fold to a
// constant below 65536.
__device__ __forceinline__ void lds_write_b64_own(uint32_t addr, uint32_t lo, uint32_t hi) {
  asm volatile("ds_write_b64 %0, %1" ::"v"(addr), "v"(__builtin_bit_cast(unsigned long long, (u32x2){lo, hi}))
               : "memory");
}
__device__ __forceinline__ u32x4 lds_read_b128_own(uint32_t base, int off) {
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1 offset:%2\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(base), "i"(off) : "memory");
  return v;
}

enum Phase { kGateUp = 0, kDown = 1 };

// Row of N-subtile ns (0..3) of wave column wn inside the 256-row B tile.
// Gate/up: gate rows [64 wn, +64) (ns 0, 1) and up rows [128 + 64 wn, +64)
// (ns 2, 3); down: columns [128 wn + 32 ns, +32).
template <int PHASE>
__device__ __forceinline__ constexpr int b_row0(int wn, int ns) {
  return PHASE == kGateUp ? (ns / 2) * (kTileN / 2) + wn * 64 + (ns % 2) * 32 : wn * 128 + ns * 32;
}

// Direct loads q < kLoadsA fill A slice q (token rows 64q .. 64q+63), the
// rest the B tile.  An item with fewer than 256 rows loads only its NA
// slices (a template parameter of its K loop, so full items run branch-free
// code): the L2 -> CU operand traffic, which bounds these kernels, then
// shrinks with the item.
struct Pipe {
  const uint16_t* src[kLoads];  // per-thread source of each direct load (chunk 0)
  int lds_off[kLoads];          // wave-uniform LDS element offset inside its A slice or B tile
  bool wnt;                     // weight loads non-temporal (uniform; see make_plan)
};

// Direct load q of a chunk: the weight loads (q >= kLoadsA) of an item whose
// weight tile no other item reads go non-temporal, so they do not push the
// token rows, which the group's other N-tiles read again, out of L2.
__device__ __forceinline__ void dload(const Pipe& p, int q, const uint16_t* src, uint16_t* dst) {
  if (q >= kLoadsA && p.wnt)
    __builtin_amdgcn_global_load_lds(src, dst, 16, 0, kNonTemporal);
  else
    __builtin_amdgcn_global_load_lds(src, dst, 16, 0, kPolicy);
}

template <int NA>
__device__ __forceinline__ constexpr bool load_used(int q) {
  return q >= kLoadsA || q < NA;
}

// One stage of operands in LDS: A slice q (64 token rows x 64) at
// a + q * kSlice, this wave's A slice (the rows it multiplies) at a_read, the
// 256 x 64 B tile at b.  A and B of every stage are separate arrays (see the
// kernel), and a_read is computed from a alone, so the compiler, which waits
// for a direct load before any LDS read that may alias it, tells the stages
// apart.
constexpr int kSlice = kStageA / kLoadsA;  // elements of one 64-row A slice

struct StageRef {
  uint16_t* a;
  const uint16_t* a_read;
  uint16_t* b;
};

__device__ __forceinline__ uint16_t* load_dst(const StageRef& st, const Pipe& p, int q) {
  return (q < kLoadsA ? st.a + q * kSlice : st.b) + p.lds_off[q];
}

template <int NA>
__device__ __forceinline__ void issue_chunk(const Pipe& p, const StageRef& st, int c) {
#pragma unroll
  for (int q = 0; q < kLoads; ++q)
    if (load_used<NA>(q)) dload(p, q, p.src[q] + c * kChunk, load_dst(st, p, q));
}

// LDS element offsets of this lane's fragment reads, per K step s: row l32
// of the wave's A slice (M-subtile 0; subtile 1 is 32 rows further) and B row
// b_row0(wn, 0) + l32 (N-subtile 0; subtile ns at b_row0(wn, ns) -
// b_row0(wn, 0) further), each at the step's swizzled slot.  All rows a lane
// reads have swz(row) = swz(l32).
struct ReadMap {
  int a[kSteps], b[kSteps];
};

// Fragments of one 16-wide K step: v[0..1] = A of M-subtiles 0..1,
// v[2..5] = B of N-subtiles 0..3.
struct Frags {
  u32x4 v[6];
};

template <int PHASE>
__device__ __forceinline__ u32x4 read_frag(const StageRef& st, const ReadMap& m, int s, int q) {
  const uint16_t* ptr = q < 2 ? st.a_read + m.a[s] + q * 32 * kChunk
                              : st.b + m.b[s] + (b_row0<PHASE>(0, q - 2) - b_row0<PHASE>(0, 0)) * kChunk;
  return *reinterpret_cast<const u32x4*>(ptr);
}

// One K step: the eight MFMAs of `cur` (if MUL), after MFMA i the LDS read i
// of the next step's fragments (step `s` of `stage` into `nxt`, i < 6, if
// READ) and, with LOADS and `issue` (uniform), direct load i of chunk `cload`
// into `other`.  The order is pinned (sched_barrier).
template <int PHASE, int NA, bool MUL, bool READ, bool LOADS>
__device__ __forceinline__ void mma_step(const Frags& cur, Frags& nxt, const StageRef& stage, const ReadMap& m,
                                         int s, const Pipe& p, const StageRef& other, int cload, bool issue,
                                         f32x16 (&acc)[2][4]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (MUL) {
      acc[i / 4][i % 4] = mfma_32x32x16(cur.v[2 + i % 4], cur.v[i / 4], acc[i / 4][i % 4]);
      __builtin_amdgcn_sched_barrier(0);
      if (READ && i < 6) {
        nxt.v[i] = read_frag<PHASE>(stage, m, s, i);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (LOADS && issue && load_used<NA>(i)) {
      dload(p, i, p.src[i] + cload * kChunk, load_dst(other, p, i));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Chunk c of an item (in `cur`), whose step-0 fragments are already in fr[0].
// Step 0 issues chunk c+1's direct loads into `other` (the stage of chunk
// c-1: every wave finished reading it before the previous barrier, its reads
// having been consumed by that chunk's MFMAs).  Steps 0-2 read steps 1-3 of
// `cur`; step 3 only multiplies.  Then each thread waits for its loads of
// chunk c+1 and the block barrier makes them visible; its first fragments
// are read last.  In the down phase the last chunk issues no loads; in
// gate/up it repeats its own loads (an L2 hit into a stage nobody reads), so
// every chunk issues and waits the same way (issuing none there measured no
// faster).  Either way the barrier after the K loop drains them, and the
// epilogue may use x1.  The final reads fetch unused data.  Waves without rows in the item (MUL = false) only load and wait.
template <int PHASE, int NA, bool MUL>
__device__ __forceinline__ void pipe_chunk(const Pipe& p, const StageRef& cur, const StageRef& other, int c, int nch,
                                           const ReadMap& m, Frags (&fr)[2], f32x16 (&acc)[2][4]) {
  const int cl = min(c + 1, nch - 1);
  const bool issue = PHASE == kGateUp || c + 1 < nch;
  mma_step<PHASE, NA, MUL, true, true>(fr[0], fr[1], cur, m, 1, p, other, cl, issue, acc);
  mma_step<PHASE, NA, MUL, true, false>(fr[1], fr[0], cur, m, 2, p, other, cl, issue, acc);
  mma_step<PHASE, NA, MUL, true, false>(fr[0], fr[1], cur, m, 3, p, other, cl, issue, acc);
  mma_step<PHASE, NA, MUL, false, false>(fr[1], fr[0], cur, m, 0, p, other, cl, issue, acc);
  __builtin_amdgcn_s_waitcnt(kWaitAll);
  __builtin_amdgcn_s_barrier();
  if (MUL) {
#pragma unroll
    for (int q = 0; q < 6; ++q) fr[0].v[q] = read_frag<PHASE>(other, m, 0, q);
  }
}

// The K loop of one item over the two stages (unrolled by two).  Chunk 0 was
// issued into stage0 before the previous item's epilogue.
template <int PHASE, int NA, bool MUL>
__device__ __forceinline__ void run_item(const Pipe& p, const StageRef& stage0, const StageRef& stage1, int nch,
                                         const ReadMap& m, f32x16 (&acc)[2][4]) {
  __builtin_amdgcn_s_waitcnt(kWaitAll);
  __builtin_amdgcn_s_barrier();
  Frags fr[2];
  if (MUL) {
#pragma unroll
    for (int q = 0; q < 6; ++q) fr[0].v[q] = read_frag<PHASE>(stage0, m, 0, q);
  }
  int c = 0;
  for (; c + 2 <= nch; c += 2) {
    pipe_chunk<PHASE, NA, MUL>(p, stage0, stage1, c, nch, m, fr, acc);
    pipe_chunk<PHASE, NA, MUL>(p, stage1, stage0, c + 1, nch, m, fr, acc);
  }
  if (c < nch) pipe_chunk<PHASE, NA, MUL>(p, stage0, stage1, c, nch, m, fr, acc);
}

// Items of one 64-row slice move 40 KiB per chunk, so three chunks fit in
// the operand memory: the ring of slots S0, S1, S2 holds chunk c in slot
// c % 3, and chunk c's first K step issues chunk c + 2, two ahead for both
// operands.  Such an item's chunk waits on the latency of its transfer more
// than on the transfer (per item on the skewed routing: gate/up 89 -> 73 us,
// down 36 -> 30 us; whole launches 3-4% faster there, 1% at prefill).  At the
// end of chunk c each thread waits for all but its five loads of chunk c + 2.
// Chunks 0 and 1 were issued into S0 and S1 before the previous item's
// epilogue.
constexpr int kLoadsSmall = 1 + kLoadsB;  // direct loads per thread per chunk of a one-slice item

template <int PHASE, bool MUL>
__device__ __forceinline__ void pipe_chunk_small(const Pipe& p, const StageRef& cur, const StageRef& ahead,
                                                 const StageRef& next, int c, int nch, const ReadMap& m,
                                                 Frags (&fr)[2], f32x16 (&acc)[2][4]) {
  const bool issue = c + 2 < nch;
  mma_step<PHASE, 1, MUL, true, true>(fr[0], fr[1], cur, m, 1, p, ahead, c + 2, issue, acc);
  mma_step<PHASE, 1, MUL, true, false>(fr[1], fr[0], cur, m, 2, p, ahead, c + 2, issue, acc);
  mma_step<PHASE, 1, MUL, true, false>(fr[0], fr[1], cur, m, 3, p, ahead, c + 2, issue, acc);
  mma_step<PHASE, 1, MUL, false, false>(fr[1], fr[0], cur, m, 0, p, ahead, c + 2, issue, acc);
  if (issue)
    __builtin_amdgcn_s_waitcnt(kWaitAll | kLoadsSmall);
  else
    __builtin_amdgcn_s_waitcnt(kWaitAll);
  __builtin_amdgcn_s_barrier();
  if (MUL) {
#pragma unroll
    for (int q = 0; q < 6; ++q) fr[0].v[q] = read_frag<PHASE>(next, m, 0, q);
  }
}

template <int PHASE, bool MUL>
__device__ __forceinline__ void run_item_small(const Pipe& p, const StageRef& S0, const StageRef& S1,
                                               const StageRef& S2, int nch, const ReadMap& m,
                                               f32x16 (&acc)[2][4]) {
  __builtin_amdgcn_s_waitcnt(kWaitAll);
  __builtin_amdgcn_s_barrier();
  Frags fr[2];
  if (MUL) {
#pragma unroll
    for (int q = 0; q < 6; ++q) fr[0].v[q] = read_frag<PHASE>(S0, m, 0, q);
  }
  int c = 0;
  for (; c + 3 <= nch; c += 3) {
    pipe_chunk_small<PHASE, MUL>(p, S0, S2, S1, c, nch, m, fr, acc);
    pipe_chunk_small<PHASE, MUL>(p, S1, S0, S2, c + 1, nch, m, fr, acc);
    pipe_chunk_small<PHASE, MUL>(p, S2, S1, S0, c + 2, nch, m, fr, acc);
  }
  if (c < nch) pipe_chunk_small<PHASE, MUL>(p, S0, S2, S1, c, nch, m, fr, acc);
  if (c + 1 < nch) pipe_chunk_small<PHASE, MUL>(p, S1, S0, S2, c + 1, nch, m, fr, acc);
}

}  // namespace

// Everything an item's K loop and epilogue need, built from its index.
struct Plan {
  Item it;
  int H, nch, na;  // hidden size of its group, K chunks, A slices (1..4)
  int ksi;         // reduction split of the item (0 unless SPLIT)
  Pipe p;
};

// SPLIT (the shared group alone, one M-tile): item N-tile index n stands for
// weight tile n % ntiles over reduction split n / ntiles of ks, each split
// nch / ks consecutive chunks.
template <int PHASE, bool SPLIT>
__device__ __forceinline__ Plan make_plan(const int* ip, const Groups& gs, int nt_routed, int nt_shared, int wi,
                                          int d, int h, int hs, const uint16_t* a_src,
                                          const uint16_t* a_src_shared, const uint16_t* w, const uint16_t* ws,
                                          int wave, int lane, int ks) {
  Plan pl;
  Item it = decode_item<kBand>(ip, gs, kTileM, nt_routed, nt_shared, wi);
  pl.H = it.shared ? hs : h;
  const int K = PHASE == kGateUp ? d : pl.H;
  pl.nch = K / kChunk;
  pl.ksi = 0;
  int k0 = 0;  // first reduction element of the item
  if (SPLIT) {
    const int ntiles = nt_shared / ks;
    pl.ksi = it.nt / ntiles;
    it.nt -= pl.ksi * ntiles;
    pl.nch /= ks;
    k0 = pl.ksi * pl.nch * kChunk;
  }
  pl.it = it;
  pl.na = min(kLoadsA, (it.nrows - it.m0 + 63) / 64);
  // A group of one M-tile reads each weight tile in one item only (skewed
  // load: gate/up 1.258 -> 1.239 ms, down 0.728 -> 0.715; prefill within
  // 1%).  Groups of more M-tiles share their weight tiles through L2.
  pl.p.wnt = __builtin_amdgcn_readfirstlane(it.nrows <= kTileM ? 1 : 0) != 0;
  const uint16_t* wmat;
  int b_lo, b_hi;  // weight-matrix row of tile row r: b_lo + r (r < 128), b_hi + r (r >= 128)
  if (PHASE == kGateUp) {
    wmat = it.shared ? ws : w + (size_t)it.group * 2 * h * d;
    b_lo = it.nt * (kTileN / 2);
    b_hi = pl.H + it.nt * (kTileN / 2) - kTileN / 2;
  } else {
    wmat = it.shared ? ws : w + (size_t)it.group * d * h;
    b_lo = it.nt * kTileN;
    b_hi = it.nt * kTileN;
  }
  // Direct-load plan.  Load q of wave `wave` fills one 1 KiB region (8 rows
  // x 8 slots) of the A (q < kLoadsA) or B part of a stage: region
  // q' * kWaves + wave, lane l -> row 8 * region + l / 8, slot l % 8 =
  // segment ^ swz(row); A region q * kWaves + wave is region `wave` of A
  // slice q.
  const uint16_t* abase = it.shared ? a_src_shared : a_src;
  const int astride = PHASE == kGateUp ? d : pl.H;
  size_t arow[kLoadsA];
#pragma unroll
  for (int q = 0; q < kLoadsA; ++q) {
    const int r = it.m0 + (q * kWaves + wave) * kRegionRows + lane / kSegs;
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
  for (int q = 0; q < kLoads; ++q) {
    const bool is_a = q < kLoadsA;
    const int region = (is_a ? q : q - kLoadsA) * kWaves + wave;
    const int row = region * kRegionRows + lane / kSegs;
    const int seg = (lane % kSegs) ^ swz(row);
    pl.p.lds_off[q] = (is_a ? wave : region) * kRegionRows * kChunk;
    if (is_a) {
      pl.p.src[q] = abase + arow[q] * astride + k0 + seg * 8;
    } else {
      const int grow = row < kTileN / 2 ? b_lo + row : b_hi + row;
      pl.p.src[q] = wmat + (size_t)grow * K + k0 + seg * 8;
    }
  }
  return pl;
}

// An item's first chunk into stage0 (one-slice items: its first two chunks
// into ring slots S0 and S1).
__device__ __forceinline__ void issue_first(const Plan& pl, const StageRef& stage0, const StageRef& S0,
                                            const StageRef& S1) {
  switch (pl.na) {
    case 4: issue_chunk<4>(pl.p, stage0, 0); break;
    case 3: issue_chunk<3>(pl.p, stage0, 0); break;
    case 2: issue_chunk<2>(pl.p, stage0, 0); break;
    default:
      issue_chunk<1>(pl.p, S0, 0);
      if (pl.nch > 1) issue_chunk<1>(pl.p, S1, 1);
      break;
  }
}

// PHASE kGateUp: A = x rows (gathered), B rows = gate/up rows, K = d,
//                out = SiLU(G) * U -> hid / hid_shared (bf16, row stride H),
//                clipped to [-clamp, clamp] when CLAMP.
// PHASE kDown:   A = hid rows, B rows = W_d rows, K = H,
//                out -> y_perm (bf16) / y_shared (f32), row stride d.
// SPLIT: the shared group alone in one M-tile, its reduction split over ks
// items per weight tile; each writes its f32 sums to partial[split][row][col]
// (col < 2 hs for gate/up: gate unit j at j, up unit j at hs + j; col < d
// for down), added up by k_swiglu_splits / k_sum_splits.
template <int PHASE, bool CLAMP = false, bool SPLIT = false>
__global__ __launch_bounds__(kThreads, 1) void k_expert_tiled(const uint16_t* __restrict__ a_src,
                                                              const uint16_t* __restrict__ a_src_shared, Groups gs,
                                                              int d, int h, int hs, const uint16_t* __restrict__ w,
                                                              const uint16_t* __restrict__ ws,
                                                              uint16_t* __restrict__ out,
                                                              void* __restrict__ out_shared,
                                                              int* __restrict__ queue, float clamp, int ks,
                                                              float* __restrict__ partial) {
  __shared__ int ip[kMaxGroups + 1];
  __shared__ int next_item;
  __shared__ int wsum[kWaves];
  // Operand memory (152 KiB): stage0 = A x0 + B y0, stage1 = A x1 + B y1;
  // the one-slice ring's slots S0 = (s0, y0), S1 = (s1, y1), S2 = (s2, x1),
  // with A slices of their own.
  __shared__ __attribute__((aligned(16))) uint16_t x0[kStageA];
  __shared__ __attribute__((aligned(16))) uint16_t y0[kStageB];
  __shared__ __attribute__((aligned(16))) uint16_t x1[kStageA];
  __shared__ __attribute__((aligned(16))) uint16_t y1[kStageB];
  __shared__ __attribute__((aligned(16))) uint16_t s0[kSlice];
  __shared__ __attribute__((aligned(16))) uint16_t s1[kSlice];
  __shared__ __attribute__((aligned(16))) uint16_t s2[kSlice];
  const int nt_routed = PHASE == kGateUp ? h / (kTileN / 2) : d / kTileN;
  const int nt_shared = (PHASE == kGateUp ? hs / (kTileN / 2) : d / kTileN) * (SPLIT ? ks : 1);
  const int items = item_prefix<kTileM, kThreads>(ip, wsum, gs, nt_routed, nt_shared);
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform per wave
  const int wm = wave / 2, wn = wave % 2;
  const int l32 = lane & 31, lhi = lane >> 5;
  const int f = swz(l32);
  ReadMap m;
#pragma unroll
  for (int st = 0; st < kSteps; ++st) {
    const int slot = ((2 * st + lhi) ^ f) * 8;
    m.a[st] = l32 * kChunk + slot;
    m.b[st] = (b_row0<PHASE>(wn, 0) + l32) * kChunk + slot;
  }
  const StageRef stage0{x0, x0 + wm * kSlice, y0};
  const StageRef stage1{x1, x1 + wm * kSlice, y1};
  const StageRef S0{s0, s0, y0};
  const StageRef S1{s1, s1, y1};
  const StageRef S2{s2, s2, x1};

  // Dynamic work queue per XCD: queue q owns items [items·q/8, items·(q+1)/8)
  // and hands them out in order, one atomic per item.  A block takes from its
  // own XCD's queue (neighbouring items share operands through that XCD's
  // L2); once that is exhausted it takes from the other queues in turn, so no
  // XCD idles while another still has items (prefill gate/up 1.97 -> 1.83 ms).
  // Only thread 0 walks the queues; `tried` only grows, so a block makes at
  // most kNumXcd failed attempts before it exits.  The next item is taken,
  // planned and its first chunk issued right after the current item's K
  // loop, so that chunk's latency overlaps the current item's epilogue.
  const int xcd = blockIdx.x % kNumXcd;
  int tried = 0;
  auto take = [&]() {
    while (tried < kNumXcd) {
      const int q = (xcd + tried) % kNumXcd;
      const int t = (int)((long long)items * q / kNumXcd) + atomicAdd(&queue[q], 1);
      if (t < (int)((long long)items * (q + 1) / kNumXcd)) return t;
      ++tried;
    }
    return -1;
  };
  if (tid == 0) next_item = take();
  __syncthreads();
  int wi = next_item;
  if (wi < 0) return;  // uniform across the block
  Plan cur = make_plan<PHASE, SPLIT>(ip, gs, nt_routed, nt_shared, wi, d, h, hs, a_src, a_src_shared, w, ws, wave, lane, ks);
  issue_first(cur, stage0, S0, S1);
  for (;;) {
    const int wave_row0 = cur.it.m0 + wm * 64;
    // A wave multiplies iff some of its 64 rows exist (wm < na; uniform per
    // wave).
    const bool mul = wave_row0 < cur.it.nrows;
    f32x16 acc[2][4];
#pragma unroll
    for (int ms = 0; ms < 2; ++ms)
#pragma unroll
      for (int ns = 0; ns < 4; ++ns)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[ms][ns][i] = 0.f;
    switch (cur.na * 2 + (mul ? 1 : 0)) {  // uniform per wave
      case 9: run_item<PHASE, 4, true>(cur.p, stage0, stage1, cur.nch, m, acc); break;
      case 8: run_item<PHASE, 4, false>(cur.p, stage0, stage1, cur.nch, m, acc); break;
      case 7: run_item<PHASE, 3, true>(cur.p, stage0, stage1, cur.nch, m, acc); break;
      case 6: run_item<PHASE, 3, false>(cur.p, stage0, stage1, cur.nch, m, acc); break;
      case 5: run_item<PHASE, 2, true>(cur.p, stage0, stage1, cur.nch, m, acc); break;
      case 4: run_item<PHASE, 2, false>(cur.p, stage0, stage1, cur.nch, m, acc); break;
      case 3: run_item_small<PHASE, true>(cur.p, S0, S1, S2, cur.nch, m, acc); break;
      default: run_item_small<PHASE, false>(cur.p, S0, S1, S2, cur.nch, m, acc); break;
    }
    // Every wave is past the K loop (its LDS reads done, its trailing loads
    // landed: the release fence of this barrier drains both), so stage0 may
    // take the next item's first chunk; next_item was last read before the
    // K loop.
    if (tid == 0) next_item = take();
    __syncthreads();
    wi = next_item;
    const bool more = wi >= 0;  // uniform across the block
    Plan nxt;
    if (more) {
      nxt = make_plan<PHASE, SPLIT>(ip, gs, nt_routed, nt_shared, wi, d, h, hs, a_src, a_src_shared, w, ws, wave, lane, ks);
      issue_first(nxt, stage0, S0, S1);
    }

    // Epilogue.  The MFMAs take the weight operand first, so the tile comes
    // out transposed: element i of acc[ms][ns] is column 8*(i/4) + 4*lhi +
    // (i%4) of N-subtile ns, row l32 of M-subtile ms -- four adjacent columns
    // of one row per lane, which pack into 8 bytes of bf16 or 16 of f32.
    // The bf16 outputs go through the wave's 4 KiB of x1 (free: the K loop's
    // last loads landed before the barrier above, and the next item's first
    // chunks went to stage0 or to slots S0 and S1), 32 rows x 64 columns at a
    // time: a lane writes its 4 columns of a row as 8 bytes, 16-byte segment
    // s of row r at slot s ^ (r & 7) of the row's 128 bytes so that the 32
    // rows of one write spread over the banks; read back as whole segments, 8
    // rows of 128 bytes per read, they go out as 16-byte stores through a
    // buffer resource (uniform base at the item's first row, 32-bit offset
    // per lane: an item's 256 rows of at most 65,536 f32 span 64 MiB).
    if (mul) {
      const Item& it = cur.it;
      const int H = cur.H;
      if (SPLIT) {
        // Raw f32 sums of this split, 16 bytes (4 columns of a row) a store.
        const int NW = PHASE == kGateUp ? 2 * H : d;
        float* pp = partial + (size_t)cur.ksi * gs.T * NW;
#pragma unroll
        for (int ms = 0; ms < 2; ++ms) {
          const int r = wave_row0 + ms * 32 + l32;
          if (r < it.nrows) {
            float* prow = pp + (size_t)(it.row0 + r) * NW;
#pragma unroll
            for (int ns = 0; ns < 4; ++ns)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const int col = (PHASE == kGateUp ? (ns < 2 ? 0 : H) + it.nt * (kTileN / 2) + wn * 64 + (ns % 2) * 32
                                                  : it.nt * kTileN + wn * 128 + ns * 32) +
                                8 * q + 4 * lhi;
                const f32x16& a = acc[ms][ns];
                *reinterpret_cast<f32x4*>(prow + col) = f32x4{a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
              }
          }
        }
      } else if (PHASE == kGateUp) {
        // Hidden unit u of the wave's 64 pairs gate acc[ms][u / 32] with up
        // acc[ms][u / 32 + 2] (same element); 64 rows x 64 units in two passes.
        const int ln = lane_here(), lr = ln & 31;
        const uint32_t sb = lds_addr(x1 + wave * 2048);
        const uint32_t wbase = sb + lr * 128 + (ln >> 5) * 8, wxor = (lr & 7) << 4;
        const int rr = ln / 8, sg = ln % 8;
        const uint32_t rbase = sb + rr * 128 + ((sg ^ rr) << 4);
        uint16_t* ob = (it.shared ? static_cast<uint16_t*>(out_shared) : out) + (size_t)(it.row0 + it.m0) * H +
                       it.nt * (kTileN / 2);
        const int ob_bytes = ((min(it.nrows - it.m0, kTileM) - 1) * H + (H - it.nt * (kTileN / 2))) * 2;
        const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(ob, (short)0, ob_bytes, 0x00020000);
        const float cl = CLAMP ? clamp : 0.f;
#pragma unroll
        for (int ms = 0; ms < 2; ++ms) {
#pragma unroll
          for (int ns = 0; ns < 2; ++ns)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const f32x16& g = acc[ms][ns];
              const f32x16& u = acc[ms][ns + 2];
              lds_write_b64_own(wbase + (((ns * 4 + q) << 4) ^ wxor),
                                pack2_bf16(swiglu(g[4 * q], u[4 * q], cl), swiglu(g[4 * q + 1], u[4 * q + 1], cl)),
                                pack2_bf16(swiglu(g[4 * q + 2], u[4 * q + 2], cl), swiglu(g[4 * q + 3], u[4 * q + 3], cl)));
            }
          wave_fence();
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const u32x4 v = lds_read_b128_own(rbase, j * 1024);
            const int r = wave_row0 + ms * 32 + 8 * j + rr;
            if (r < it.nrows)
              __builtin_amdgcn_raw_buffer_store_b128(v, orsrc, ((r - it.m0) * H + wn * 64 + sg * 8) * 2, 0, 0);
          }
          wave_fence();
        }
      } else if (!it.shared) {
        const int ln = lane_here(), lr = ln & 31;
        const uint32_t sb = lds_addr(x1 + wave * 2048);
        const uint32_t wbase = sb + lr * 128 + (ln >> 5) * 8, wxor = (lr & 7) << 4;
        const int rr = ln / 8, sg = ln % 8;
        const uint32_t rbase = sb + rr * 128 + ((sg ^ rr) << 4);
        uint16_t* ob = out + (size_t)(it.row0 + it.m0) * d + it.nt * kTileN;
        const int ob_bytes = ((min(it.nrows - it.m0, kTileM) - 1) * d + (d - it.nt * kTileN)) * 2;
        const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(ob, (short)0, ob_bytes, 0x00020000);
#pragma unroll
        for (int ms = 0; ms < 2; ++ms) {
#pragma unroll
          for (int nh = 0; nh < 2; ++nh) {
#pragma unroll
            for (int n2 = 0; n2 < 2; ++n2)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const f32x16& a = acc[ms][2 * nh + n2];
                lds_write_b64_own(wbase + (((n2 * 4 + q) << 4) ^ wxor), pack2_bf16(a[4 * q], a[4 * q + 1]),
                                  pack2_bf16(a[4 * q + 2], a[4 * q + 3]));
              }
            wave_fence();
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const u32x4 v = lds_read_b128_own(rbase, j * 1024);
              const int r = wave_row0 + ms * 32 + 8 * j + rr;
              if (r < it.nrows)
                __builtin_amdgcn_raw_buffer_store_b128(v, orsrc, ((r - it.m0) * d + wn * 128 + nh * 64 + sg * 8) * 2,
                                                       0, 0);
            }
            wave_fence();
          }
        }
      } else {
        // f32 rows of the shared expert: a lane's 4 columns of a row are 16
        // contiguous bytes, stored through a buffer resource as above.
        float* ob = static_cast<float*>(out_shared) + (size_t)(it.row0 + it.m0) * d + it.nt * kTileN;
        const int ob_bytes = ((min(it.nrows - it.m0, kTileM) - 1) * d + (d - it.nt * kTileN)) * 4;
        const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(ob, (short)0, ob_bytes, 0x00020000);
#pragma unroll
        for (int ms = 0; ms < 2; ++ms) {
          const int r = wave_row0 + ms * 32 + l32;
          if (r < it.nrows) {
#pragma unroll
            for (int ns = 0; ns < 4; ++ns)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const f32x16& a = acc[ms][ns];
                const u32x4 v = {__float_as_uint(a[4 * q]), __float_as_uint(a[4 * q + 1]),
                                 __float_as_uint(a[4 * q + 2]), __float_as_uint(a[4 * q + 3])};
                __builtin_amdgcn_raw_buffer_store_b128(
                    v, orsrc, ((r - it.m0) * d + wn * 128 + ns * 32 + 8 * q + 4 * lhi) * 4, 0, 0);
              }
          }
        }
      }
    }
    if (!more) break;
    cur = nxt;
  }
  // No direct load may still be writing this block's LDS when it exits.
  __builtin_amdgcn_s_waitcnt(kWaitAll);
}

namespace {

__global__ void k_clear_queue(int* queue) {
  if (threadIdx.x < kNumXcd) queue[threadIdx.x] = 0;
}

// Gate/up splits: hid[t][j] = SwiGLU(sum_s P[s][t][j], sum_s P[s][t][H + j]),
// the splits added in s order; four units per thread (H % 4 == 0).
__global__ __launch_bounds__(256) void k_swiglu_splits(const float* __restrict__ P, int ks, int T, int H,
                                                       float clamp, uint16_t* __restrict__ hid) {
  const size_t plane = (size_t)T * 2 * H, n4 = (size_t)T * H / 4;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    const size_t t = i / (H / 4), j = (i % (H / 4)) * 4;
    const float* g0 = P + t * 2 * H + j;
    float4 g = *reinterpret_cast<const float4*>(g0), u = *reinterpret_cast<const float4*>(g0 + H);
    for (int s = 1; s < ks; ++s) {
      const float4 gs = *reinterpret_cast<const float4*>(g0 + s * plane);
      const float4 us = *reinterpret_cast<const float4*>(g0 + s * plane + H);
      g.x += gs.x, g.y += gs.y, g.z += gs.z, g.w += gs.w;
      u.x += us.x, u.y += us.y, u.z += us.z, u.w += us.w;
    }
    const uint32_t lo = pack2_bf16(swiglu(g.x, u.x, clamp), swiglu(g.y, u.y, clamp));
    const uint32_t hi = pack2_bf16(swiglu(g.z, u.z, clamp), swiglu(g.w, u.w, clamp));
    *reinterpret_cast<uint2*>(hid + t * H + j) = make_uint2(lo, hi);
  }
}

// Down splits: y[i] = sum_s P[s][i] in s order (n % 4 == 0).
__global__ __launch_bounds__(256) void k_sum_splits(const float* __restrict__ P, int ks, size_t n,
                                                    float* __restrict__ y) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n / 4; i += (size_t)gridDim.x * 256) {
    float4 v = reinterpret_cast<const float4*>(P)[i];
    for (int s = 1; s < ks; ++s) {
      const float4 w = reinterpret_cast<const float4*>(P + s * n)[i];
      v.x += w.x, v.y += w.y, v.z += w.z, v.w += w.w;
    }
    reinterpret_cast<float4*>(y)[i] = v;
  }
}

unsigned finish_grid(size_t n4) {
  const size_t blocks = (n4 + 255) / 256;
  return (unsigned)(blocks < 4096 ? blocks : 4096);
}

// Reduction splits of a launch of the shared group alone: with one M-tile
// of rows the launch has only `ntiles` items (88 for gate/up at hidden
// 11,264, 16 for down at d = 4,096), too few for 256 CUs.  Take the smallest
// split of the nch chunks that gives at least kSplitItems items while every
// split keeps at least kSplitMinChunks chunks (else the largest that does).
constexpr int kSplitItems = 320;
constexpr int kSplitMinChunks = 8;

int tiled_splits(int T, int ntiles, int nch) {
  if (T > kTileM || ntiles >= kSplitItems) return 1;
  int best = 1;
  for (int ks = 2; nch / ks >= kSplitMinChunks; ++ks) {
    if (nch % ks) continue;
    best = ks;
    if (ntiles * ks >= kSplitItems) break;
  }
  return best;
}

int gate_up_splits(int T, int d, int hs) { return tiled_splits(T, hs / (kTileN / 2), d / kChunk); }
int down_splits(int T, int d, int hs) { return tiled_splits(T, d / kTileN, hs / kChunk); }

}  // namespace

// Scratch for the splits the two launchers above take, each under the
// condition that sends its phase to the tiled kernels: gate/up when hs is a
// multiple of 128 (whatever d), down when d is a multiple of 256 (whatever
// hs).  Either may split while the other does not tile at all.
size_t tiled_split_bytes(int T, int d, int hs) {
  if (T > kTileM) return 0;
  const int kg = hs % (kTileN / 2) == 0 ? gate_up_splits(T, d, hs) : 1;
  const int kd = d % kTileN == 0 ? down_splits(T, d, hs) : 1;
  const size_t g = kg > 1 ? (size_t)kg * T * 2 * hs * sizeof(float) : 0;
  const size_t n = kd > 1 ? (size_t)kd * T * d * sizeof(float) : 0;
  return ((g > n ? g : n) + 255) / 256 * 256;
}

hipError_t launch_gate_up_tiled(int T, int d, int E, int k, int h, int hs, const uint16_t* x, const int32_t* offsets,
                                const int32_t* perm, const uint16_t* w_gu, const uint16_t* ws_gu, uint16_t* hid,
                                uint16_t* hid_shared, int32_t* queue, hipStream_t stream, float act_clamp,
                                float* partial) {
  if (T == 0) return hipSuccess;
  const Groups gs = make_groups(T, E, k, offsets, perm, ws_gu != nullptr);
  const int ks = partial && !offsets && ws_gu ? gate_up_splits(T, d, hs) : 1;
  hipLaunchKernelGGL(k_clear_queue, dim3(1), dim3(64), 0, stream, queue);
  if (ks > 1) {
    const auto kern = k_expert_tiled<kGateUp, false, true>;
    hipLaunchKernelGGL(kern, dim3(persistent_grid(kern, kThreads)), dim3(kThreads), 0, stream, x, x, gs, d, h, hs,
                       w_gu, ws_gu, hid, static_cast<void*>(hid_shared), queue, 0.f, ks, partial);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k_swiglu_splits, dim3(finish_grid((size_t)T * hs / 4)), dim3(256), 0, stream, partial, ks, T,
                       hs, act_clamp, hid_shared);
    return hipGetLastError();
  }
  const auto kern = act_clamp > 0.f ? k_expert_tiled<kGateUp, true> : k_expert_tiled<kGateUp, false>;
  hipLaunchKernelGGL(kern, dim3(persistent_grid(kern, kThreads)), dim3(kThreads), 0, stream, x, x, gs, d, h, hs,
                     w_gu, ws_gu, hid, static_cast<void*>(hid_shared), queue, act_clamp, 1, nullptr);
  return hipGetLastError();
}

hipError_t launch_down_tiled(int T, int d, int E, int k, int h, int hs, const int32_t* offsets, const uint16_t* hid,
                             const uint16_t* hid_shared, const uint16_t* w_down, const uint16_t* ws_down,
                             uint16_t* y_perm, float* y_shared, int32_t* queue, hipStream_t stream, float* partial) {
  if (T == 0) return hipSuccess;
  const Groups gs = make_groups(T, E, k, offsets, nullptr, ws_down != nullptr);
  const int ks = partial && !offsets && ws_down ? down_splits(T, d, hs) : 1;
  hipLaunchKernelGGL(k_clear_queue, dim3(1), dim3(64), 0, stream, queue);
  if (ks > 1) {
    const auto kern = k_expert_tiled<kDown, false, true>;
    hipLaunchKernelGGL(kern, dim3(persistent_grid(kern, kThreads)), dim3(kThreads), 0, stream, hid, hid_shared, gs,
                       d, h, hs, w_down, ws_down, y_perm, static_cast<void*>(y_shared), queue, 0.f, ks, partial);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const size_t n = (size_t)T * d;
    hipLaunchKernelGGL(k_sum_splits, dim3(finish_grid(n / 4)), dim3(256), 0, stream, partial, ks, n, y_shared);
    return hipGetLastError();
  }
  const auto kern = k_expert_tiled<kDown>;
  hipLaunchKernelGGL(kern, dim3(persistent_grid(kern, kThreads)), dim3(kThreads), 0, stream, hid, hid_shared, gs, d,
                     h, hs, w_down, ws_down, y_perm, static_cast<void*>(y_shared), queue, 0.f, 1, nullptr);
  return hipGetLastError();
}

}  // namespace moe
