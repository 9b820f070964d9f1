// permute.hip -- stable (expert, token) permutation of the T*k routed pairs:
// the gather/scatter order of the grouped expert GEMMs ([Blog] "Step 3.5
// Flash: Open Frontier-Level Intelligence with 11B Active Parameters" §3.2.4,
// fused MoE gather/scatter with grouped GEMM).
//
// Tokens are cut into chunks of 64 (one wavefront lane per token).  Within a
// chunk each expert gets a 64-bit LDS mask of the tokens that chose it, so a
// pair's rank among the chunk's pairs of the same expert is a popcount of the
// mask below its lane: the order inside an expert is the token order, with no
// sorting and no atomics on positions.
//   k_perm_count:   per-chunk, per-expert pair counts
//   k_perm_scan:    expert totals -> exclusive offsets; per-chunk bases
//   k_perm_scatter: perm_pairs / pair_pos from base + rank
// Small batches (at most kFusedChunks chunks) run the same three steps in one
// block, with the masks and bases in LDS: one launch instead of three.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kChunk = 64;

namespace {

__device__ __forceinline__ void build_chunk_masks(unsigned long long* mask, const int32_t* __restrict__ ids, int T,
                                                  int E, int k, int chunk) {
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += blockDim.x) mask[e] = 0ull;
  __syncthreads();
  if (tid < kChunk) {
    const int t = chunk * kChunk + tid;
    if (t < T)
      for (int j = 0; j < k; ++j) atomicOr(&mask[ids[(size_t)t * k + j]], 1ull << tid);
  }
  __syncthreads();
}

}  // namespace

__global__ __launch_bounds__(256) void k_perm_count(const int32_t* __restrict__ ids, int T, int E, int k,
                                                    int32_t* __restrict__ chunk_cnt) {
  __shared__ unsigned long long mask[1024];
  build_chunk_masks(mask, ids, T, E, k, blockIdx.x);
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    chunk_cnt[(size_t)blockIdx.x * E + e] = __popcll(mask[e]);
}

// One block of 1024 threads; thread e owns expert e.  Its column of chunk
// counts is read kScanBatch chunks at a time (loads of a batch in flight
// together), summed, then rewritten as running bases.
constexpr int kScanBatch = 32;

__global__ __launch_bounds__(1024) void k_perm_scan(int32_t* __restrict__ chunk_cnt, int nchunks, int E,
                                                    int32_t* __restrict__ offsets) {
  __shared__ int buf[2][1024];
  const int e = threadIdx.x;
  int total = 0;
  if (e < E)
    for (int c0 = 0; c0 < nchunks; c0 += kScanBatch) {
      int v[kScanBatch];
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) v[i] = c0 + i < nchunks ? chunk_cnt[(size_t)(c0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) total += v[i];
    }
  // Inclusive Hillis-Steele scan over the 1024 expert totals.
  int cur = 0;
  buf[cur][e] = total;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = buf[cur][e] + (e >= off ? buf[cur][e - off] : 0);
    buf[cur ^ 1][e] = v;
    cur ^= 1;
    __syncthreads();
  }
  const int excl = buf[cur][e] - total;
  if (e < E) {
    offsets[e] = excl;
    int run = excl;
    for (int c0 = 0; c0 < nchunks; c0 += kScanBatch) {
      int v[kScanBatch];
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) v[i] = c0 + i < nchunks ? chunk_cnt[(size_t)(c0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) {
        if (c0 + i < nchunks) chunk_cnt[(size_t)(c0 + i) * E + e] = run;
        run += v[i];
      }
    }
    if (e == E - 1) offsets[E] = excl + total;
  }
}

__global__ __launch_bounds__(256) void k_perm_scatter(const int32_t* __restrict__ ids, int T, int E, int k,
                                                      const int32_t* __restrict__ chunk_base,
                                                      int32_t* __restrict__ perm_pairs,
                                                      int32_t* __restrict__ pair_pos) {
  __shared__ unsigned long long mask[1024];
  build_chunk_masks(mask, ids, T, E, k, blockIdx.x);
  const int tid = threadIdx.x;
  if (tid < kChunk) {
    const int t = blockIdx.x * kChunk + tid;
    if (t < T) {
      const unsigned long long below = (1ull << tid) - 1ull;
      for (int j = 0; j < k; ++j) {
        const int e = ids[(size_t)t * k + j];
        const int pos = chunk_base[(size_t)blockIdx.x * E + e] + __popcll(mask[e] & below);
        perm_pairs[pos] = t * k + j;
        pair_pos[(size_t)t * k + j] = pos;
      }
    }
  }
}

constexpr int kFusedChunks = 16;          // chunks of the one-block path (T <= 1024)
constexpr int kFusedSlots = 8192;         // LDS (chunk, expert) slots of the one-block path

// The whole permutation in one block of 1024 threads (16 waves): wave c
// builds the masks of chunk c, thread e scans expert e's chunk counts and the
// block scans the expert totals, then thread t scatters token t's pairs.
// Same order as the three-kernel path: ranks are popcounts below the token's
// lane within its chunk, chunk bases follow chunk order.
__global__ __launch_bounds__(1024) void k_perm_fused(const int32_t* __restrict__ ids, int T, int E, int k,
                                                     int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ perm_pairs,
                                                     int32_t* __restrict__ pair_pos) {
  __shared__ unsigned long long mask[kFusedSlots];  // [chunk][expert]
  __shared__ int base[kFusedSlots];                 // [chunk][expert]
  __shared__ int buf[2][1024];
  const int tid = threadIdx.x;
  const int nchunks = (T + kChunk - 1) / kChunk;
  for (int i = tid; i < nchunks * E; i += 1024) mask[i] = 0ull;
  __syncthreads();
  const int lane = tid % kChunk;
  if (tid < T)
    for (int j = 0; j < k; ++j) atomicOr(&mask[(tid / kChunk) * E + ids[(size_t)tid * k + j]], 1ull << lane);
  __syncthreads();
  int total = 0;
  if (tid < E)
    for (int c = 0; c < nchunks; ++c) total += __popcll(mask[c * E + tid]);
  int cur = 0;
  buf[cur][tid] = total;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = buf[cur][tid] + (tid >= off ? buf[cur][tid - off] : 0);
    buf[cur ^ 1][tid] = v;
    cur ^= 1;
    __syncthreads();
  }
  if (tid < E) {
    const int excl = buf[cur][tid] - total;
    offsets[tid] = excl;
    int run = excl;
    for (int c = 0; c < nchunks; ++c) {
      base[c * E + tid] = run;
      run += __popcll(mask[c * E + tid]);
    }
    if (tid == E - 1) offsets[E] = excl + total;
  }
  __syncthreads();
  if (tid < T) {
    const int c = tid / kChunk;
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int j = 0; j < k; ++j) {
      const int e = ids[(size_t)tid * k + j];
      const int pos = base[c * E + e] + __popcll(mask[c * E + e] & below);
      perm_pairs[pos] = tid * k + j;
      pair_pos[(size_t)tid * k + j] = pos;
    }
  }
}

hipError_t launch_permute(int T, int E, int k, const int32_t* topk_ids, int32_t* expert_offsets,
                          int32_t* perm_pairs, int32_t* pair_pos, void* workspace, hipStream_t stream) {
  const int nchunks = (T + kChunk - 1) / kChunk;
  if (nchunks > 0 && nchunks <= kFusedChunks && nchunks * E <= kFusedSlots) {
    hipLaunchKernelGGL(k_perm_fused, dim3(1), dim3(1024), 0, stream, topk_ids, T, E, k, expert_offsets, perm_pairs,
                       pair_pos);
    return hipGetLastError();
  }
  int32_t* chunk_cnt = static_cast<int32_t*>(workspace);
  if (nchunks > 0) {
    hipLaunchKernelGGL(k_perm_count, dim3(nchunks), dim3(256), 0, stream, topk_ids, T, E, k, chunk_cnt);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(k_perm_scan, dim3(1), dim3(1024), 0, stream, chunk_cnt, nchunks, E, expert_offsets);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || nchunks == 0) return err;
  hipLaunchKernelGGL(k_perm_scatter, dim3(nchunks), dim3(256), 0, stream, topk_ids, T, E, k, chunk_cnt,
                     perm_pairs, pair_pos);
  return hipGetLastError();
}

size_t permute_workspace_bytes(int T, int E) {
  const size_t nchunks = (size_t)(T + kChunk - 1) / kChunk;
  return nchunks * (size_t)E * sizeof(int32_t);
}

}  // namespace moe
