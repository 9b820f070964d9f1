// kernels.h -- libmoe-internal launchers (one per kernel family).  Shapes are
// validated by the C ABI layer before any of these is called.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kMaxTopK = 16;  // largest top_k the C ABI accepts

// How the router's logits are computed: the split of the d-long reduction
// into ksplit chunks of kchunk, and whether the LDS-staged kernel (large
// batches) is used.
struct RouteSplit {
  int ksplit, kchunk;
  bool tiled;
};
RouteSplit route_split(int T, int d, int E);

// Routing diagnostics produced beside the routing outputs: p_e [E], f_e [E]
// and summary [2] = (L_EP over `groups` contiguous expert groups, routing
// confidence).
struct RouteDiag {
  int groups;
  float* p_e;
  float* f_e;
  float* summary;
};
// RMSNorm in front of the router: x is the un-normalised stream h, and the
// normalised rows bf16(h / rms(h) * (1 + gamma)) are written to x_out (the
// experts' input) and routed.
struct RouteNorm {
  const float* gamma;
  float eps;
  uint16_t* x_out;
};
hipError_t launch_route(int T, int d, int E, int k, const uint16_t* x, const uint16_t* w_router,
                        const float* sel_bias, const float* logit_bias, int32_t* topk_ids, float* topk_weights,
                        int32_t* counts, float* topk_gap, const RouteDiag* diag, void* workspace,
                        hipStream_t stream, const RouteNorm* norm = nullptr);
size_t route_workspace_bytes(int T, int d, int E);

hipError_t launch_permute(int T, int E, int k, const int32_t* topk_ids, int32_t* expert_offsets,
                          int32_t* perm_pairs, int32_t* pair_pos, void* workspace, hipStream_t stream);
size_t permute_workspace_bytes(int T, int E);

// Grouped expert GEMMs.  Routed groups come from expert_offsets/perm (NULL
// offsets: none); the shared expert is one more group when its weights are
// given (ws_gu / ws_down non-NULL).  `queue` is kQueueBytes of device scratch
// for the work queue of the compute-regime kernels.
constexpr size_t kQueueBytes = 256;
// e_total: the experts the routing chose among, when the routed groups are a
// contiguous share of them (offsets then points at the share's first entry
// and E counts the share); 0 means E.  It sets the regime, which follows the
// average rows per expert.  act_clamp > 0 clips every hidden activation to
// [-act_clamp, act_clamp] before its bf16 rounding.
// partial: optional f32 scratch of split_partial_bytes(T, d, hs) for a
// launch of the shared group alone with few rows, which may then split the
// reduction over items and add their sums afterwards (in a fixed order).
hipError_t launch_gate_up(int T, int d, int E, int k, int h, int hs, const uint16_t* x, const int32_t* offsets,
                          const int32_t* perm, const uint16_t* w_gu, const uint16_t* ws_gu, uint16_t* hid,
                          uint16_t* hid_shared, int32_t* queue, hipStream_t stream, int e_total = 0,
                          float act_clamp = 0.f, float* partial = nullptr);
// The streaming down kernel's split for the shared group alone: kDownSplits
// items per output tile, up to kDownSplitMaxTokens tokens.
constexpr int kDownSplits = 4;
constexpr int kDownSplitMaxTokens = 256;
hipError_t launch_down(int T, int d, int E, int k, int h, int hs, const int32_t* offsets, const uint16_t* hid,
                       const uint16_t* hid_shared, const uint16_t* w_down, const uint16_t* ws_down, uint16_t* y_perm,
                       float* y_shared, int32_t* queue, hipStream_t stream, int e_total = 0,
                       float* partial = nullptr);
size_t split_partial_bytes(int T, int d, int hs);
// The compute-regime (LDS-tiled, MFMA 32x32x16) versions of the same two
// phases; the launchers above pick them when groups are large.  With
// `partial` (the shared group alone, one M-tile of rows) they split the
// reduction over items as tiled_split_bytes allows for.
hipError_t launch_gate_up_tiled(int T, int d, int E, int k, int h, int hs, const uint16_t* x, const int32_t* offsets,
                                const int32_t* perm, const uint16_t* w_gu, const uint16_t* ws_gu, uint16_t* hid,
                                uint16_t* hid_shared, int32_t* queue, hipStream_t stream, float act_clamp = 0.f,
                                float* partial = nullptr);
hipError_t launch_down_tiled(int T, int d, int E, int k, int h, int hs, const int32_t* offsets, const uint16_t* hid,
                             const uint16_t* hid_shared, const uint16_t* w_down, const uint16_t* ws_down,
                             uint16_t* y_perm, float* y_shared, int32_t* queue, hipStream_t stream,
                             float* partial = nullptr);
size_t tiled_split_bytes(int T, int d, int hs);
// The dense SwiGLU FFN at up to kDenseMaxTokens tokens (each CU streams a
// fixed share of both weight matrices once).  dense_ffn_fits says whether a
// shape suits it.  hid: T x H bf16; partial: kDenseDownSplits x T x d floats
// (split_partial_bytes covers it).
constexpr int kDenseMaxTokens = 64;
constexpr int kDenseDownSplits = kDownSplits;
bool dense_ffn_fits(int T, int d, int H);
hipError_t launch_dense_ffn(int T, int d, int H, const uint16_t* x, const uint16_t* w_gu, const uint16_t* w_d,
                            uint16_t* hid, float* partial, float* y, float clamp, hipStream_t stream);
size_t expert_hid_bytes(int T, int k, int h);
size_t shared_hid_bytes(int T, int hs);

// Per-expert activation RMS produced by the combine: rms [E+1] (entry E:
// the shared expert) and, if non-NULL, ratio [2] = (min, max) / median over
// the routed experts that received rows.  Uses combine_diag_workspace_bytes.
struct CombineDiag {
  int E;
  const int32_t* offsets;
  float* rms;
  float* ratio;
};
hipError_t launch_combine(int T, int d, int k, const uint16_t* y_perm, const int32_t* pair_pos,
                          const float* topk_weights, const float* y_shared, const uint16_t* residual,
                          float routed_scale, uint16_t* y, const CombineDiag* diag, void* workspace,
                          hipStream_t stream);
size_t combine_diag_workspace_bytes(int T, int k);
hipError_t launch_rmsnorm(int rows, int cols, const uint16_t* in, const float* gamma, float eps, uint16_t* out,
                          hipStream_t stream);

}  // namespace moe
