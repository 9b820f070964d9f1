// abi.hip -- the C ABI of libmoe (declared in include/moe.h): host-side
// argument validation, workspace sizing, and dispatch to the kernel launchers.
// Validation runs before any HIP call, so a rejected call enqueues nothing.
#include <math.h>
#include <stdint.h>

#include <initializer_list>
#include <mutex>

#include "../../include/moe.h"
#include "kernels.h"

namespace {

constexpr int kMaxTokens = 1 << 20;
constexpr int kMaxDim = 65536;
constexpr int kMaxExperts = 1024;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

moe_status check_shape(const moe_shape* s) {
  if (!s) return MOE_ERR_INVALID_ARGUMENT;
  if (s->num_tokens < 0 || s->num_tokens > kMaxTokens) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (s->d_model < 64 || s->d_model > kMaxDim || s->d_model % 64) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (s->num_experts < 1 || s->num_experts > kMaxExperts) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (s->top_k < 1 || s->top_k > moe::kMaxTopK || s->top_k > s->num_experts) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (s->d_expert < 64 || s->d_expert > kMaxDim || s->d_expert % 64) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (s->d_shared != 0 && (s->d_shared < 64 || s->d_shared > kMaxDim || s->d_shared % 64))
    return MOE_ERR_UNSUPPORTED_SHAPE;
  // Every index the kernels form fits the int32 pair/row arithmetic.
  if ((int64_t)s->num_tokens * s->top_k > INT32_MAX / 2) return MOE_ERR_UNSUPPORTED_SHAPE;
  return MOE_OK;
}

size_t workspace_bytes(const moe_shape* s) {
  const int T = s->num_tokens, d = s->d_model, E = s->num_experts, k = s->top_k, h = s->d_expert;
  size_t b = moe::route_workspace_bytes(T, d, E);
  b = b > moe::permute_workspace_bytes(T, E) ? b : moe::permute_workspace_bytes(T, E);
  const size_t experts = moe::expert_hid_bytes(T, k, h) + moe::shared_hid_bytes(T, s->d_shared) + moe::kQueueBytes;
  b = b > experts ? b : experts;
  b = b > moe::combine_diag_workspace_bytes(T, k) ? b : moe::combine_diag_workspace_bytes(T, k);
  return round256(b > 256 ? b : 256);
}

moe_status check_workspace(const moe_shape* s, const void* ws, size_t ws_bytes) {
  if (!ws) return MOE_ERR_INVALID_ARGUMENT;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return MOE_ERR_MISALIGNED;
  if (ws_bytes < workspace_bytes(s)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return MOE_OK;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

}  // namespace

extern "C" {

const char* moe_status_str(moe_status status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED_SHAPE: return "MOE_ERR_UNSUPPORTED_SHAPE";
    case MOE_ERR_MISALIGNED: return "MOE_ERR_MISALIGNED";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

moe_status moe_check_shape(const moe_shape* shape) { return check_shape(shape); }

moe_status moe_workspace_bytes(const moe_shape* shape, size_t* bytes) {
  const moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID_ARGUMENT;
  *bytes = workspace_bytes(shape);
  return MOE_OK;
}

moe_status moe_route(const moe_shape* shape, const uint16_t* x, const uint16_t* w_router, const float* sel_bias,
                     const float* logit_bias, int32_t* topk_ids, float* topk_weights, int32_t* expert_counts,
                     float* topk_gap, void* workspace, size_t ws_bytes, void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!x || !w_router || !sel_bias || !topk_ids || !topk_weights || !expert_counts) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(w_router) || !aligned4(sel_bias) || !aligned4(topk_ids) ||
      !aligned4(topk_weights) || !aligned4(expert_counts) || (logit_bias && !aligned4(logit_bias)) ||
      (topk_gap && !aligned4(topk_gap)))
    return MOE_ERR_MISALIGNED;
  if ((st = check_workspace(shape, workspace, ws_bytes)) != MOE_OK) return st;
  return hip_status(moe::launch_route(shape->num_tokens, shape->d_model, shape->num_experts, shape->top_k, x,
                                      w_router, sel_bias, logit_bias, topk_ids, topk_weights, expert_counts,
                                      topk_gap, nullptr, workspace, (hipStream_t)stream));
}

moe_status moe_rmsnorm_route(const moe_shape* shape, const uint16_t* h, const float* gamma, float eps,
                             const uint16_t* w_router, const float* sel_bias, const float* logit_bias,
                             uint16_t* x_out, int32_t* topk_ids, float* topk_weights, int32_t* expert_counts,
                             float* topk_gap, void* workspace, size_t ws_bytes, void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!h || !w_router || !sel_bias || !x_out || !topk_ids || !topk_weights || !expert_counts)
    return MOE_ERR_INVALID_ARGUMENT;
  if (h == x_out || !(eps >= 0.0f) || !isfinite(eps)) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(h) || !aligned16(x_out) || !aligned16(w_router) || !aligned4(sel_bias) || !aligned4(topk_ids) ||
      !aligned4(topk_weights) || !aligned4(expert_counts) || (gamma && !aligned4(gamma)) ||
      (logit_bias && !aligned4(logit_bias)) || (topk_gap && !aligned4(topk_gap)))
    return MOE_ERR_MISALIGNED;
  if ((st = check_workspace(shape, workspace, ws_bytes)) != MOE_OK) return st;
  const moe::RouteNorm norm{gamma, eps, x_out};
  return hip_status(moe::launch_route(shape->num_tokens, shape->d_model, shape->num_experts, shape->top_k, h,
                                      w_router, sel_bias, logit_bias, topk_ids, topk_weights, expert_counts,
                                      topk_gap, nullptr, workspace, (hipStream_t)stream, &norm));
}

moe_status moe_route_diag(const moe_shape* shape, const uint16_t* x, const uint16_t* w_router, const float* sel_bias,
                          const float* logit_bias, int32_t* topk_ids, float* topk_weights, int32_t* expert_counts,
                          float* topk_gap, int32_t ep_groups, float* p_e, float* f_e, float* summary,
                          void* workspace, size_t ws_bytes, void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!x || !w_router || !sel_bias || !topk_ids || !topk_weights || !expert_counts || !p_e || !f_e || !summary)
    return MOE_ERR_INVALID_ARGUMENT;
  if (ep_groups < 1 || ep_groups > shape->num_experts || shape->num_experts % ep_groups != 0)
    return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(w_router) || !aligned4(sel_bias) || !aligned4(topk_ids) ||
      !aligned4(topk_weights) || !aligned4(expert_counts) || (logit_bias && !aligned4(logit_bias)) ||
      (topk_gap && !aligned4(topk_gap)) || !aligned4(p_e) || !aligned4(f_e) || !aligned4(summary))
    return MOE_ERR_MISALIGNED;
  if ((st = check_workspace(shape, workspace, ws_bytes)) != MOE_OK) return st;
  const moe::RouteDiag diag{ep_groups, p_e, f_e, summary};
  return hip_status(moe::launch_route(shape->num_tokens, shape->d_model, shape->num_experts, shape->top_k, x,
                                      w_router, sel_bias, logit_bias, topk_ids, topk_weights, expert_counts,
                                      topk_gap, &diag, workspace, (hipStream_t)stream));
}

moe_status moe_permute(const moe_shape* shape, const int32_t* topk_ids, int32_t* expert_offsets,
                       int32_t* perm_pairs, int32_t* pair_pos, void* workspace, size_t ws_bytes, void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!topk_ids || !expert_offsets || !perm_pairs || !pair_pos) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned4(topk_ids) || !aligned4(expert_offsets) || !aligned4(perm_pairs) || !aligned4(pair_pos))
    return MOE_ERR_MISALIGNED;
  if ((st = check_workspace(shape, workspace, ws_bytes)) != MOE_OK) return st;
  return hip_status(moe::launch_permute(shape->num_tokens, shape->num_experts, shape->top_k, topk_ids,
                                        expert_offsets, perm_pairs, pair_pos, workspace, (hipStream_t)stream));
}

// The shared-expert pointers of the grouped calls come as a set: all NULL
// (routed experts only) or all given (then d_shared > 0).
static moe_status shared_set(const moe_shape* s, std::initializer_list<const void*> ptrs, bool* use) {
  int given = 0;
  for (const void* p : ptrs) given += p != nullptr;
  if (given != 0 && given != (int)ptrs.size()) return MOE_ERR_INVALID_ARGUMENT;
  if (given != 0 && s->d_shared == 0) return MOE_ERR_INVALID_ARGUMENT;
  *use = given != 0;
  return MOE_OK;
}

moe_status moe_expert_gate_up(const moe_shape* shape, const uint16_t* x, const int32_t* expert_offsets,
                              const int32_t* perm_pairs, const uint16_t* w_gate_up, const uint16_t* ws_gate_up,
                              uint16_t* hid, uint16_t* hid_shared, void* workspace, size_t ws_bytes, void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!x || !expert_offsets || !perm_pairs || !w_gate_up || !hid) return MOE_ERR_INVALID_ARGUMENT;
  bool shared = false;
  if ((st = shared_set(shape, {ws_gate_up, hid_shared}, &shared)) != MOE_OK) return st;
  if (!aligned16(x) || !aligned16(w_gate_up) || !aligned16(hid) || !aligned4(expert_offsets) ||
      !aligned4(perm_pairs) || (shared && (!aligned16(ws_gate_up) || !aligned16(hid_shared))))
    return MOE_ERR_MISALIGNED;
  if ((st = check_workspace(shape, workspace, ws_bytes)) != MOE_OK) return st;
  return hip_status(moe::launch_gate_up(shape->num_tokens, shape->d_model, shape->num_experts, shape->top_k,
                                        shape->d_expert, shape->d_shared, x, expert_offsets, perm_pairs, w_gate_up,
                                        shared ? ws_gate_up : nullptr, hid, hid_shared,
                                        static_cast<int32_t*>(workspace), (hipStream_t)stream));
}

moe_status moe_expert_down(const moe_shape* shape, const int32_t* expert_offsets, const uint16_t* hid,
                           const uint16_t* hid_shared, const uint16_t* w_down, const uint16_t* ws_down,
                           uint16_t* y_perm, float* y_shared, void* workspace, size_t ws_bytes, void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!expert_offsets || !hid || !w_down || !y_perm) return MOE_ERR_INVALID_ARGUMENT;
  bool shared = false;
  if ((st = shared_set(shape, {hid_shared, ws_down, y_shared}, &shared)) != MOE_OK) return st;
  if (!aligned16(hid) || !aligned16(w_down) || !aligned16(y_perm) || !aligned4(expert_offsets) ||
      (shared && (!aligned16(hid_shared) || !aligned16(ws_down) || !aligned16(y_shared))))
    return MOE_ERR_MISALIGNED;
  if ((st = check_workspace(shape, workspace, ws_bytes)) != MOE_OK) return st;
  return hip_status(moe::launch_down(shape->num_tokens, shape->d_model, shape->num_experts, shape->top_k,
                                     shape->d_expert, shape->d_shared, expert_offsets, hid, hid_shared, w_down,
                                     shared ? ws_down : nullptr, y_perm, y_shared, static_cast<int32_t*>(workspace),
                                     (hipStream_t)stream));
}

// Checks of moe_expert_swiglu's arguments other than the workspace.
static moe_status expert_swiglu_args(const moe_shape* shape, const uint16_t* x, const int32_t* expert_offsets,
                                     const int32_t* perm_pairs, const uint16_t* w_gate_up, const uint16_t* w_down,
                                     const uint16_t* ws_gate_up, const uint16_t* ws_down, const uint16_t* y_perm,
                                     const float* y_shared, bool* shared) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!x || !expert_offsets || !perm_pairs || !w_gate_up || !w_down || !y_perm) return MOE_ERR_INVALID_ARGUMENT;
  if ((st = shared_set(shape, {ws_gate_up, ws_down, y_shared}, shared)) != MOE_OK) return st;
  if (!aligned16(x) || !aligned16(w_gate_up) || !aligned16(w_down) || !aligned16(y_perm) ||
      !aligned4(expert_offsets) || !aligned4(perm_pairs) ||
      (*shared && (!aligned16(ws_gate_up) || !aligned16(ws_down) || !aligned16(y_shared))))
    return MOE_ERR_MISALIGNED;
  return MOE_OK;
}

// Scratch of the grouped expert calls, [work queue | hid | hid_shared]:
// its size, and the launches of both phases on it.
static size_t expert_scratch_bytes(const moe_shape* s, bool shared) {
  return moe::kQueueBytes + moe::expert_hid_bytes(s->num_tokens, s->top_k, s->d_expert) +
         (shared ? moe::shared_hid_bytes(s->num_tokens, s->d_shared) : 0);
}

static moe_status expert_swiglu_on(const moe_shape* shape, const uint16_t* x, const int32_t* expert_offsets,
                                   const int32_t* perm_pairs, const uint16_t* w_gate_up, const uint16_t* w_down,
                                   const uint16_t* ws_gate_up, const uint16_t* ws_down, uint16_t* y_perm,
                                   float* y_shared, bool shared, void* scratch, void* stream) {
  const int T = shape->num_tokens, d = shape->d_model, E = shape->num_experts, k = shape->top_k;
  const int h = shape->d_expert, hs = shape->d_shared;
  int32_t* queue = static_cast<int32_t*>(scratch);
  uint16_t* hid = reinterpret_cast<uint16_t*>(static_cast<char*>(scratch) + moe::kQueueBytes);
  uint16_t* hid_shared = shared ? hid + moe::expert_hid_bytes(T, k, h) / 2 : nullptr;
  hipError_t err = moe::launch_gate_up(T, d, E, k, h, hs, x, expert_offsets, perm_pairs, w_gate_up,
                                       shared ? ws_gate_up : nullptr, hid, hid_shared, queue, (hipStream_t)stream);
  if (err == hipSuccess)
    err = moe::launch_down(T, d, E, k, h, hs, expert_offsets, hid, hid_shared, w_down, shared ? ws_down : nullptr,
                           y_perm, shared ? y_shared : nullptr, queue, (hipStream_t)stream);
  return hip_status(err);
}

moe_status moe_expert_swiglu(const moe_shape* shape, const uint16_t* x, const int32_t* expert_offsets,
                             const int32_t* perm_pairs, const uint16_t* w_gate_up, const uint16_t* w_down,
                             const uint16_t* ws_gate_up, const uint16_t* ws_down, uint16_t* y_perm, float* y_shared,
                             void* workspace, size_t ws_bytes, void* stream) {
  bool shared = false;
  moe_status st = expert_swiglu_args(shape, x, expert_offsets, perm_pairs, w_gate_up, w_down, ws_gate_up, ws_down,
                                     y_perm, y_shared, &shared);
  if (st != MOE_OK) return st;
  if ((st = check_workspace(shape, workspace, ws_bytes)) != MOE_OK) return st;
  return expert_swiglu_on(shape, x, expert_offsets, perm_pairs, w_gate_up, w_down, ws_gate_up, ws_down, y_perm,
                          y_shared, shared, workspace, stream);
}

}  // extern "C"

// Scratch of moe_expert_swiglu_noalloc: one array per GPU, in the library's
// own device memory, held until the process ends.  In host code `scratch` is
// only a handle of the symbol, not a device address: the address each device
// holds its copy at is looked up once per device (device_scratch) and only
// that address is handed to kernels.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_addr[kMaxDevices];

// This device's copy of `scratch` (the current device), looked up on the
// first call on that device with it current.
hipError_t device_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    scratch_addr[dev] = p;
  }
  *out = scratch_addr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

moe_status moe_expert_swiglu_noalloc(const moe_shape* shape, const uint16_t* x, const int32_t* expert_offsets,
                                     const int32_t* perm_pairs, const uint16_t* w_gate_up, const uint16_t* w_down,
                                     const uint16_t* ws_gate_up, const uint16_t* ws_down, uint16_t* y_perm,
                                     float* y_shared, void* stream) {
  bool shared = false;
  const moe_status st = expert_swiglu_args(shape, x, expert_offsets, perm_pairs, w_gate_up, w_down, ws_gate_up,
                                           ws_down, y_perm, y_shared, &shared);
  if (st != MOE_OK) return st;
  if (expert_scratch_bytes(shape, shared) > kNoAllocScratchBytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  if (device_scratch(&ws) != hipSuccess) return MOE_ERR_HIP;
  return expert_swiglu_on(shape, x, expert_offsets, perm_pairs, w_gate_up, w_down, ws_gate_up, ws_down, y_perm,
                          y_shared, shared, ws, stream);
}

moe_status moe_expert_swiglu_clamped(const moe_shape* shape, const uint16_t* x, const int32_t* expert_offsets,
                                     const int32_t* perm_pairs, const uint16_t* w_gate_up, const uint16_t* w_down,
                                     const uint16_t* ws_gate_up, const uint16_t* ws_down, uint16_t* y_perm,
                                     float* y_shared, float act_clamp, void* workspace, size_t ws_bytes,
                                     void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!(act_clamp > 0.0f) || !isfinite(act_clamp)) return MOE_ERR_INVALID_ARGUMENT;
  if (!x || !expert_offsets || !perm_pairs || !w_gate_up || !w_down || !y_perm) return MOE_ERR_INVALID_ARGUMENT;
  bool shared = false;
  if ((st = shared_set(shape, {ws_gate_up, ws_down, y_shared}, &shared)) != MOE_OK) return st;
  if (!aligned16(x) || !aligned16(w_gate_up) || !aligned16(w_down) || !aligned16(y_perm) ||
      !aligned4(expert_offsets) || !aligned4(perm_pairs) ||
      (shared && (!aligned16(ws_gate_up) || !aligned16(ws_down) || !aligned16(y_shared))))
    return MOE_ERR_MISALIGNED;
  if ((st = check_workspace(shape, workspace, ws_bytes)) != MOE_OK) return st;
  const int T = shape->num_tokens, d = shape->d_model, E = shape->num_experts, k = shape->top_k;
  const int h = shape->d_expert, hs = shape->d_shared;
  int32_t* queue = static_cast<int32_t*>(workspace);
  uint16_t* hid = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + moe::kQueueBytes);
  uint16_t* hid_shared = shared ? hid + moe::expert_hid_bytes(T, k, h) / 2 : nullptr;
  hipError_t err = moe::launch_gate_up(T, d, E, k, h, hs, x, expert_offsets, perm_pairs, w_gate_up,
                                       shared ? ws_gate_up : nullptr, hid, hid_shared, queue, (hipStream_t)stream, 0,
                                       act_clamp);
  if (err == hipSuccess)
    err = moe::launch_down(T, d, E, k, h, hs, expert_offsets, hid, hid_shared, w_down, shared ? ws_down : nullptr,
                           y_perm, shared ? y_shared : nullptr, queue, (hipStream_t)stream);
  return hip_status(err);
}

moe_status moe_expert_swiglu_range(const moe_shape* shape, int32_t expert_begin, int32_t expert_end,
                                   const uint16_t* x, const int32_t* expert_offsets, const int32_t* perm_pairs,
                                   const uint16_t* w_gate_up, const uint16_t* w_down, uint16_t* y_perm,
                                   void* workspace, size_t ws_bytes, void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (expert_begin < 0 || expert_end > shape->num_experts || expert_begin >= expert_end)
    return MOE_ERR_INVALID_ARGUMENT;
  if (!x || !expert_offsets || !perm_pairs || !w_gate_up || !w_down || !y_perm) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(w_gate_up) || !aligned16(w_down) || !aligned16(y_perm) ||
      !aligned4(expert_offsets) || !aligned4(perm_pairs))
    return MOE_ERR_MISALIGNED;
  if ((st = check_workspace(shape, workspace, ws_bytes)) != MOE_OK) return st;
  // The share's groups are experts begin..end-1: their offsets entries hold
  // absolute rows of the permuted order, so the share's rows land where the
  // whole call would put them; the weights are the share's own.
  const int T = shape->num_tokens, d = shape->d_model, E = shape->num_experts, k = shape->top_k;
  const int h = shape->d_expert, hs = shape->d_shared, El = expert_end - expert_begin;
  const int32_t* off = expert_offsets + expert_begin;
  int32_t* queue = static_cast<int32_t*>(workspace);
  uint16_t* hid = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + moe::kQueueBytes);
  hipError_t err = moe::launch_gate_up(T, d, El, k, h, hs, x, off, perm_pairs, w_gate_up, nullptr, hid, nullptr,
                                       queue, (hipStream_t)stream, E);
  if (err == hipSuccess)
    err = moe::launch_down(T, d, El, k, h, hs, off, hid, nullptr, w_down, nullptr, y_perm, nullptr, queue,
                           (hipStream_t)stream, E);
  return hip_status(err);
}

moe_status moe_shared_swiglu(const moe_shape* shape, const uint16_t* x, const uint16_t* ws_gate_up,
                             const uint16_t* ws_down, float* y_shared, void* workspace, size_t ws_bytes,
                             void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (shape->d_shared == 0) return MOE_ERR_INVALID_ARGUMENT;
  if (!x || !ws_gate_up || !ws_down || !y_shared) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(ws_gate_up) || !aligned16(ws_down) || !aligned16(y_shared))
    return MOE_ERR_MISALIGNED;
  if ((st = check_workspace(shape, workspace, ws_bytes)) != MOE_OK) return st;
  const int T = shape->num_tokens, d = shape->d_model, E = shape->num_experts, k = shape->top_k;
  const int h = shape->d_expert, hs = shape->d_shared;
  // Workspace: [work queue | hid_shared].
  int32_t* queue = static_cast<int32_t*>(workspace);
  uint16_t* hid_shared = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + moe::kQueueBytes);
  hipError_t err = moe::launch_gate_up(T, d, E, k, h, hs, x, nullptr, nullptr, nullptr, ws_gate_up, nullptr,
                                       hid_shared, queue, (hipStream_t)stream);
  if (err == hipSuccess)
    err = moe::launch_down(T, d, E, k, h, hs, nullptr, nullptr, hid_shared, nullptr, ws_down, nullptr, y_shared,
                           queue, (hipStream_t)stream);
  return hip_status(err);
}

moe_status moe_combine(const moe_shape* shape, const uint16_t* y_perm, const int32_t* pair_pos,
                       const float* topk_weights, const float* y_shared, float routed_scale, uint16_t* y,
                       void* stream) {
  const moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!y_perm || !pair_pos || !topk_weights || !y) return MOE_ERR_INVALID_ARGUMENT;
  if (!isfinite(routed_scale)) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(y_perm) || !aligned16(y) || !aligned4(pair_pos) || !aligned4(topk_weights) ||
      (y_shared && !aligned16(y_shared)))
    return MOE_ERR_MISALIGNED;
  return hip_status(moe::launch_combine(shape->num_tokens, shape->d_model, shape->top_k, y_perm, pair_pos,
                                        topk_weights, y_shared, nullptr, routed_scale, y, nullptr, nullptr,
                                        (hipStream_t)stream));
}

moe_status moe_combine_residual(const moe_shape* shape, const uint16_t* y_perm, const int32_t* pair_pos,
                                const float* topk_weights, const float* y_shared, float routed_scale,
                                const uint16_t* residual, uint16_t* y, void* stream) {
  const moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!y_perm || !pair_pos || !topk_weights || !residual || !y) return MOE_ERR_INVALID_ARGUMENT;
  if (!isfinite(routed_scale)) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(y_perm) || !aligned16(y) || !aligned16(residual) || !aligned4(pair_pos) ||
      !aligned4(topk_weights) || (y_shared && !aligned16(y_shared)))
    return MOE_ERR_MISALIGNED;
  return hip_status(moe::launch_combine(shape->num_tokens, shape->d_model, shape->top_k, y_perm, pair_pos,
                                        topk_weights, y_shared, residual, routed_scale, y, nullptr, nullptr,
                                        (hipStream_t)stream));
}

moe_status moe_combine_diag(const moe_shape* shape, const uint16_t* y_perm, const int32_t* pair_pos,
                            const float* topk_weights, const float* y_shared, float routed_scale, uint16_t* y,
                            const int32_t* expert_offsets, float* expert_rms, float* rms_ratio, void* workspace,
                            size_t ws_bytes, void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!y_perm || !pair_pos || !topk_weights || !y || !expert_offsets || !expert_rms) return MOE_ERR_INVALID_ARGUMENT;
  if (!isfinite(routed_scale)) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(y_perm) || !aligned16(y) || !aligned4(pair_pos) || !aligned4(topk_weights) ||
      (y_shared && !aligned16(y_shared)) || !aligned4(expert_offsets) || !aligned4(expert_rms) ||
      (rms_ratio && !aligned4(rms_ratio)))
    return MOE_ERR_MISALIGNED;
  if ((st = check_workspace(shape, workspace, ws_bytes)) != MOE_OK) return st;
  const moe::CombineDiag diag{shape->num_experts, expert_offsets, expert_rms, rms_ratio};
  return hip_status(moe::launch_combine(shape->num_tokens, shape->d_model, shape->top_k, y_perm, pair_pos,
                                        topk_weights, y_shared, nullptr, routed_scale, y, &diag, workspace,
                                        (hipStream_t)stream));
}

moe_status moe_dense_workspace_bytes(int32_t num_tokens, int32_t d_model, int32_t d_hidden, size_t* bytes) {
  if (!bytes) return MOE_ERR_INVALID_ARGUMENT;
  if (num_tokens < 0 || num_tokens > kMaxTokens || d_model < 64 || d_model > kMaxDim || d_model % 64 ||
      d_hidden < 64 || d_hidden > kMaxDim || d_hidden % 64)
    return MOE_ERR_UNSUPPORTED_SHAPE;
  *bytes = round256(moe::kQueueBytes + moe::shared_hid_bytes(num_tokens, d_hidden) +
                    moe::split_partial_bytes(num_tokens, d_model, d_hidden));
  return MOE_OK;
}

moe_status moe_dense_swiglu(int32_t num_tokens, int32_t d_model, int32_t d_hidden, const uint16_t* x,
                            const uint16_t* w_gate_up, const uint16_t* w_down, float* y, void* workspace,
                            size_t ws_bytes, void* stream) {
  size_t need = 0;
  moe_status st = moe_dense_workspace_bytes(num_tokens, d_model, d_hidden, &need);
  if (st != MOE_OK) return st;
  if (!x || !w_gate_up || !w_down || !y || !workspace) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(w_gate_up) || !aligned16(w_down) || !aligned16(y)) return MOE_ERR_MISALIGNED;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return MOE_ERR_MISALIGNED;
  if (ws_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  // One group holding every token: the shared-expert group of the grouped
  // launches, with no routed groups (the routed sizes are placeholders that
  // no kernel reads).
  const int T = num_tokens, d = d_model, H = d_hidden;
  int32_t* queue = static_cast<int32_t*>(workspace);
  uint16_t* hid = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + moe::kQueueBytes);
  // Workspace: [work queue | hid | split partial sums].
  float* partial = moe::split_partial_bytes(T, d, H)
                       ? reinterpret_cast<float*>(static_cast<char*>(workspace) + moe::kQueueBytes +
                                                  moe::shared_hid_bytes(T, H))
                       : nullptr;
  if (moe::dense_ffn_fits(T, d, H))
    return hip_status(moe::launch_dense_ffn(T, d, H, x, w_gate_up, w_down, hid, partial, y, 0.f, (hipStream_t)stream));
  hipError_t err = moe::launch_gate_up(T, d, 1, 1, 128, H, x, nullptr, nullptr, nullptr, w_gate_up, nullptr, hid,
                                       queue, (hipStream_t)stream, 0, 0.f, partial);
  if (err == hipSuccess)
    err = moe::launch_down(T, d, 1, 1, 128, H, nullptr, nullptr, hid, nullptr, w_down, nullptr, y, queue,
                           (hipStream_t)stream, 0, partial);
  return hip_status(err);
}

moe_status moe_rmsnorm(int32_t rows, int32_t cols, const uint16_t* in, const float* gamma, float eps, uint16_t* out,
                       void* stream) {
  if (rows < 0 || rows > kMaxTokens || cols < 8 || cols > kMaxDim || cols % 8) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (!in || !out || in == out) return MOE_ERR_INVALID_ARGUMENT;
  if (!(eps >= 0.0f) || !isfinite(eps)) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(in) || !aligned16(out) || (gamma && !aligned4(gamma))) return MOE_ERR_MISALIGNED;
  return hip_status(moe::launch_rmsnorm(rows, cols, in, gamma, eps, out, (hipStream_t)stream));
}

}  // extern "C"
