/* moe.h -- libmoe: forward pass of one fine-grained sparse Mixture-of-Experts
 * FFN layer on an AMD Instinct MI355X (gfx950).
 *
 * Pages cited (by title):
 *   [Blog]    "Step 3.5 Flash: Open Frontier-Level Intelligence with 11B Active
 *             Parameters" (section-numbered summary of the paper)
 *   [Digest]  "Step 3.5 Flash 技术论文深度解读：196B MoE 如何做到 11B 激活打 37B"
 *   [Article] "StepFun团队Step 3.5 Flash：11B参数实现前沿智能水平"
 *
 * The layer ([Blog] §2.2 and §2.2.2; [Digest] architecture table): a router
 * scores every token against E routed experts, a bias used only for selection
 * steers the top-k choice (loss-free balancing, [Digest] note under the
 * architecture table; [Article] §9), the chosen SwiGLU experts ([Digest]
 * activation-explosion cause 3: gate and up branches) run on the token, one
 * shared expert runs on every token, and the routed outputs are weighted,
 * explicitly scaled ([Blog] §4.1.2) and added to the shared output.  The
 * pages' own kernels fuse MoE gather/scatter with a grouped GEMM ([Blog]
 * §3.2.4); here the same structure is five calls:
 *
 *   moe_route          router logits, sigmoid, biased top-k, weights, counts
 *   moe_permute        stable (expert, token) permutation of the k*T pairs
 *   moe_expert_swiglu  grouped gate/up GEMM + SwiGLU, then grouped down GEMM
 *                      (also callable as its two phases, moe_expert_gate_up
 *                      and moe_expert_down, on a contiguous share of the
 *                      experts, moe_expert_swiglu_range, and with clipped
 *                      hidden activations, moe_expert_swiglu_clamped)
 *   moe_shared_swiglu  the always-on shared expert
 *   moe_combine        y = y_shared + routed_scale * sum_j w_j * y_perm[pos]
 *
 * with fused variants of the first and last (the RMSNorm in front of the
 * layer, the residual add behind it):
 *   moe_rmsnorm_route    RMSNorm(h) -> x_out, then moe_route on it
 *   moe_combine_residual moe_combine plus the skip connection
 * and diagnostic variants of two of them (same outputs, plus side outputs):
 *   moe_route_diag     + load-balance and confidence statistics of the routing
 *   moe_combine_diag   + per-expert activation RMS and its spread
 *
 * plus moe_rmsnorm, the zero-centred RMSNorm that sits in front of every FFN
 * sub-layer ([Blog] §2.2, Figure 2 caption), used between stacked layers.
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates or frees device memory and keeps no state between
 *     calls (the one exception: moe_expert_swiglu_noalloc's static scratch
 *     array, below).  bf16 tensors are passed as uint16_t bit patterns.
 *   - Matrices are row-major [out][in] (the reduction dimension contiguous).
 *   - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *     Calls only enqueue work: they never synchronise and never copy to the
 *     host.  Asynchronous kernel faults surface at the caller's next
 *     synchronisation.
 *   - Arguments are validated on the host before anything is enqueued; on a
 *     validation failure nothing is enqueued and the error code is returned.
 *     A failed kernel launch returns MOE_ERR_HIP.  No C++ exception crosses
 *     this interface.
 *   - Device data coming from elsewhere (ids, offsets, positions) is a
 *     precondition, not checked: it must be what moe_route / moe_permute
 *     produce for the same shape.
 *   - `workspace` is caller-provided device scratch of at least
 *     moe_workspace_bytes() bytes, 256-byte aligned.  Nothing in it survives
 *     a call.  Calls that may run concurrently (on different streams) need
 *     distinct workspaces.
 *   - Vector-loaded tensors must be 16-byte aligned (MOE_ERR_MISALIGNED).
 */
#ifndef LIBMOE_MOE_H_
#define LIBMOE_MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Layer shape.  Limits (MOE_ERR_UNSUPPORTED_SHAPE otherwise):
 *   0 <= num_tokens <= 1048576
 *   64 <= d_model <= 65536, d_model % 64 == 0
 *   1 <= num_experts <= 1024
 *   1 <= top_k <= min(num_experts, 16)
 *   64 <= d_expert <= 65536, d_expert % 64 == 0
 *   d_shared == 0 (no shared expert) or as d_expert                         */
typedef struct moe_shape {
  int32_t num_tokens;  /* T   */
  int32_t d_model;     /* d   */
  int32_t num_experts; /* E   */
  int32_t top_k;       /* k   */
  int32_t d_expert;    /* h   routed expert hidden size  */
  int32_t d_shared;    /* h_s shared expert hidden size (0: none) */
} moe_shape;

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,   /* NULL required pointer, NULL shape, bad scalar */
  MOE_ERR_UNSUPPORTED_SHAPE = 2,  /* shape outside the limits above */
  MOE_ERR_MISALIGNED = 3,         /* a vector-loaded pointer not 16-byte aligned */
  MOE_ERR_WORKSPACE_TOO_SMALL = 4,
  MOE_ERR_HIP = 5                 /* a HIP launch failed */
} moe_status;

/* Static, human-readable name of a status code. */
const char* moe_status_str(moe_status status);

/* Checks a shape against the limits above. */
moe_status moe_check_shape(const moe_shape* shape);

/* Device workspace every call below needs for this shape (the maximum over
 * the calls), a multiple of 256 bytes.  *bytes is written on success. */
moe_status moe_workspace_bytes(const moe_shape* shape, size_t* bytes);

/* Router ([Blog] §2.2.2: routing probabilities p_{t,e}, top-K set S_t, mask
 * s_{t,e}; [Digest]: loss-free balancing by a bias adjustment).
 *   z[t,e]    = sum_i x[t,i] * w_router[e,i]  (+ logit_bias[e])
 *   s[t,e]    = 1 / (1 + exp(-z[t,e]))
 *   beta[t,e] = s[t,e] + sel_bias[e]                 (selection only)
 *   S_t       = the k largest beta[t,.], ties to the lower expert index
 * In:  x [T,d] bf16; w_router [E,d] bf16; sel_bias [E] f32;
 *      logit_bias [E] f32 or NULL (a per-expert additive logit term).
 * Out: topk_ids [T,k] int32, S_t in ascending expert order;
 *      topk_weights [T,k] f32, w = s / sum_{S_t} s, aligned with topk_ids;
 *      expert_counts [E] int32, |{t : e in S_t}| (overwritten, not added to);
 *      topk_gap [T] f32 or NULL: k-th minus (k+1)-th largest beta
 *      (+inf when k == E).
 * Math in f32 (bf16 products, f32 accumulation).                            */
moe_status moe_route(const moe_shape* shape, const uint16_t* x, const uint16_t* w_router, const float* sel_bias,
                     const float* logit_bias, int32_t* topk_ids, float* topk_weights, int32_t* expert_counts,
                     float* topk_gap, void* workspace, size_t ws_bytes, void* stream);

/* Pre-norm router: the zero-centred RMSNorm in front of the FFN sub-layer
 * ([Blog] §2.2, Figure 2 caption; the [Digest] notes the pre-norm placement)
 * fused with moe_route:
 *   x_out[t,i] = bf16(h[t,i] / sqrt(mean_i(h[t,:]^2) + eps) * (1 + gamma[i]))
 * then moe_route on x_out.  x_out is bit-identical to moe_rmsnorm's output
 * and the routing outputs to moe_route's on it; for batches that take the
 * router's LDS-staged kernel (>= 1024 tokens) the normalisation runs first
 * and the router reads x_out back, otherwise the router normalises h as it
 * loads it.
 * In:  h [T,d] bf16 (the residual stream); gamma [d] f32 or NULL (unit
 *      gain); eps >= 0 finite; w_router, sel_bias, logit_bias as moe_route.
 * Out: x_out [T,d] bf16 (the experts' input; must not alias h), and the
 *      outputs of moe_route.  The workspace rule is the one of every call.  */
moe_status moe_rmsnorm_route(const moe_shape* shape, const uint16_t* h, const float* gamma, float eps,
                             const uint16_t* w_router, const float* sel_bias, const float* logit_bias,
                             uint16_t* x_out, int32_t* topk_ids, float* topk_weights, int32_t* expert_counts,
                             float* topk_gap, void* workspace, size_t ws_bytes, void* stream);

/* moe_route plus routing statistics ([Blog] §2.2.2: routing probability
 * p_{t,e}, dispatch fraction f_e, their per-group sums and the EP-level
 * balance L_EP over G expert groups; §5.2.3: routing confidence, the
 * probability mass of the activated experts).  With the unbiased scores s:
 *   p_{t,e}  = s[t,e] / sum_e' s[t,e']       (normalised over all E experts)
 *   p_e      = (1/T) sum_t p_{t,e}            f_e = expert_counts[e] / (T k)
 *   L_EP     = G * sum_g (sum_{e in g} f_e) (sum_{e in g} p_e), the groups
 *              being ep_groups contiguous blocks of E / G experts
 *   Sigma_k  = (1/T) sum_t sum_{e in S_t} p_{t,e}
 * In/out: as moe_route, plus ep_groups (1 <= G <= E, E % G == 0, else
 * MOE_ERR_INVALID_ARGUMENT).
 * Out: p_e [E] f32, f_e [E] f32, summary [2] f32 = (L_EP, Sigma_k); all zero
 *      when T == 0.  Sums are formed in a fixed order (f32 per token, f64
 *      across tokens): the same inputs give the same bits.  The workspace
 *      rule is the one of every call.                                       */
moe_status moe_route_diag(const moe_shape* shape, const uint16_t* x, const uint16_t* w_router, const float* sel_bias,
                          const float* logit_bias, int32_t* topk_ids, float* topk_weights, int32_t* expert_counts,
                          float* topk_gap, int32_t ep_groups, float* p_e, float* f_e, float* summary,
                          void* workspace, size_t ws_bytes, void* stream);

/* Token-to-expert permutation: the gather/scatter order of the grouped
 * expert GEMMs ([Blog] §3.2.4: fused MoE gather/scatter with grouped GEMM).
 * Pair p = t*k + j is token t's j-th chosen expert.
 * In:  topk_ids [T,k] int32 (as moe_route writes them).
 * Out: expert_offsets [E+1] int32, exclusive prefix sum of the per-expert
 *      pair counts (expert_offsets[E] = T*k);
 *      perm_pairs [T*k] int32: row r of the permuted order holds pair
 *      perm_pairs[r]; rows are ordered by expert, then by token (stable);
 *      pair_pos [T*k] int32: inverse, pair_pos[perm_pairs[r]] = r.          */
moe_status moe_permute(const moe_shape* shape, const int32_t* topk_ids, int32_t* expert_offsets,
                       int32_t* perm_pairs, int32_t* pair_pos, void* workspace, size_t ws_bytes, void* stream);

/* Routed experts ([Digest] architecture table: E SwiGLU experts of hidden h;
 * activation-explosion cause 3: gate and up projection branches).  For every
 * permuted row r of expert e, with token t = perm_pairs[r] / k:
 *   hid[r,:]    = SiLU(W_g^e x[t]) * (W_u^e x[t]),  SiLU(v) = v / (1 + exp(-v))
 *   y_perm[r,:] = W_d^e hid[r,:]
 * In:  x [T,d] bf16; expert_offsets [E+1], perm_pairs [T*k] (moe_permute);
 *      w_gate_up [E, 2h, d] bf16 (rows 0..h-1 gate, h..2h-1 up);
 *      w_down [E, d, h] bf16.
 * Out: y_perm [T*k, d] bf16, unweighted expert outputs in permuted order.
 * Optionally the shared expert runs inside the same grouped launches (one
 * more group holding every token): pass ws_gate_up [2h_s, d], ws_down
 * [d, h_s] and y_shared [T,d] f32 together (all three or none; d_shared > 0),
 * with the result of moe_shared_swiglu.
 * hid is rounded to bf16 between the two GEMMs; accumulation is f32.        */
moe_status moe_expert_swiglu(const moe_shape* shape, const uint16_t* x, const int32_t* expert_offsets,
                             const int32_t* perm_pairs, const uint16_t* w_gate_up, const uint16_t* w_down,
                             const uint16_t* ws_gate_up, const uint16_t* ws_down, uint16_t* y_perm, float* y_shared,
                             void* workspace, size_t ws_bytes, void* stream);

/* moe_expert_swiglu for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, with no workspace argument.  Its
 * scratch ([work queue | hid | hid_shared]: 256 + T*k*h*2 + T*h_s*2 bytes,
 * each part rounded up to 256) lives in a static array of the library,
 * 32 MiB per GPU, held from the library's first use on a GPU until the
 * process ends (at the model's shape, h = h_s = 1280 and k = 8: up to 1,456
 * tokens).  A shape needing more returns MOE_ERR_WORKSPACE_TOO_SMALL and
 * enqueues nothing.  The call allocates nothing: the array's address on the
 * current device is looked up on the first call on that device (a failure
 * returns MOE_ERR_HIP).  Every call on one GPU shares that GPU's array:
 * calls that may overlap on one GPU (different streams, or host threads
 * without ordering) race and must be serialised by the caller; each call
 * clears what it needs cleared.  Other arguments, outputs and errors as
 * moe_expert_swiglu.                                                       */
moe_status moe_expert_swiglu_noalloc(const moe_shape* shape, const uint16_t* x, const int32_t* expert_offsets,
                                     const int32_t* perm_pairs, const uint16_t* w_gate_up, const uint16_t* w_down,
                                     const uint16_t* ws_gate_up, const uint16_t* ws_down, uint16_t* y_perm,
                                     float* y_shared, void* stream);

/* moe_expert_swiglu with activation clipping ([Blog] §4.1.3 and Figure 4:
 * clipping the activations, unlike the weights, keeps the largest expert
 * output norm bounded in the deepest MoE layers; the pages give no
 * threshold): every hidden activation, routed and shared, is clipped to
 * [-act_clamp, act_clamp] before its bf16 rounding,
 *   hid = min(max(SiLU(W_g x) * (W_u x), -act_clamp), act_clamp)
 * (the [Digest] places the sparse huge activations in the product of the
 * aligned gate and up branches).  act_clamp > 0 and finite, else
 * MOE_ERR_INVALID_ARGUMENT.  Other arguments as moe_expert_swiglu.        */
moe_status moe_expert_swiglu_clamped(const moe_shape* shape, const uint16_t* x, const int32_t* expert_offsets,
                                     const int32_t* perm_pairs, const uint16_t* w_gate_up, const uint16_t* w_down,
                                     const uint16_t* ws_gate_up, const uint16_t* ws_down, uint16_t* y_perm,
                                     float* y_shared, float act_clamp, void* workspace, size_t ws_bytes,
                                     void* stream);

/* moe_expert_swiglu on one contiguous share of the experts, as one GPU of
 * an expert-parallel group runs it ([Blog] §2.2: expert parallelism for
 * scalable deployment, §2.2.2: EP-group balance, §3.2: 8-way expert
 * parallelism; [Digest] inference-cost table: EP8 serving): the routed
 * groups are experts expert_begin .. expert_end-1 and nothing else (no
 * shared expert; call moe_shared_swiglu for it).
 * In:  x, expert_offsets [E+1] and perm_pairs as for moe_expert_swiglu (the
 *      whole routing; the share's pairs are rows expert_offsets[expert_begin]
 *      .. expert_offsets[expert_end]-1 of the permuted order);
 *      w_gate_up [E_l, 2h, d] and w_down [E_l, d, h] bf16, the share's
 *      E_l = expert_end - expert_begin experts only.
 * Out: y_perm [T*k, d] bf16: the share's rows, exactly as moe_expert_swiglu
 *      computes them (same kernels and reduction order); other rows are not
 *      written.
 * 0 <= expert_begin < expert_end <= E, else MOE_ERR_INVALID_ARGUMENT.  The
 * workspace rule is the one of every call.                                  */
moe_status moe_expert_swiglu_range(const moe_shape* shape, int32_t expert_begin, int32_t expert_end,
                                   const uint16_t* x, const int32_t* expert_offsets, const int32_t* perm_pairs,
                                   const uint16_t* w_gate_up, const uint16_t* w_down, uint16_t* y_perm,
                                   void* workspace, size_t ws_bytes, void* stream);

/* The two phases of moe_expert_swiglu, for callers that keep the hidden
 * activations themselves: hid [T*k, h] bf16 (permuted order) and, with the
 * shared expert, hid_shared [T, h_s] bf16.  Shared-expert pointers come as a
 * set (gate/up: ws_gate_up + hid_shared; down: hid_shared + ws_down +
 * y_shared), all given or all NULL.  The workspace holds the kernels' work
 * queue (the size rule is the one of every call).                          */
moe_status moe_expert_gate_up(const moe_shape* shape, const uint16_t* x, const int32_t* expert_offsets,
                              const int32_t* perm_pairs, const uint16_t* w_gate_up, const uint16_t* ws_gate_up,
                              uint16_t* hid, uint16_t* hid_shared, void* workspace, size_t ws_bytes, void* stream);
moe_status moe_expert_down(const moe_shape* shape, const int32_t* expert_offsets, const uint16_t* hid,
                           const uint16_t* hid_shared, const uint16_t* w_down, const uint16_t* ws_down,
                           uint16_t* y_perm, float* y_shared, void* workspace, size_t ws_bytes, void* stream);

/* Shared expert ([Blog] §2.2: one shared expert, always active):
 *   y_shared[t,:] = W_d^s (SiLU(W_g^s x[t]) * (W_u^s x[t]))
 * In:  x [T,d] bf16; ws_gate_up [2h_s, d] bf16; ws_down [d, h_s] bf16.
 * Out: y_shared [T,d] f32.  Requires d_shared > 0.                          */
moe_status moe_shared_swiglu(const moe_shape* shape, const uint16_t* x, const uint16_t* ws_gate_up,
                             const uint16_t* ws_down, float* y_shared, void* workspace, size_t ws_bytes,
                             void* stream);

/* Weighted scatter-combine ([Blog] §4.1.2: routed-expert aggregation needs
 * explicit scaling):
 *   y[t,:] = y_shared[t,:] + routed_scale * sum_{j<k} topk_weights[t,j] * y_perm[pair_pos[t*k+j],:]
 * summed over j in order (ascending expert id), in f32, stored as bf16.
 * In:  y_perm [T*k, d] bf16; pair_pos [T*k] int32; topk_weights [T,k] f32;
 *      y_shared [T,d] f32 or NULL (treated as zero); routed_scale finite.
 * Out: y [T,d] bf16.                                                        */
moe_status moe_combine(const moe_shape* shape, const uint16_t* y_perm, const int32_t* pair_pos,
                       const float* topk_weights, const float* y_shared, float routed_scale, uint16_t* y,
                       void* stream);

/* moe_combine with the pre-norm block's skip connection ([Blog] §2.2,
 * Figure 2 caption: the normalised sub-layer's output is added back to the
 * stream):
 *   y[t,:] = residual[t,:] + (y_shared[t,:] + routed_scale * sum_j w_j y_perm[..])
 * in f32, rounded once to bf16.  residual [T,d] bf16 (required, 16-byte
 * aligned; it may alias y: each element is read before it is written by the
 * same thread).  Other arguments as moe_combine.                           */
moe_status moe_combine_residual(const moe_shape* shape, const uint16_t* y_perm, const int32_t* pair_pos,
                                const float* topk_weights, const float* y_shared, float routed_scale,
                                const uint16_t* residual, uint16_t* y, void* stream);

/* moe_combine plus the per-expert activation RMS ([Blog] §4.1.2: monitor
 * per-expert activation norms; §4.1.3, Figure 4: maximum against median
 * expert output norm; [Digest] expert collapse: min-to-median ratio):
 *   expert_rms[e] = sqrt(mean of y_perm[r,i]^2 over the rows r of expert e
 *                   and all i), 0 for an expert with no rows;
 *   expert_rms[E] = the same over y_shared (0 when y_shared is NULL);
 *   rms_ratio     = (min_e, max_e) expert_rms[e] / median_e expert_rms[e]
 *                   over the routed experts with at least one row (median
 *                   of an even count: mean of the two middle values);
 *                   (0, 0) when there is none or the median is 0.
 * In/out: as moe_combine, plus expert_offsets [E+1] int32 (moe_permute's),
 * expert_rms [E+1] f32 out, rms_ratio [2] f32 out or NULL, and the
 * workspace (the rule of every call).  y is bit-identical to moe_combine's.  */
moe_status moe_combine_diag(const moe_shape* shape, const uint16_t* y_perm, const int32_t* pair_pos,
                            const float* topk_weights, const float* y_shared, float routed_scale, uint16_t* y,
                            const int32_t* expert_offsets, float* expert_rms, float* rms_ratio, void* workspace,
                            size_t ws_bytes, void* stream);

/* Dense SwiGLU FFN ([Digest] architecture table: dense FFN hidden size
 * 11,264; [Blog] §2.2, Figure 2 caption: the first three blocks and the MTP
 * heads use a dense FFN): up to 64 tokens with a hidden size of at least
 * 16 units per CU, by kernels in which each CU streams a fixed share of both
 * weight matrices; otherwise by the grouped expert kernels as one group of
 * all T tokens:
 *   y[t,:] = W_d (SiLU(W_g x[t]) * (W_u x[t]))
 * In:  x [T, d] bf16; w_gate_up [2H, d] bf16 (rows 0..H-1 gate, H..2H-1
 *      up); w_down [d, H] bf16.
 * Out: y [T, d] f32.  The hidden activation is rounded to bf16 between the
 *      two GEMMs; accumulation is f32.
 * Limits: 0 <= T <= 1048576; d, H in [64, 65536], multiples of 64
 * (MOE_ERR_UNSUPPORTED_SHAPE).  The workspace (256-byte aligned) holds the
 * hidden activations and, up to 256 tokens, the f32 partial sums of the
 * reductions split over several work items (added in a fixed order, so the
 * result is reproducible): moe_dense_workspace_bytes gives its size.       */
moe_status moe_dense_workspace_bytes(int32_t num_tokens, int32_t d_model, int32_t d_hidden, size_t* bytes);
moe_status moe_dense_swiglu(int32_t num_tokens, int32_t d_model, int32_t d_hidden, const uint16_t* x,
                            const uint16_t* w_gate_up, const uint16_t* w_down, float* y, void* workspace,
                            size_t ws_bytes, void* stream);

/* Zero-centred RMSNorm of bf16 rows ([Blog] §2.2, Figure 2 caption; the
 * [Digest] notes the pre-norm placement):
 *   out[t,i] = in[t,i] / sqrt(mean_i(in[t,:]^2) + eps) * (1 + gamma[i])
 * gamma [cols] f32 or NULL (unit gain).  in/out [rows, cols] bf16 (may not
 * alias).  cols % 8 == 0, 8 <= cols <= 65536, rows >= 0, eps >= 0.          */
moe_status moe_rmsnorm(int32_t rows, int32_t cols, const uint16_t* in, const float* gamma, float eps,
                       uint16_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBMOE_MOE_H_ */
