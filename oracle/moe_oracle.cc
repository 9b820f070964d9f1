// moe_oracle.cc -- plain, slow CPU oracle for the forward pass of one
// fine-grained sparse MoE FFN layer (Step 3.5 Flash shape).
//
// TEST INFRASTRUCTURE ONLY.  Only the test-suite, the package's smoke check
// and the benchmark's CPU-baseline leg may load or call this library.  The GPU
// library never links, loads or calls it, and it shares no code with the GPU
// library (its own bf16 decoding, its own loops, its own sort).
//
// Pages cited (by title):
//   [Blog]    "Step 3.5 Flash: Open Frontier-Level Intelligence with 11B Active
//             Parameters" (section-numbered summary of the paper)
//   [Digest]  "Step 3.5 Flash 技术论文深度解读：196B MoE 如何做到 11B 激活打 37B"
//   [Article] "StepFun团队Step 3.5 Flash：11B参数实现前沿智能水平"
//
// What it computes, and where the pages say so:
//   * each MoE layer has E routed experts plus one always-on shared expert and
//     activates the top-k routed experts per token ([Blog] §2.2; [Digest]
//     architecture table: 288 routed + 1 shared, top-8, routed hidden 1,280);
//   * routing: per-token routing probabilities p_{t,e}, the top-K set S_t and
//     its mask s_{t,e} ([Blog] §2.2.2, EP-balance formulas); balance comes
//     from a bias adjustment rather than an auxiliary loss ([Digest] note
//     under the architecture table; [Article] §9), read here as a bias added
//     to the scores for selection only;
//   * experts are SwiGLU FFNs with gate and up projection branches ([Digest]
//     local-activation-explosion root cause 3);
//   * routed-expert aggregation is explicitly scaled ([Blog] §4.1.2), exposed
//     as a scalar routed_scale.
// The pages leave the gate nonlinearity, tie rule and weight normalisation
// open; this oracle takes: sigmoid scores s = sigma(z), biased scores
// beta = s + b used only to pick the set, ties toward the lower expert index,
// weights w = s / sum_{S_t} s from the unbiased scores, ids reported in
// ascending expert order, and y = y_shared + routed_scale * sum_j w_j o_j
// summed in ascending expert order.
//
// Precision: inputs are bf16 values (decoded exactly to float).  Every dot
// product is accumulated in double and rounded to float once per output
// element; every other intermediate (scores, SwiGLU activations, weights) is
// computed in double from float operands and rounded to float once.  The
// selection itself compares float values beta = fl32(s + b), the precision the
// GPU path decides in.
//
// Everything runs on the calling thread.  Functions return 0 on success and a
// negative code on a bad argument.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <limits>
#include <vector>

namespace {

float bf16_value(uint16_t v) {
  const uint32_t bits = (uint32_t)v << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return f;
}

uint16_t to_bf16_nearest_even(float f) {
  uint32_t bits;
  memcpy(&bits, &f, sizeof bits);
  if (std::isnan(f)) return (uint16_t)((bits >> 16) | 0x40);
  const uint32_t lsb = (bits >> 16) & 1u;
  bits += 0x7FFFu + lsb;
  return (uint16_t)(bits >> 16);
}

// sum_i a[i] * b[i] over bf16 vectors, accumulated in double, rounded once.
float dot_bf16(const uint16_t* a, const uint16_t* b, int n) {
  double acc = 0.0;
  for (int i = 0; i < n; ++i) acc += (double)bf16_value(a[i]) * (double)bf16_value(b[i]);
  return (float)acc;
}

double sigmoid(double v) { return 1.0 / (1.0 + std::exp(-v)); }

// Routing of one token row.  Writes k ids (ascending), k weights, the gap
// between the k-th and (k+1)-th biased score, and optionally all E scores.
void route_token(int d, int E, int k, const uint16_t* x_row, const uint16_t* w_router, const float* sel_bias,
                 const float* logit_bias, int32_t* ids, float* weights, float* gap, float* scores) {
  std::vector<float> s(E), beta(E);
  for (int e = 0; e < E; ++e) {
    float z = dot_bf16(x_row, w_router + (size_t)e * d, d);
    if (logit_bias) z = z + logit_bias[e];
    s[e] = (float)sigmoid((double)z);
    beta[e] = s[e] + sel_bias[e];
    if (scores) scores[e] = s[e];
  }
  // Experts ordered by biased score, highest first; equal scores keep the
  // lower expert index first (stable sort of an ascending index list).
  std::vector<int> order(E);
  for (int e = 0; e < E; ++e) order[e] = e;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return beta[a] > beta[b]; });
  if (gap) {
    *gap = (k < E) ? (float)((double)beta[order[k - 1]] - (double)beta[order[k]])
                   : std::numeric_limits<float>::infinity();
  }
  std::vector<int> chosen(order.begin(), order.begin() + k);
  std::sort(chosen.begin(), chosen.end());
  double total = 0.0;
  for (int j = 0; j < k; ++j) total += (double)s[chosen[j]];
  for (int j = 0; j < k; ++j) {
    ids[j] = chosen[j];
    weights[j] = (float)((double)s[chosen[j]] / total);
  }
}

// One SwiGLU expert on one token: out = W_d (SiLU(W_g x) * (W_u x)).
// w_gu is [2h, d] (rows 0..h-1 gate, h..2h-1 up), w_d is [d, h].
// clamp > 0: each hidden activation is clipped to [-clamp, clamp] (activation
// clipping, [Blog] §4.1.3 and Figure 4; placed on the SwiGLU product, where
// the [Digest] locates the sparse huge activations of aligned gate and up
// branches).
void swiglu_token(int d, int h, const uint16_t* x_row, const uint16_t* w_gu, const uint16_t* w_d, float* out,
                  double clamp = 0.0) {
  std::vector<float> act(h);
  for (int j = 0; j < h; ++j) {
    const float g = dot_bf16(w_gu + (size_t)j * d, x_row, d);
    const float u = dot_bf16(w_gu + (size_t)(h + j) * d, x_row, d);
    double a = (double)g * sigmoid((double)g) * (double)u;
    if (clamp > 0.0) a = std::min(std::max(a, -clamp), clamp);
    act[j] = (float)a;
  }
  for (int i = 0; i < d; ++i) {
    double acc = 0.0;
    const uint16_t* row = w_d + (size_t)i * h;
    for (int j = 0; j < h; ++j) acc += (double)bf16_value(row[j]) * (double)act[j];
    out[i] = (float)acc;
  }
}

bool shape_ok(int T, int d, int E, int k) { return T >= 0 && d > 0 && E > 0 && k >= 1 && k <= E; }

// Steps after the selection for one token whose chosen set is given: the
// weights from the unbiased scores of the chosen experts ([Blog] §2.2.2: the
// mask s_{t,e} of the top-K set), the chosen SwiGLU experts, the shared
// expert, and the scaled sum in ascending expert order ([Blog] §4.1.2).
//   ids [k]      the chosen set, ascending, distinct, in [0, E)
//   wts [k]      out: w_e = s_e / sum_{S_t} s
//   y   [d]      out (f32)
// Returns -3 if a chosen expert has no weights.
int forward_token_given_set(int d, int E, int k, int h, int hs, const uint16_t* xr, const uint16_t* w_router,
                            const float* logit_bias, const int32_t* ids, const uint16_t* const* w_gu,
                            const uint16_t* const* w_d, const uint16_t* ws_gu, const uint16_t* ws_d,
                            float routed_scale, float* wts, float* y) {
  std::vector<float> s(k), shared(d), expert_out((size_t)k * d);
  double total = 0.0;
  for (int j = 0; j < k; ++j) {
    const int e = ids[j];
    float z = dot_bf16(xr, w_router + (size_t)e * d, d);
    if (logit_bias) z = z + logit_bias[e];
    s[j] = (float)sigmoid((double)z);
    total += (double)s[j];
  }
  for (int j = 0; j < k; ++j) wts[j] = (float)((double)s[j] / total);
  for (int j = 0; j < k; ++j) {
    if (!w_gu[ids[j]] || !w_d[ids[j]]) return -3;
    swiglu_token(d, h, xr, w_gu[ids[j]], w_d[ids[j]], expert_out.data() + (size_t)j * d);
  }
  if (hs > 0) swiglu_token(d, hs, xr, ws_gu, ws_d, shared.data());
  for (int i = 0; i < d; ++i) {
    double routed = 0.0;
    for (int j = 0; j < k; ++j) routed += (double)wts[j] * (double)expert_out[(size_t)j * d + i];
    const double base = hs > 0 ? (double)shared[i] : 0.0;
    y[i] = (float)(base + (double)routed_scale * routed);
  }
  return 0;
}

bool set_ok(int E, int k, const int32_t* ids) {
  for (int j = 0; j < k; ++j) {
    if (ids[j] < 0 || ids[j] >= E) return false;
    if (j > 0 && ids[j] <= ids[j - 1]) return false;
  }
  return true;
}

}  // namespace

extern "C" {


// Router for all T tokens.  x [T,d] bf16, w_router [E,d] bf16, sel_bias [E]
// f32, logit_bias [E] f32 or NULL.  Outputs topk_ids [T,k] (ascending),
// topk_weights [T,k], topk_gap [T] (NULL allowed), scores [T,E] (NULL allowed).
int oracle_route(int T, int d, int E, int k, const uint16_t* x, const uint16_t* w_router, const float* sel_bias,
                 const float* logit_bias, int32_t* topk_ids, float* topk_weights, float* topk_gap, float* scores) {
  if (!shape_ok(T, d, E, k) || !x || !w_router || !sel_bias || !topk_ids || !topk_weights) return -1;
  for (int t = 0; t < T; ++t)
    route_token(d, E, k, x + (size_t)t * d, w_router, sel_bias, logit_bias, topk_ids + (size_t)t * k,
                topk_weights + (size_t)t * k, topk_gap ? topk_gap + t : nullptr,
                scores ? scores + (size_t)t * E : nullptr);
  return 0;
}

// Token-to-expert permutation from the routing ids [T,k].
//   counts[e]        number of (token, slot) pairs routed to e
//   offsets[e]       exclusive prefix sum of counts, offsets[E] = T*k
//   perm_pairs[r]    pair index t*k+j of the r-th row, rows ordered by
//                    expert, then token (stable counting sort)
//   pair_pos[t*k+j]  inverse of perm_pairs
int oracle_permute(int T, int E, int k, const int32_t* topk_ids, int32_t* counts, int32_t* offsets,
                   int32_t* perm_pairs, int32_t* pair_pos) {
  if (T < 0 || E <= 0 || k < 1 || !topk_ids || !counts || !offsets || !perm_pairs || !pair_pos) return -1;
  const int64_t P = (int64_t)T * k;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t p = 0; p < P; ++p) {
    const int e = topk_ids[p];
    if (e < 0 || e >= E) return -2;
    counts[e] += 1;
  }
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int64_t row = 0;
  for (int e = 0; e < E; ++e)
    for (int t = 0; t < T; ++t)
      for (int j = 0; j < k; ++j)
        if (topk_ids[(size_t)t * k + j] == e) perm_pairs[row++] = t * k + j;
  for (int64_t r = 0; r < P; ++r) pair_pos[perm_pairs[r]] = (int32_t)r;
  return 0;
}

// One SwiGLU expert applied to one bf16 token row; out [d] f32.
int oracle_expert(int d, int h, const uint16_t* x_row, const uint16_t* w_gu, const uint16_t* w_d, float* out) {
  if (d <= 0 || h <= 0 || !x_row || !w_gu || !w_d || !out) return -1;
  swiglu_token(d, h, x_row, w_gu, w_d, out);
  return 0;
}

// oracle_expert with the hidden activations clipped to [-clamp, clamp]
// (clamp > 0).
int oracle_expert_clamped(int d, int h, const uint16_t* x_row, const uint16_t* w_gu, const uint16_t* w_d,
                          double clamp, float* out) {
  if (d <= 0 || h <= 0 || !x_row || !w_gu || !w_d || !out || !(clamp > 0.0)) return -1;
  swiglu_token(d, h, x_row, w_gu, w_d, out, clamp);
  return 0;
}

// Whole layer for a list of token rows.
//   w_gu[e], w_d[e]  expert e's weights ([2h,d] and [d,h] bf16); an entry may
//                    be NULL only if no listed token selects expert e
//   ws_gu, ws_d      shared expert ([2hs,d], [d,hs]); ignored when hs == 0
//   tokens           n_tok row indices into x (NULL: rows 0..n_tok-1)
// Outputs per listed token: topk_ids [n,k], topk_weights [n,k], topk_gap [n]
// (each NULL allowed) and y [n,d] f32.  Returns -3 if a selected expert has
// no weights.
int oracle_layer(int T, int d, int E, int k, int h, int hs, const uint16_t* x, const uint16_t* w_router,
                 const float* sel_bias, const float* logit_bias, const uint16_t* const* w_gu,
                 const uint16_t* const* w_d, const uint16_t* ws_gu, const uint16_t* ws_d, float routed_scale,
                 int n_tok, const int32_t* tokens, int32_t* topk_ids, float* topk_weights, float* topk_gap,
                 float* y) {
  if (!shape_ok(T, d, E, k) || h <= 0 || hs < 0 || n_tok < 0 || !x || !w_router || !sel_bias || !w_gu || !w_d ||
      !y)
    return -1;
  if (hs > 0 && (!ws_gu || !ws_d)) return -1;
  std::vector<int32_t> ids(k);
  std::vector<float> wts(k), wts_route(k);
  for (int n = 0; n < n_tok; ++n) {
    const int t = tokens ? tokens[n] : n;
    if (t < 0 || t >= T) return -2;
    const uint16_t* xr = x + (size_t)t * d;
    float gap = 0.f;
    route_token(d, E, k, xr, w_router, sel_bias, logit_bias, ids.data(), wts_route.data(), &gap, nullptr);
    const int rc = forward_token_given_set(d, E, k, h, hs, xr, w_router, logit_bias, ids.data(), w_gu, w_d, ws_gu,
                                           ws_d, routed_scale, wts.data(), y + (size_t)n * d);
    if (rc != 0) return rc;
    if (topk_ids) memcpy(topk_ids + (size_t)n * k, ids.data(), sizeof(int32_t) * k);
    if (topk_weights) memcpy(topk_weights + (size_t)n * k, wts.data(), sizeof(float) * k);
    if (topk_gap) topk_gap[n] = gap;
  }
  return 0;
}

// The layer for listed tokens under a given routing: every step after the
// selection (weights, experts, shared expert, scaled combine) on the chosen
// sets passed in, instead of the sets this oracle's own selection would
// pick.  Output comparisons "given the same routing" use it where two sets
// are both correct (a near-tie between the k-th and (k+1)-th biased score).
//   ids [n_tok, k]   each row ascending, distinct, in [0, E) (else -4)
//   tokens           n_tok row indices into x (NULL: rows 0..n_tok-1)
// Outputs: topk_weights [n,k] (NULL allowed) and y [n,d] f32.  Other
// arguments as oracle_layer (no selection bias: it does not enter).
int oracle_forward_given_routing(int T, int d, int E, int k, int h, int hs, const uint16_t* x,
                                 const uint16_t* w_router, const float* logit_bias, const uint16_t* const* w_gu,
                                 const uint16_t* const* w_d, const uint16_t* ws_gu, const uint16_t* ws_d,
                                 float routed_scale, int n_tok, const int32_t* tokens, const int32_t* ids,
                                 float* topk_weights, float* y) {
  if (!shape_ok(T, d, E, k) || h <= 0 || hs < 0 || n_tok < 0 || !x || !w_router || !w_gu || !w_d || !ids || !y)
    return -1;
  if (hs > 0 && (!ws_gu || !ws_d)) return -1;
  std::vector<float> wts(k);
  for (int n = 0; n < n_tok; ++n) {
    const int t = tokens ? tokens[n] : n;
    if (t < 0 || t >= T) return -2;
    const int32_t* set = ids + (size_t)n * k;
    if (!set_ok(E, k, set)) return -4;
    const int rc = forward_token_given_set(d, E, k, h, hs, x + (size_t)t * d, w_router, logit_bias, set, w_gu, w_d,
                                           ws_gu, ws_d, routed_scale, wts.data(), y + (size_t)n * d);
    if (rc != 0) return rc;
    if (topk_weights) memcpy(topk_weights + (size_t)n * k, wts.data(), sizeof(float) * k);
  }
  return 0;
}

// Weighted combine on its own ([Blog] §4.1.2, explicit scaling of the
// routed aggregation): y[t,i] = y_shared[t,i] + routed_scale *
// sum_{j<k} weights[t,j] * y_perm[pair_pos[t*k+j], i], with y_perm bf16 rows,
// y_shared f32 or NULL (zero), everything summed in double, y f32.
// residual [T,d] bf16 or NULL: the pre-norm block's skip connection ([Blog]
// §2.2, Figure 2 caption: zero-centred RMSNorm in front of each sub-layer,
// whose output is added back to the stream), summed with the FFN output
// before the single rounding.
int oracle_combine(int T, int d, int k, const uint16_t* y_perm, const int32_t* pair_pos, const float* weights,
                   const float* y_shared, float routed_scale, const uint16_t* residual, float* y) {
  if (T < 0 || d <= 0 || k < 1 || !y_perm || !pair_pos || !weights || !y) return -1;
  for (int t = 0; t < T; ++t) {
    for (int i = 0; i < d; ++i) {
      double routed = 0.0;
      for (int j = 0; j < k; ++j) {
        const int64_t row = pair_pos[(size_t)t * k + j];
        routed += (double)weights[(size_t)t * k + j] * (double)bf16_value(y_perm[(size_t)row * d + i]);
      }
      const double base = y_shared ? (double)y_shared[(size_t)t * d + i] : 0.0;
      const double skip = residual ? (double)bf16_value(residual[(size_t)t * d + i]) : 0.0;
      y[(size_t)t * d + i] = (float)(skip + (base + (double)routed_scale * routed));
    }
  }
  return 0;
}

// Routing diagnostics ([Blog] §2.2.2, EP-level load balance: p_e, f_e, their
// group sums p_g, f_g and L_EP = G * sum_g f_g p_g over G disjoint expert
// groups; §5.2.3, routing confidence: the mean probability mass of the
// activated experts).  Readings: the routing probability p_{t,e} of a sigmoid
// router is the token's unbiased scores normalised over all E experts (so
// that sum_e p_e = 1 and L_EP is 1 under uniform routing, as the loss
// intends); the G groups are contiguous blocks of E/G experts (expert
// parallelism placing consecutive experts on one rank).
//   scores [T,E]  unbiased sigmoid scores s_{t,e} (oracle_route's output)
//   topk_ids [T,k] the chosen set S_t
//   p_e [E], f_e [E], l_ep, confidence: outputs (double)
// f_e = |{t : e in S_t}| / (T k).  T = 0 gives zeros.
int oracle_route_diag(int T, int E, int k, int G, const float* scores, const int32_t* topk_ids, double* p_e,
                      double* f_e, double* l_ep, double* confidence) {
  if (T < 0 || E <= 0 || k < 1 || k > E || G < 1 || E % G != 0 || !p_e || !f_e || !l_ep || !confidence) return -1;
  if (T > 0 && (!scores || !topk_ids)) return -1;
  for (int e = 0; e < E; ++e) p_e[e] = f_e[e] = 0.0;
  double mass = 0.0;
  std::vector<double> p(E);
  for (int t = 0; t < T; ++t) {
    double total = 0.0;
    for (int e = 0; e < E; ++e) total += (double)scores[(size_t)t * E + e];
    for (int e = 0; e < E; ++e) {
      p[e] = (double)scores[(size_t)t * E + e] / total;
      p_e[e] += p[e];
    }
    for (int j = 0; j < k; ++j) {
      const int e = topk_ids[(size_t)t * k + j];
      if (e < 0 || e >= E) return -2;
      f_e[e] += 1.0;
      mass += p[e];
    }
  }
  *l_ep = 0.0;
  *confidence = 0.0;
  if (T == 0) return 0;
  for (int e = 0; e < E; ++e) {
    p_e[e] /= (double)T;
    f_e[e] /= (double)T * k;
  }
  const int per = E / G;
  for (int g = 0; g < G; ++g) {
    double pg = 0.0, fg = 0.0;
    for (int e = g * per; e < (g + 1) * per; ++e) {
      pg += p_e[e];
      fg += f_e[e];
    }
    *l_ep += fg * pg;
  }
  *l_ep *= G;
  *confidence = mass / T;
  return 0;
}

// Root mean square of one expert's activations ([Blog] §4.1.2, per-expert
// activation norms as an expert-collapse signal; [Digest] expert collapse:
// monitor each expert's activation RMS against the median): the expert's
// output rows o_{t,e} [n, d] (f32) -> sqrt(mean of o^2), 0 for n = 0.
int oracle_activation_rms(int n, int d, const float* rows, double* rms) {
  if (n < 0 || d <= 0 || !rms || (n > 0 && !rows)) return -1;
  double ss = 0.0;
  for (int64_t i = 0; i < (int64_t)n * d; ++i) ss += (double)rows[i] * (double)rows[i];
  *rms = n > 0 ? std::sqrt(ss / ((double)n * d)) : 0.0;
  return 0;
}

// Zero-centred RMSNorm (pre-norm placement, [Blog] §2.2, Figure 2 caption): each
// row v -> v / sqrt(mean(v^2) + eps) * (1 + gamma), gamma NULL meaning 0 (unit
// gain).  in [T,d] bf16 -> out [T,d] bf16 (round to nearest even).
int oracle_rmsnorm(int T, int d, const uint16_t* in, const float* gamma, float eps, uint16_t* out) {
  if (T < 0 || d <= 0 || !in || !out) return -1;
  for (int t = 0; t < T; ++t) {
    double ss = 0.0;
    for (int i = 0; i < d; ++i) {
      const double v = bf16_value(in[(size_t)t * d + i]);
      ss += v * v;
    }
    const double inv = 1.0 / std::sqrt(ss / d + (double)eps);
    for (int i = 0; i < d; ++i) {
      const double g = gamma ? 1.0 + (double)gamma[i] : 1.0;
      out[(size_t)t * d + i] = to_bf16_nearest_even((float)((double)bf16_value(in[(size_t)t * d + i]) * inv * g));
    }
  }
  return 0;
}

}  // extern "C"
