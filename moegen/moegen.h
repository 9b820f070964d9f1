// moegen.h -- seeded, counter-based input generator for the sparse MoE FFN
// layer's synthetic workloads.
//
// This module only draws numbers.  It holds none of the layer's arithmetic
// (no router, no SwiGLU, no combine).  It is the one piece of code that both
// the CPU oracle's tests and the GPU benchmark use, so that both see the same
// bf16 inputs.
//
// Definition (so the host and device fills agree bit for bit):
//   * Stream:   SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
//               number generators", OOPSLA 2014).  Output i of a stream with
//               initial state s is mix64(s + (i+1) * 0x9E3779B97F4A7C15).
//   * Key:      a tensor's stream state is derived from
//               (seed, layer, tensor kind, expert) by chaining mix64.
//   * Normal:   Box-Muller (1958) on the two 32-bit halves of one output:
//               u1 = (hi + 0.5) / 2^32, u2 = lo / 2^32,
//               z  = sqrt(-2 ln u1) * cos(2 pi u2).
//               ln, cos and sqrt are evaluated below with +, -, * only
//               (table + short series, Newton for 1/sqrt), with FP
//               contraction disabled, so every IEEE-754 double unit gives the
//               same bits.  Their accuracy (~1e-15 relative) is far below what
//               survives the final rounding to bf16.
//   * Rounding: double -> float (IEEE round-to-nearest-even), then
//               float -> bf16 round-to-nearest-even on the bit pattern.
//
// Compiled only by hipcc (host and device code of the same functions).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define MG_HD __host__ __device__ __forceinline__

namespace moegen {

static constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;

MG_HD uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// i-th output (0-based) of the SplitMix64 sequence started from `state`.
MG_HD uint64_t splitmix(uint64_t state, uint64_t i) { return mix64(state + (i + 1) * kGolden); }

// Stream state for one tensor.
MG_HD uint64_t stream_key(uint64_t seed, uint64_t layer, uint64_t kind, uint64_t expert) {
  uint64_t k = splitmix(seed, 0);
  k = splitmix(k ^ (layer + 1), 0);
  k = splitmix(k ^ (kind + 1), 0);
  k = splitmix(k ^ (expert + 1), 0);
  return k;
}

MG_HD double bits_to_double(uint64_t b) { return __builtin_bit_cast(double, b); }
MG_HD uint64_t double_to_bits(double d) { return __builtin_bit_cast(uint64_t, d); }

// ln(1 + (j + 0.5)/32) and its reciprocal argument, j = 0..31, rounded to double.
struct LogEntry { double inv_c, ln_c; };

MG_HD double mg_log(double x) {
#pragma clang fp contract(off)
  // x in (0, 1]: x = m * 2^e, m in [1, 2).
  static constexpr LogEntry kTab[32] = {
      {0.9846153846153847, 0.015504186535965254}, {0.9552238805970149, 0.0458095360312942},
      {0.927536231884058, 0.07522342123758753},   {0.9014084507042254, 0.10379679368164356},
      {0.8767123287671232, 0.13157635778871926},  {0.8533333333333334, 0.15860503017663857},
      {0.8311688311688312, 0.184922338494012},    {0.810126582278481, 0.21056476910734964},
      {0.7901234567901234, 0.2355660713127669},   {0.7710843373493976, 0.25995752443692605},
      {0.7529411764705882, 0.2837681731306446},   {0.735632183908046, 0.3070250352949119},
      {0.7191011235955056, 0.329753286372468},    {0.7032967032967034, 0.3519764231571782},
      {0.6881720430107527, 0.37371640979358406},  {0.6736842105263158, 0.394993808240869},
      {0.6597938144329897, 0.415827895143711},    {0.6464646464646465, 0.43623676677491807},
      {0.6336633663366337, 0.4562374334815876},   {0.6213592233009708, 0.4758459048699639},
      {0.6095238095238096, 0.4950772667978515},   {0.5981308411214953, 0.5139457511022343},
      {0.5871559633027523, 0.5324647988694718},   {0.5765765765765766, 0.5506471179526623},
      {0.5663716814159292, 0.5685047353526688},   {0.5565217391304348, 0.5860490450035782},
      {0.5470085470085471, 0.6032908514380843},   {0.5378151260504201, 0.6202404097518576},
      {0.5289256198347108, 0.6369074622370692},   {0.5203252032520326, 0.6533012720127457},
      {0.512, 0.6694306539426292},                {0.5039370078740157, 0.6853040030989194}};
  const uint64_t b = double_to_bits(x);
  const int e = (int)((b >> 52) & 0x7ff) - 1023;
  const double m = bits_to_double((b & 0x000FFFFFFFFFFFFFull) | 0x3FF0000000000000ull);
  const int j = (int)((b >> 47) & 31);  // top 5 mantissa bits
  const double r = m * kTab[j].inv_c - 1.0;  // |r| < 1/64
  // ln(1 + r) = r - r^2/2 + r^3/3 - ... (Horner, 9 terms)
  double p = 1.0 / 9.0;
  p = 1.0 / 8.0 - r * p;
  p = 1.0 / 7.0 - r * p;
  p = 1.0 / 6.0 - r * p;
  p = 1.0 / 5.0 - r * p;
  p = 1.0 / 4.0 - r * p;
  p = 1.0 / 3.0 - r * p;
  p = 1.0 / 2.0 - r * p;
  p = 1.0 - r * p;
  const double ln2 = 0.6931471805599453;
  return (double)e * ln2 + kTab[j].ln_c + r * p;
}

// sin and cos of t in [0, pi/4] by their Taylor series (to t^17 / t^16).
MG_HD double mg_sin_small(double t) {
#pragma clang fp contract(off)
  const double t2 = t * t;
  double p = 1.0 / 355687428096000.0;    // 1/17!
  p = -1.0 / 1307674368000.0 + t2 * p;   // -1/15!
  p = 1.0 / 6227020800.0 + t2 * p;       // 1/13!
  p = -1.0 / 39916800.0 + t2 * p;        // -1/11!
  p = 1.0 / 362880.0 + t2 * p;           // 1/9!
  p = -1.0 / 5040.0 + t2 * p;            // -1/7!
  p = 1.0 / 120.0 + t2 * p;              // 1/5!
  p = -1.0 / 6.0 + t2 * p;               // -1/3!
  p = 1.0 + t2 * p;
  return t * p;
}
MG_HD double mg_cos_small(double t) {
#pragma clang fp contract(off)
  const double t2 = t * t;
  double p = 1.0 / 20922789888000.0;     // 1/16!
  p = -1.0 / 87178291200.0 + t2 * p;     // -1/14!
  p = 1.0 / 479001600.0 + t2 * p;        // 1/12!
  p = -1.0 / 3628800.0 + t2 * p;         // -1/10!
  p = 1.0 / 40320.0 + t2 * p;            // 1/8!
  p = -1.0 / 720.0 + t2 * p;             // -1/6!
  p = 1.0 / 24.0 + t2 * p;               // 1/4!
  p = -0.5 + t2 * p;                     // -1/2!
  p = 1.0 + t2 * p;
  return p;
}

// cos(2 pi * lo / 2^32) for a 32-bit lo, by octant reduction.
MG_HD double mg_cos_2pi_u32(uint32_t lo) {
#pragma clang fp contract(off)
  const uint32_t oct = lo >> 29;
  const double f = (double)(lo & 0x1FFFFFFFu) * (1.0 / 536870912.0);  // [0,1), exact
  const double g = 1.0 - f;                                             // exact
  const double q = 0.7853981633974483;                                  // pi/4
  switch (oct) {
    case 0: return mg_cos_small(f * q);
    case 1: return mg_sin_small(g * q);
    case 2: return -mg_sin_small(f * q);
    case 3: return -mg_cos_small(g * q);
    case 4: return -mg_cos_small(f * q);
    case 5: return -mg_sin_small(g * q);
    case 6: return mg_sin_small(f * q);
    default: return mg_cos_small(g * q);
  }
}

// sqrt(a) for a > 0 via Newton iterations on 1/sqrt(a).
MG_HD double mg_sqrt(double a) {
#pragma clang fp contract(off)
  double y = bits_to_double(0x5FE6EB50C7B537A9ull - (double_to_bits(a) >> 1));
  for (int it = 0; it < 6; ++it) y = y * (1.5 - 0.5 * a * y * y);
  return a * y;
}

// Standard normal from one 64-bit SplitMix64 output.
MG_HD double normal_from_u64(uint64_t u) {
#pragma clang fp contract(off)
  const uint32_t hi = (uint32_t)(u >> 32);
  const uint32_t lo = (uint32_t)u;
  const double u1 = ((double)hi + 0.5) * (1.0 / 4294967296.0);  // (0,1), exact
  const double r = mg_sqrt(-2.0 * mg_log(u1));
  return r * mg_cos_2pi_u32(lo);
}

// Uniform [0,1) with 53 bits from one output.
MG_HD double uniform_from_u64(uint64_t u) { return (double)(u >> 11) * (1.0 / 9007199254740992.0); }

MG_HD uint16_t f32_to_bf16_rne(float f) {
  uint32_t b = __builtin_bit_cast(uint32_t, f);
  if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x007FFFFFu)) return (uint16_t)((b >> 16) | 0x40);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

// Element i of a N(0, std^2) tensor stored as bf16.
MG_HD uint16_t normal_bf16(uint64_t key, uint64_t i, double stdev) {
#pragma clang fp contract(off)
  const double z = normal_from_u64(splitmix(key, i)) * stdev;
  return f32_to_bf16_rne((float)z);
}

}  // namespace moegen
