// Seeded synthetic-input generator: shared arithmetic for the host build (g++)
// and the device build (hipcc). Nothing here belongs to the MoE method; it only
// draws random numbers.
//
// Every function uses IEEE double add, subtract, multiply and divide only (no
// library transcendental, no fused multiply-add: both builds use
// -ffp-contract=off), so the host and the device produce bit-identical values.
//
// Random bits: the splitmix64 sequence (Steele, Lea, Flood, "Fast splittable
// pseudorandom number generators", OOPSLA 2014): state_i = key + (i+1)*golden,
// output = mix64(state_i). The key is derived from (seed, stream) the same way.
#pragma once
#include <stdint.h>

#ifdef __HIPCC__
#define GEN_HD __host__ __device__ inline
#else
#define GEN_HD static inline
#endif

#define GEN_GOLDEN 0x9E3779B97F4A7C15ull

GEN_HD uint64_t gen_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

GEN_HD uint64_t gen_key(uint64_t seed, uint64_t stream) {
  return gen_mix64(seed * GEN_GOLDEN + stream * 0xD1B54A32D192ED03ull + 1ull);
}

GEN_HD uint64_t gen_bits(uint64_t key, uint64_t i) { return gen_mix64(key + (i + 1ull) * GEN_GOLDEN); }

// Uniform in the open interval (0, 1): ((bits >> 11) + 0.5) * 2^-53.
GEN_HD double gen_uniform(uint64_t key, uint64_t i) {
  return ((double)(gen_bits(key, i) >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

GEN_HD double gen_as_double(uint64_t b) {
  union { uint64_t u; double d; } v; v.u = b; return v.d;
}
GEN_HD uint64_t gen_as_bits(double d) {
  union { uint64_t u; double d; } v; v.d = d; return v.u;
}

// Natural log for a positive normal double: x = m * 2^e with m in [sqrt(1/2), sqrt(2)),
// ln(m) = 2*atanh(s), s = (m-1)/(m+1), |s| <= 0.172, series to s^25.
GEN_HD double gen_ln(double x) {
  uint64_t b = gen_as_bits(x);
  int e = (int)((b >> 52) & 0x7FF) - 1023;
  double m = gen_as_double((b & 0x000FFFFFFFFFFFFFull) | 0x3FF0000000000000ull);
  if (m > 1.4142135623730951) { m = m * 0.5; e = e + 1; }
  double s = (m - 1.0) / (m + 1.0);
  double s2 = s * s;
  double p = 0.04;                      // 1/25
  p = 0.043478260869565216 + s2 * p;    // 1/23
  p = 0.047619047619047616 + s2 * p;    // 1/21
  p = 0.05263157894736842 + s2 * p;     // 1/19
  p = 0.058823529411764705 + s2 * p;    // 1/17
  p = 0.06666666666666667 + s2 * p;     // 1/15
  p = 0.07692307692307693 + s2 * p;     // 1/13
  p = 0.09090909090909091 + s2 * p;     // 1/11
  p = 0.1111111111111111 + s2 * p;      // 1/9
  p = 0.14285714285714285 + s2 * p;     // 1/7
  p = 0.2 + s2 * p;                     // 1/5
  p = 0.3333333333333333 + s2 * p;      // 1/3
  p = 1.0 + s2 * p;                     // 1/1
  return (double)e * 0.6931471805599453 + 2.0 * s * p;
}

// Square root of y > 0 by Newton's iteration from an exponent-halved first guess.
GEN_HD double gen_sqrt(double y) {
  uint64_t b = gen_as_bits(y);
  double g = gen_as_double((b >> 1) + 0x1FF8000000000000ull);
  for (int it = 0; it < 7; it++) g = 0.5 * (g + y / g);
  return g;
}

// sin and cos of x in [0, pi/2) by Taylor series to x^25 / x^24.
GEN_HD void gen_sincos_quarter(double x, double* s, double* c) {
  double x2 = x * x;
  double cs = 1.6117375710961184e-24;          // 1/24!
  cs = -8.896791392450574e-22 + x2 * cs;       // 1/22!
  cs = 4.110317623312165e-19 + x2 * cs;        // 1/20!
  cs = -1.5619206968586225e-16 + x2 * cs;      // 1/18!
  cs = 4.779477332387385e-14 + x2 * cs;        // 1/16!
  cs = -1.1470745597729725e-11 + x2 * cs;      // 1/14!
  cs = 2.08767569878681e-09 + x2 * cs;         // 1/12!
  cs = -2.755731922398589e-07 + x2 * cs;       // 1/10!
  cs = 2.48015873015873e-05 + x2 * cs;         // 1/8!
  cs = -0.001388888888888889 + x2 * cs;        // 1/6!
  cs = 0.041666666666666664 + x2 * cs;         // 1/4!
  cs = -0.5 + x2 * cs;                         // 1/2!
  cs = 1.0 + x2 * cs;
  double sn = 6.446950284384474e-26;           // 1/25!
  sn = -3.868170170630684e-23 + x2 * sn;       // 1/23!
  sn = 1.9572941063391263e-20 + x2 * sn;       // 1/21!
  sn = -8.22063524662433e-18 + x2 * sn;        // 1/19!
  sn = 2.8114572543455206e-15 + x2 * sn;       // 1/17!
  sn = -7.647163731819816e-13 + x2 * sn;       // 1/15!
  sn = 1.6059043836821613e-10 + x2 * sn;       // 1/13!
  sn = -2.505210838544172e-08 + x2 * sn;       // 1/11!
  sn = 2.7557319223985893e-06 + x2 * sn;       // 1/9!
  sn = -0.0001984126984126984 + x2 * sn;       // 1/7!
  sn = 0.008333333333333333 + x2 * sn;         // 1/5!
  sn = -0.16666666666666666 + x2 * sn;         // 1/3!
  sn = 1.0 + x2 * sn;
  *s = x * sn;
  *c = cs;
}

// sin(2*pi*v), cos(2*pi*v) for v in [0, 1), reduced by quadrant.
GEN_HD void gen_sincos_turn(double v, double* s, double* c) {
  double t = v * 4.0;
  int q = (int)t;
  if (q > 3) q = 3;
  double x = (t - (double)q) * 1.5707963267948966;
  double sx, cx;
  gen_sincos_quarter(x, &sx, &cx);
  if (q == 0) { *s = sx; *c = cx; }
  else if (q == 1) { *s = cx; *c = -sx; }
  else if (q == 2) { *s = -sx; *c = -cx; }
  else { *s = -cx; *c = sx; }
}

// Standard normal number i of a stream: Box-Muller on the uniform pair (2p, 2p+1),
// p = i/2; even i takes the cosine branch, odd i the sine branch.
GEN_HD double gen_normal(uint64_t key, uint64_t i) {
  uint64_t p = i >> 1;
  double u1 = gen_uniform(key, 2 * p);
  double u2 = gen_uniform(key, 2 * p + 1);
  double r = gen_sqrt(-2.0 * gen_ln(u1));
  double s, c;
  gen_sincos_turn(u2, &s, &c);
  return (i & 1) ? r * s : r * c;
}

// Student-t with integer nu: z0 / sqrt((z1^2 + ... + z_nu^2) / nu), normals
// (nu+1)*i .. (nu+1)*i + nu of the stream.
GEN_HD double gen_student_t(uint64_t key, uint64_t i, int nu) {
  uint64_t base = (uint64_t)(nu + 1) * i;
  double z0 = gen_normal(key, base);
  double ss = 0.0;
  for (int j = 1; j <= nu; j++) {
    double z = gen_normal(key, base + (uint64_t)j);
    ss = ss + z * z;
  }
  return z0 / gen_sqrt(ss / (double)nu);
}
