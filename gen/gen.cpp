// Seeded synthetic inputs for tests and benchmarks (host build).
// Holds no arithmetic of the MoE method: random tensors, router ids and router weights only.
#include <stdint.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <vector>
#include <algorithm>
#include "gen_math.h"

extern "C" {

// out[i] = (float)(scale * N(0,1) number (start + i) of (seed, stream)).
void gen_fill_normal(uint64_t seed, uint64_t stream, uint64_t start, int64_t n, double scale, float* out) {
  const uint64_t key = gen_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) out[i] = (float)(scale * gen_normal(key, start + (uint64_t)i));
}

// out[i] = (float)(scale * Student-t(nu) number (start + i) of (seed, stream)).
void gen_fill_student_t(uint64_t seed, uint64_t stream, uint64_t start, int64_t n, int32_t nu, double scale,
                        float* out) {
  const uint64_t key = gen_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) out[i] = (float)(scale * gen_student_t(key, start + (uint64_t)i, nu));
}

// out[i] = uniform (0,1) number (start + i), as double.
void gen_fill_uniform(uint64_t seed, uint64_t stream, uint64_t start, int64_t n, double* out) {
  const uint64_t key = gen_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; i++) out[i] = gen_uniform(key, start + (uint64_t)i);
}

// Top-k of one token's scores (descending, ties to the lower expert id), then router
// weights = softmax over the k selected scores (double, stored as float).
static void topk_softmax(const double* score, const unsigned char* allowed, int32_t E, int32_t k, int32_t* ids,
                         float* w) {
  std::vector<int32_t> order;
  order.reserve(E);
  for (int32_t e = 0; e < E; e++)
    if (allowed == nullptr || allowed[e]) order.push_back(e);
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return score[a] > score[b]; });
  double mx = score[order[0]];
  double den = 0.0;
  for (int32_t j = 0; j < k; j++) den += exp(score[order[j]] - mx);
  for (int32_t j = 0; j < k; j++) {
    ids[j] = order[j];
    w[j] = (float)(exp(score[order[j]] - mx) / den);
  }
}

#define GEN_STREAM_ROUTER_LOGITS (3ull << 48)
#define GEN_STREAM_ZIPF_PERM (4ull << 48)
#define GEN_STREAM_GUMBEL (5ull << 48)

// Uniform routing: logits U(0,1) per (token, expert), top-k, softmax router weights.
// Returns 0, or -1 if k is not in [1, E].
int gen_route_uniform(uint64_t seed, int64_t T, int32_t E, int32_t k, int32_t* ids, float* w) {
  if (k < 1 || k > E) return -1;
  const uint64_t key = gen_key(seed, GEN_STREAM_ROUTER_LOGITS);
#pragma omp parallel
  {
    std::vector<double> sc(E);
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; t++) {
      for (int32_t e = 0; e < E; e++) sc[e] = gen_uniform(key, (uint64_t)t * (uint64_t)E + (uint64_t)e);
      topk_softmax(sc.data(), nullptr, E, k, ids + t * k, w + t * k);
    }
  }
  return 0;
}

// Zipf(s) expert popularity: rank r (1-based) has weight r^-s; ranks map to experts by a
// seeded Fisher-Yates permutation; the n_zero least popular ranks get weight 0 (never
// chosen). Each token draws k distinct experts by Gumbel-top-k on log-popularity
// (sampling without replacement); router weights = softmax over the selected perturbed
// scores. Returns 0, or -1 if k exceeds the number of allowed experts.
int gen_route_zipf(uint64_t seed, int64_t T, int32_t E, int32_t k, double s, int32_t n_zero, int32_t* ids,
                   float* w) {
  if (k < 1 || k > E - n_zero || n_zero < 0) return -1;
  std::vector<int32_t> perm(E);
  for (int32_t e = 0; e < E; e++) perm[e] = e;
  const uint64_t pkey = gen_key(seed, GEN_STREAM_ZIPF_PERM);
  for (int32_t i = E - 1; i > 0; i--) {
    int32_t j = (int32_t)(gen_uniform(pkey, (uint64_t)i) * (double)(i + 1));
    if (j > i) j = i;
    std::swap(perm[i], perm[j]);
  }
  std::vector<double> logpop(E);
  std::vector<unsigned char> allowed(E, 1);
  for (int32_t r = 0; r < E; r++) {
    int32_t e = perm[r];
    logpop[e] = -s * gen_ln((double)(r + 1));
    if (r >= E - n_zero) allowed[e] = 0;
  }
  const uint64_t gkey = gen_key(seed, GEN_STREAM_GUMBEL);
#pragma omp parallel
  {
    std::vector<double> sc(E);
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; t++) {
      for (int32_t e = 0; e < E; e++) {
        double u = gen_uniform(gkey, (uint64_t)t * (uint64_t)E + (uint64_t)e);
        sc[e] = logpop[e] - gen_ln(-gen_ln(u));
      }
      topk_softmax(sc.data(), allowed.data(), E, k, ids + t * k, w + t * k);
    }
  }
  return 0;
}

}  // extern "C"
