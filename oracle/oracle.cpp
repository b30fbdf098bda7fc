// CPU oracle for the paired-4:8 sparse NVFP4 MoE expert path.
//
// TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU
// baseline leg may load this library. The product path never calls it, and it shares no
// code, header or table with the HIP library.
//
// It is written to be read against the pages ("Hardware-Native Joint Sparse-Quantization
// for Trillion-Scale Mixture-of-Experts", arxiv 2610.02241, and the model card
// "Kimi-K2.5-P48NVFP4-MoESQ"): plain loops in the order the pages state each step.
// Where the method reaches a result with a plain definition (the grouped GEMM, the
// stable permutation, the combine), the oracle writes that definition out in double
// precision. The encodings (E2M1, E4M3, Eq. 5, pruning, pair-bitmask packing) follow
// their definitions step by step in the precision noted at each function.
//
// Readings of points the pages leave open are marked READING; the same list is kept
// with the design notes.
#include <stdint.h>
#include <string.h>
#include <math.h>
#include <vector>
#include <algorithm>

extern "C" {

// Status codes returned by the oracle (mirrors the meaning of the library's codes).
enum { ORC_OK = 0, ORC_ERR_ARG = -1, ORC_ERR_PATTERN = -4 };

// ---------------------------------------------------------------------------------------
// E2M1 value grid. Paper, Appendix A, Figure 3: the retained values lie on
// {0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6}. A 4-bit code is sign (bit 3) and a 3-bit
// magnitude index into that ordered grid (E2M1 = 1 sign, 2 exponent, 1 mantissa bit).
// ---------------------------------------------------------------------------------------
static const double kE2M1Mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_e2m1_decode(uint8_t code) {
  double m = kE2M1Mag[code & 7];
  return (code & 8) ? -m : m;
}

// Nearest-neighbour projection onto the grid (paper Eq. 3, Pi_G).
// READING: a value exactly between two grid points goes to the even code (codes
// 0, 2, 4, 6 = magnitudes 0, 1, 2, 4); magnitudes beyond 6 go to 6 (the nearest point);
// the sign bit is set only for a nonzero magnitude, so -0 is never produced.
uint8_t orc_e2m1_encode(float r) {
  double a = fabs((double)r);
  // beyond 6 the nearest grid point is 6; clamping first keeps the distances below exact even where
  // a - 4 and a - 6 would round to the same double (|r| past about 2^54)
  if (a > 6.0) a = 6.0;
  int best = 0;
  double bestd = INFINITY;
  for (int c = 0; c < 8; c++) {
    double d = fabs(a - kE2M1Mag[c]);
    if (d < bestd || (d == bestd && (c % 2) == 0)) {
      best = c;
      bestd = d;
    }
  }
  uint8_t code = (uint8_t)best;
  if (best != 0 && signbit(r)) code |= 8;
  return code;
}

// ---------------------------------------------------------------------------------------
// UE4M3 scale. Paper Section 3.4 (Eq. 5) names 448 as the largest E4M3 magnitude, which
// identifies the OCP "E4M3FN" encoding: bias 7, 3 mantissa bits, subnormals, no
// infinity, 0x7F = NaN. The block scale is unsigned (Appendix A, Figure 3 caption).
// ---------------------------------------------------------------------------------------
double orc_e4m3_decode(uint8_t code) {
  int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = (double)m * ldexp(1.0, -9);
  else v = (1.0 + (double)m / 8.0) * ldexp(1.0, e - 7);
  return s ? -v : v;
}

// Nearest finite non-negative E4M3 value to u >= 0.
// READING: round to nearest, ties to the even code; values above 448 give 448
// (saturation, the nearest finite point); never NaN.
uint8_t orc_e4m3_encode(float u) {
  double a = (double)u;
  if (!(a > 0.0)) return 0;
  // Codes 0x00..0x7E are the finite non-negative values in increasing order.
  int lo = 0, hi = 0x7E;
  if (a >= orc_e4m3_decode(0x7E)) return 0x7E;
  // find the smallest code whose value is >= a
  while (lo < hi) {
    int mid = (lo + hi) / 2;
    if (orc_e4m3_decode((uint8_t)mid) >= a) hi = mid; else lo = mid + 1;
  }
  int up = lo;
  if (up == 0) return 0;
  int dn = up - 1;
  double dup = orc_e4m3_decode((uint8_t)up) - a;
  double ddn = a - orc_e4m3_decode((uint8_t)dn);
  if (dup < ddn) return (uint8_t)up;
  if (ddn < dup) return (uint8_t)dn;
  return (uint8_t)((up % 2 == 0) ? up : dn);
}

// ---------------------------------------------------------------------------------------
// Two-level NVFP4 scaling, paper Section 3.4, Eq. 5:
//   gamma = 448 / (max_b ||Y_b||_inf / 6),   s_b = Pi_E4M3(gamma ||Y_b||_inf / 6) / gamma,
// and Eq. 3: Q(Y)_b = s_b * Pi_G(Y_b / s_b).
// READING (precision and order): IEEE fp32, no fused multiply-add, in exactly this order:
//   t = amax / 6; gamma = 448 / t                      (tensor scale)
//   t = gamma * amax_b; u = t / 6; code = E4M3(u)      (block scale code)
//   s = E4M3value(code) / gamma; q = E2M1(x / s)       (element code; s == 0 -> q = 0)
// READING: an all-zero tensor gets gamma = 1.
// ---------------------------------------------------------------------------------------
float orc_global_scale(float amax) {
  if (!(amax > 0.0f)) return 1.0f;
  volatile float t = amax / 6.0f;
  volatile float g = 448.0f / t;
  return g;
}

// Amax over a float array (exact: max is order independent).
float orc_amax(const float* x, int64_t n) {
  float m = 0.0f;
  for (int64_t i = 0; i < n; i++) {
    float a = fabsf(x[i]);
    if (a > m) m = a;
  }
  return m;
}

// Quantize one block of 32 consecutive values with tensor scale gamma.
// codes[i/2] holds element i in its low nibble (even i) or high nibble (odd i).
static void quantize_block32(const float* x, float gamma, uint8_t* codes16, uint8_t* scale_code) {
  float amax = 0.0f;
  for (int i = 0; i < 32; i++) {
    float a = fabsf(x[i]);
    if (a > amax) amax = a;
  }
  volatile float t = gamma * amax;
  volatile float u = t / 6.0f;
  uint8_t sc = orc_e4m3_encode(u);
  volatile float s = (float)orc_e4m3_decode(sc) / gamma;
  for (int i = 0; i < 16; i++) codes16[i] = 0;
  for (int i = 0; i < 32; i++) {
    uint8_t q = 0;
    if (s != 0.0f) {
      volatile float r = x[i] / s;
      q = orc_e2m1_encode(r);
    }
    codes16[i / 2] |= (i % 2 == 0) ? q : (uint8_t)(q << 4);
  }
  *scale_code = sc;
}

// Quantize rows of a row-major [R][C] float tensor (C % 32 == 0), blocks along C.
// Row r uses gamma[row_group[r]] if row_group is given, else gamma[0].
// q: [R][C/2] (two codes per byte, low nibble = lower column), s: [R][C/32] E4M3 codes.
int orc_quantize_rows(const float* x, int64_t R, int32_t C, int64_t ld, const float* gamma,
                      const int32_t* row_group, uint8_t* q, uint8_t* s) {
  if (C % 32 != 0 || R < 0) return ORC_ERR_ARG;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < R; r++) {
    float g = gamma[row_group ? row_group[r] : 0];
    for (int32_t b = 0; b < C / 32; b++)
      quantize_block32(x + r * ld + 32 * b, g, q + r * (C / 2) + 16 * b, s + r * (C / 32) + b);
  }
  return ORC_OK;
}

// ---------------------------------------------------------------------------------------
// Paired-4:8 sparsity, paper Section 3.2 (m = 8, P = 6) and Appendix A (Eq. 6): every
// group of 8 consecutive K elements keeps two of its four adjacent pairs
// (elements 2i, 2i+1 form pair i).
// Pruning rule for synthetic weights (not on the pages; the workload recipe): keep the two
// pairs with the largest L2 norm, norms in double; on equal norms the lower pair index
// wins.
// ---------------------------------------------------------------------------------------
void orc_prune_paired48(const float* w, int64_t rows, int32_t K, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; r++) {
    for (int32_t g = 0; g < K / 8; g++) {
      const float* x = w + r * K + 8 * g;
      float* y = out + r * K + 8 * g;
      double nrm[4];
      for (int i = 0; i < 4; i++) nrm[i] = (double)x[2 * i] * x[2 * i] + (double)x[2 * i + 1] * x[2 * i + 1];
      int first = 0;
      for (int i = 1; i < 4; i++)
        if (nrm[i] > nrm[first]) first = i;
      int second = -1;
      for (int i = 0; i < 4; i++) {
        if (i == first) continue;
        if (second < 0 || nrm[i] > nrm[second]) second = i;
      }
      for (int i = 0; i < 4; i++) {
        bool keep = (i == first || i == second);
        y[2 * i] = keep ? x[2 * i] : 0.0f;
        y[2 * i + 1] = keep ? x[2 * i + 1] : 0.0f;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// Pair-bitmask v1 storage, model card "Sparse storage layout (paired48_sparse,
// pair-bitmask v1)": dense NVFP4 holds two adjacent K elements per byte (one pair per
// byte), so a paired-4:8 row has exactly two nonzero bytes in every 4-byte chunk.
//   packed [rows][K/4]: the two kept bytes of every chunk, in K order;
//   mask   [rows][K/16]: 4 bits per chunk, bit i set = byte i kept, exactly two set,
//          low nibble = lower-K chunk;
// a chunk with fewer than two nonzero bytes marks its lowest-index zero bytes as kept.
// READING: in a dense byte the lower-K element is the low nibble.
// ---------------------------------------------------------------------------------------
int orc_pack_pair_bitmask(const uint8_t* dense, int64_t rows, int32_t K, uint8_t* packed, uint8_t* mask) {
  if (K % 16 != 0) return ORC_ERR_ARG;
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t r = 0; r < rows; r++) {
    for (int32_t c = 0; c < K / 8; c++) {
      const uint8_t* b = dense + r * (K / 2) + 4 * c;
      int nib = 0, cnt = 0;
      for (int i = 0; i < 4; i++)
        if (b[i] != 0) { nib |= 1 << i; cnt++; }
      if (cnt > 2) { bad = 1; nib = 0; cnt = 0; }
      for (int i = 0; i < 4 && cnt < 2; i++)
        if (!(nib & (1 << i))) { nib |= 1 << i; cnt++; }
      int o = 0;
      for (int i = 0; i < 4; i++)
        if (nib & (1 << i)) packed[r * (K / 4) + 2 * c + (o++)] = b[i];
      uint8_t* m = mask + r * (K / 16) + c / 2;
      if (c % 2 == 0) *m = (uint8_t)nib; else *m = (uint8_t)(*m | (nib << 4));
    }
  }
  return bad ? ORC_ERR_PATTERN : ORC_OK;
}

int orc_unpack_pair_bitmask(const uint8_t* packed, const uint8_t* mask, int64_t rows, int32_t K, uint8_t* dense) {
  if (K % 16 != 0) return ORC_ERR_ARG;
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t r = 0; r < rows; r++) {
    for (int32_t c = 0; c < K / 8; c++) {
      uint8_t mb = mask[r * (K / 16) + c / 2];
      int nib = (c % 2 == 0) ? (mb & 15) : (mb >> 4);
      uint8_t* b = dense + r * (K / 2) + 4 * c;
      int cnt = 0;
      for (int i = 0; i < 4; i++) cnt += (nib >> i) & 1;
      if (cnt != 2) bad = 1;
      int o = 0;
      for (int i = 0; i < 4; i++) b[i] = (nib & (1 << i)) && o < 2 ? packed[r * (K / 4) + 2 * c + (o++)] : 0;
    }
  }
  return bad ? ORC_ERR_PATTERN : ORC_OK;
}

// Dense NVFP4 bytes from per-element codes: byte j of a row = code(2j) | code(2j+1) << 4.
// (The per-element codes are already stored two per byte in that order, so the dense
// layout is the code array itself; kept as a named step for readability.)

// ---------------------------------------------------------------------------------------
// Weight compression for one projection of E experts (setup step; paper Section 3.4 last
// paragraph and Appendix A): prune to paired-4:8, compute the tensor scale per expert from
// the pruned weights (Eq. 5), quantize 32-element blocks along K (Eq. 3 + 5), write
// dense NVFP4 bytes, then store them as pair-bitmask v1.
// w: [E][N][K] fp32. Outputs: packed [E][N][K/4], mask [E][N][K/16], scale [E][N][K/32],
// gscale [E] (gamma of Eq. 5; dequantized weight = e2m1 * e4m3 / gamma).
// ---------------------------------------------------------------------------------------
int orc_compress_weights(const float* w, int32_t E, int32_t N, int32_t K, uint8_t* packed, uint8_t* mask,
                         uint8_t* scale, float* gscale) {
  if (K % 32 != 0 || E <= 0 || N <= 0) return ORC_ERR_ARG;
  const int64_t per = (int64_t)N * K;
  std::vector<float> pruned(per);
  std::vector<uint8_t> dense(per / 2);
  int rc_all = ORC_OK;
  for (int32_t e = 0; e < E; e++) {
    orc_prune_paired48(w + e * per, N, K, pruned.data());
    float g = orc_global_scale(orc_amax(pruned.data(), per));
    gscale[e] = g;
    orc_quantize_rows(pruned.data(), N, K, K, &g, nullptr, dense.data(), scale + e * (per / 32));
    int rc = orc_pack_pair_bitmask(dense.data(), N, K, packed + e * (per / 4), mask + e * (per / 16));
    if (rc != ORC_OK) rc_all = rc;
  }
  return rc_all;
}

// ---------------------------------------------------------------------------------------
// Routing / permutation (paper Appendix D.1: routing, dispatch planning and token
// combination are the shared MoE steps; token counts stay on the device).
// The permutation is a stable sort of the flat slots f = t*k + j by expert id.
// READING: inside one expert the slots keep ascending f order.
// counts [E], offsets [E+1] (exclusive prefix sum), sorted_slot [T*k], slot_pos [T*k]
// (slot_pos[sorted_slot[p]] = p). Ids outside [0, E) are an argument error.
// ---------------------------------------------------------------------------------------
int orc_route(const int32_t* ids, int64_t T, int32_t k, int32_t E, int32_t* counts, int32_t* offsets,
              int32_t* sorted_slot, int32_t* slot_pos) {
  const int64_t n = T * k;
  for (int32_t e = 0; e < E; e++) counts[e] = 0;
  for (int64_t f = 0; f < n; f++) {
    if (ids[f] < 0 || ids[f] >= E) return ORC_ERR_ARG;
    counts[ids[f]]++;
  }
  offsets[0] = 0;
  for (int32_t e = 0; e < E; e++) offsets[e + 1] = offsets[e] + counts[e];
  std::vector<int32_t> fill(offsets, offsets + E);
  for (int64_t f = 0; f < n; f++) {
    int32_t p = fill[ids[f]]++;
    sorted_slot[p] = (int32_t)f;
    slot_pos[f] = p;
  }
  return ORC_OK;
}

// Expert owning permuted row p (offsets[e] <= p < offsets[e+1]).
static int32_t expert_of_row(const int32_t* offsets, int32_t E, int64_t p) {
  for (int32_t e = 0; e < E; e++)
    if (p >= offsets[e] && p < offsets[e + 1]) return e;
  return -1;
}

// Dispatch + activation quantization (Appendix D.1: activations are quantized at run time
// into 32-element blocks, fused with token dispatch): permuted row p is token
// sorted_slot[p] / k quantized with the tensor scale of its expert (model card: the
// activation tensor scale is stored per expert linear).
int orc_dispatch_quantize(const float* x, int64_t T, int32_t K, const int32_t* sorted_slot, int32_t k,
                          const int32_t* offsets, int32_t E, const float* gamma, uint8_t* q, uint8_t* s) {
  if (K % 32 != 0) return ORC_ERR_ARG;
  const int64_t rows = offsets[E];
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t p = 0; p < rows; p++) {
    int64_t t = sorted_slot[p] / k;
    int32_t e = expert_of_row(offsets, E, p);
    if (t < 0 || t >= T || e < 0) { bad = 1; continue; }
    float g = gamma[e];
    for (int32_t b = 0; b < K / 32; b++)
      quantize_block32(x + t * (int64_t)K + 32 * b, g, q + p * (K / 2) + 16 * b, s + p * (K / 32) + b);
  }
  return bad ? ORC_ERR_ARG : ORC_OK;
}

// ---------------------------------------------------------------------------------------
// Dequantization (exact in double): value = E2M1(code) * E4M3(block scale).
// Weights: the pair-bitmask row is expanded to dense bytes first.
// ---------------------------------------------------------------------------------------
void orc_dequant_codes(const uint8_t* q, const uint8_t* s, int64_t R, int32_t C, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < R; r++)
    for (int32_t c = 0; c < C; c++) {
      uint8_t byte = q[r * (C / 2) + c / 2];
      uint8_t code = (c % 2 == 0) ? (byte & 15) : (byte >> 4);
      out[r * C + c] = orc_e2m1_decode(code) * orc_e4m3_decode(s[r * (C / 32) + c / 32]);
    }
}

// ---------------------------------------------------------------------------------------
// Grouped GEMM (paper Section 2 and Section 3.4: Y_e = X_e W_e^T for every expert, with
// the per-expert factor alpha_e = 1 / (gamma_w,e * gamma_a,e) applied to the accumulated
// products of the block-scaled operands). Computed in double on fully dequantized operands.
// Only the permuted rows listed in row_list are evaluated: y[i][n] for row row_list[i].
// ---------------------------------------------------------------------------------------
int orc_grouped_gemm(const uint8_t* packed, const uint8_t* mask, const uint8_t* wscale, const float* gscale_w,
                     int32_t E, int32_t N, int32_t K, const uint8_t* q, const uint8_t* s, const float* gamma_a,
                     const int32_t* offsets, const int64_t* row_list, int64_t n_list, double* y) {
  if (K % 32 != 0) return ORC_ERR_ARG;
  const int64_t per = (int64_t)N * K;
  std::vector<uint8_t> dense(per / 2);
  std::vector<double> wd(per);
  std::vector<double> xd(K);
  for (int32_t e = 0; e < E; e++) {
    bool any = false;
    for (int64_t i = 0; i < n_list && !any; i++)
      if (row_list[i] >= offsets[e] && row_list[i] < offsets[e + 1]) any = true;
    if (!any) continue;
    int rc = orc_unpack_pair_bitmask(packed + e * (per / 4), mask + e * (per / 16), N, K, dense.data());
    if (rc != ORC_OK) return rc;
    orc_dequant_codes(dense.data(), wscale + e * (per / 32), N, K, wd.data());
    const double denom = (double)gscale_w[e] * (double)gamma_a[e];
    for (int64_t i = 0; i < n_list; i++) {
      int64_t p = row_list[i];
      if (p < offsets[e] || p >= offsets[e + 1]) continue;
      orc_dequant_codes(q + p * (K / 2), s + p * (K / 32), 1, K, xd.data());
#pragma omp parallel for schedule(static)
      for (int32_t n = 0; n < N; n++) {
        double acc = 0.0;
        const double* wr = wd.data() + (int64_t)n * K;
        for (int32_t kk = 0; kk < K; kk++) acc += wr[kk] * xd[kk];
        y[i * N + n] = acc / denom;
      }
    }
  }
  return ORC_OK;
}

// SwiGLU on a gate_up output row set (model card: gate_proj, up_proj, down_proj per expert;
// paper Appendix D.1: fused SwiGLU before the second GEMM). READING: the first I columns
// are the gate, the next I the up projection; SiLU(g) = g / (1 + exp(-g)).
void orc_swiglu(const double* y13, int64_t R, int32_t I, double* h) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < R; r++)
    for (int32_t i = 0; i < I; i++) {
      double g = y13[r * 2 * I + i], u = y13[r * 2 * I + I + i];
      h[r * I + i] = g / (1.0 + exp(-g)) * u;
    }
}

// Router-weighted combine (Appendix D.1 "token combination"): for every token t,
// out[t] = sum over j = 0..k-1 of w[t][j] * y[slot_pos[t*k + j]], in j order, double.
void orc_combine(const double* y, int32_t H, const int32_t* slot_pos, const float* w, int64_t T, int32_t k,
                 double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; t++)
    for (int32_t c = 0; c < H; c++) {
      double acc = 0.0;
      for (int32_t j = 0; j < k; j++) acc += (double)w[t * k + j] * y[(int64_t)slot_pos[t * k + j] * H + c];
      out[t * H + c] = acc;
    }
}

}  // extern "C"
