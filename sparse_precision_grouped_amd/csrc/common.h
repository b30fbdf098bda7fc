// Device helpers for the gfx950 kernels: vector types, the E2M1 / UE4M3 codecs, the Eq. 5
// block quantizer, and the operand decoders that feed the sparse MFMA.
//
// Paper: "Hardware-Native Joint Sparse-Quantization for Trillion-Scale Mixture-of-Experts"
// (Section 3.4, Eq. 5; Appendix A, Figure 3). Model card: "Kimi-K2.5-P48NVFP4-MoESQ" (storage).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moesq.h"

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define MOESQ_DEV __device__ __forceinline__

// ---------------------------------------------------------------- codecs -----------------------
// E2M1 code of r: nearest point of {0, .5, 1, 1.5, 2, 3, 4, 6} in magnitude, ties to the even
// code, saturating at 6, sign bit only for a nonzero magnitude. The magnitude index equals the
// number of decision thresholds |r| has passed; a threshold between an odd and an even code is
// inclusive toward the even one.
MOESQ_DEV uint32_t e2m1_encode(float r) {
  const float a = __builtin_fabsf(r);
  uint32_t m = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) + (uint32_t)(a >= 1.75f) +
               (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
  const uint32_t neg = (__float_as_uint(r) >> 31) & (m != 0u);
  return m | (neg << 3);
}

// UE4M3 (E4M3 with bias 7, largest finite 448) code of u >= 0: round to nearest even on the fp32
// bit pattern for normal results, on the 2^-9 grid for subnormal ones; >= 448 saturates to 0x7E.
MOESQ_DEV uint32_t e4m3_encode(float u) {
  if (!(u > 0.0f)) return 0u;
  if (u >= 448.0f) return 0x7Eu;
  if (u < 0.015625f) return (uint32_t)__builtin_rintf(u * 512.0f);  // m * 2^-9, m in 0..8
  const uint32_t b = __float_as_uint(u);
  const uint32_t r = b + 0x7FFFFu + ((b >> 20) & 1u);
  const uint32_t code = (r >> 20) - (120u << 3);
  return code > 0x7Eu ? 0x7Eu : code;
}

// Value of a UE4M3 code as fp32 (exact).
MOESQ_DEV float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  if (e == 0u) return (float)m * 0.001953125f;
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// Eq. 5 tensor scale gamma = 448 / (amax / 6) in fp32 (1 for an all-zero tensor).
MOESQ_DEV float global_scale_from_amax(float amax) {
  if (!(amax > 0.0f)) return 1.0f;
  const float t = amax / 6.0f;
  return 448.0f / t;
}

// E2M1 codes of the correctly rounded quotients x[i] / s (element i in nibble i), given r = RN(1/s),
// with no full division per element: q0 = RN(x r), e = x - s q0 (exact by fma), RN(q0 + e r) is
// RN(x / s) (Markstein) unless e underflows, which needs |x / s| < 2^-90, where every quotient encodes
// to 0 anyway. The hardware FP4 convert rounds to nearest, ties to the even code, and saturates at 6,
// as E2M1 does (checked on every fp32 value in [-8, 8]), except that it gives -0 (code 8) where E2M1
// gives +0: the last mask clears those sign bits. The caller keeps |x r| far below the fp32 range.
MOESQ_DEV float quot_rn(float x, float s, float r) {
  const float q0 = x * r;
  return __builtin_fmaf(__builtin_fmaf(-s, q0, x), r, q0);
}
MOESQ_DEV uint32_t e2m1_codes4(float x0, float x1, float x2, float x3, float s, float r) {
  uint32_t c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, quot_rn(x0, s, r), quot_rn(x1, s, r), 1.0f, 0);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, quot_rn(x2, s, r), quot_rn(x3, s, r), 1.0f, 1) & 0xFFFFu;
  return c & ((((c & 0x7777u) + 0x7777u) & 0x8888u) | 0x7777u);
}
MOESQ_DEV uint32_t e2m1_codes8(const float x[8], float s, float r) {
  uint32_t c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, quot_rn(x[0], s, r), quot_rn(x[1], s, r), 1.0f, 0);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, quot_rn(x[2], s, r), quot_rn(x[3], s, r), 1.0f, 1);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, quot_rn(x[4], s, r), quot_rn(x[5], s, r), 1.0f, 2);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, quot_rn(x[6], s, r), quot_rn(x[7], s, r), 1.0f, 3);
  return c & ((((c & 0x77777777u) + 0x77777777u) & 0x88888888u) | 0x77777777u);
}

// Quantize 8 consecutive values held by one lane; four consecutive lanes (lane % 4 = 0..3) form one
// 32-element block. Returns the 8 E2M1 codes (element i in nibble i) and the block's UE4M3 code.
// Eq. 5 order in fp32: t = gamma*amax; u = t/6; code = E4M3(u); s = value(code)/gamma; q = E2M1(x/s).
MOESQ_DEV void quant8_block4(const float v[8], float gamma, uint32_t& codes, uint32_t& scode) {
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i++) am = __builtin_fmaxf(am, __builtin_fabsf(v[i]));
  am = __builtin_fmaxf(am, __shfl_xor(am, 1));
  am = __builtin_fmaxf(am, __shfl_xor(am, 2));
  const float t = gamma * am;
  const float u = t / 6.0f;
  scode = e4m3_encode(u);
  const float s = e4m3_value(scode) / gamma;
  codes = 0u;
  if (s != 0.0f) {
    const float r = 1.0f / s;
    if (am * r < 1e30f) {
      codes = e2m1_codes8(v, s, r);
    } else {  // a huge or non-finite block: the plain division and encoder
#pragma unroll
      for (int i = 0; i < 8; i++) codes |= e2m1_encode(v[i] / s) << (4 * i);
    }
  }
}

// ------------------------------------------------ sparse-MFMA operand decoding -------------------
// The kernels use v_smfmac_f32_16x16x64_f16 (2:4 structured-sparse A). Its lane layout on gfx950:
//   A (sparse, 8 stored f16 per lane): lane l holds row l%16 and covers the 16 K positions
//     [16*(l/16), +16) as four 4-groups; stored values 2g, 2g+1 belong to 4-group g and sit at the
//     positions named by 2-bit indices in bits [4g, 4g+4) of the 16-bit index operand.
//   B (dense, 16 f16 per lane): lane l holds column l%16, K = 8*(l/16) + j for j < 8 and
//     K = 32 + 8*(l/16) + (j - 8) for j >= 8.
//   D: lane l holds rows 4*(l/16) + r (r = 0..3) of column l%16.
// Paired 4:8 becomes 2:4 by de-interleaving every 8-group: the even elements (0,2,4,6) form one
// 4-group and the odd elements (1,3,5,7) the next. A group that keeps pairs i < j then has exactly
// two nonzeros at positions i and j in both 4-groups, for all six patterns.

// Two E2M1 codes in byte `sel` of w -> two f16 (low nibble first), unscaled.
#define MOESQ_CVT_FP4(w, sel) __builtin_amdgcn_cvt_scalef32_pk_f16_fp4((w), 1.0f, (sel))

MOESQ_DEV uint32_t f16x2_bits(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }
MOESQ_DEV f16x2 bits_f16x2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }

// Two UE4M3 codes in the low 16 bits of w (hi: the high 16 bits) -> (v0, v0) and (v1, v1) as f16x2
// (exact: the gfx950 FP8 convert with unit scale, on the bytes duplicated by a perm). Selecting the
// half in the perm, not by a shift where the word is loaded, keeps a freshly loaded word untouched
// until it is used, so its load is not waited for early.
MOESQ_DEV void e4m3_pair_f16x2(uint32_t w, f16x2& s0, f16x2& s1, bool hi = false) {
  const uint32_t d = __builtin_amdgcn_perm(0u, w, hi ? 0x03030202u : 0x01010000u);  // (b0, b0, b1, b1)
  s0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d, 1.0f, false);
  s1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d, 1.0f, true);
}

// Dense activation 8-group (codes word c: element i in nibble i) -> 4 f16x2 in de-interleaved
// order (a0,a2), (a4,a6), (a1,a3), (a5,a7), scaled by sc.
MOESQ_DEV u32x4 decode_x_group(uint32_t c, f16x2 sc) {
  const uint32_t x0 = f16x2_bits(MOESQ_CVT_FP4(c, 0) * sc);  // (a0, a1)
  const uint32_t x1 = f16x2_bits(MOESQ_CVT_FP4(c, 1) * sc);  // (a2, a3)
  const uint32_t x2 = f16x2_bits(MOESQ_CVT_FP4(c, 2) * sc);  // (a4, a5)
  const uint32_t x3 = f16x2_bits(MOESQ_CVT_FP4(c, 3) * sc);  // (a6, a7)
  u32x4 o;
  o.x = __builtin_amdgcn_perm(x1, x0, 0x05040100u);  // (a0, a2)
  o.y = __builtin_amdgcn_perm(x3, x2, 0x05040100u);  // (a4, a6)
  o.z = __builtin_amdgcn_perm(x1, x0, 0x07060302u);  // (a1, a3)
  o.w = __builtin_amdgcn_perm(x3, x2, 0x07060302u);  // (a5, a7)
  return o;
}

// Sparse-index code of a pair-bitmask nibble (exactly two bits i < j set): i | j << 2. Both
// 4-groups of the de-interleaved 8-group use it.
MOESQ_DEV uint32_t pair_index_code(uint32_t nib) {
  const uint32_t i = (uint32_t)__builtin_ctz(nib | 16u);
  const uint32_t j = (uint32_t)(31 - __builtin_clz(nib | 1u));
  return (i & 3u) | ((j & 3u) << 2);
}

// Sparse index operands of one lane for a 256-K super-step. The kernel layout stores the index
// codes of the lane's eight 8-groups g = 2s + h (step s, half h) as nibbles in the order
// (g0, g2, g4, g6, g1, g3, g5, g7). Returns i02 = index words of steps 0 (low 16 bits) and 2
// (high), i13 = steps 1 and 3; each 16-bit word is c(s,0)*0x11 | c(s,1)*0x11 << 8.
MOESQ_DEV void sparse_index_words(uint32_t m, uint32_t& i02, uint32_t& i13) {
  const uint32_t e = (m & 0x0F0F0F0Fu) * 17u;          // bytes c(0,0) c(2,0) c(0,1) c(2,1), duplicated
  const uint32_t o = ((m >> 4) & 0x0F0F0F0Fu) * 17u;   // bytes c(1,0) c(3,0) c(1,1) c(3,1)
  i02 = __builtin_amdgcn_perm(0u, e, 0x03010200u);
  i13 = __builtin_amdgcn_perm(0u, o, 0x03010200u);
}

// Round an fp32 to bf16 bits, nearest even (finite inputs).
MOESQ_DEV uint32_t f32_to_bf16_bits(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}
MOESQ_DEV float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// ---------------------------------------------------------------- block scan -------------------
// Exclusive scan of vals[0..E) (LDS) into out[0..E] (LDS, out[E] = total) by a block of THREADS:
// each thread sums a contiguous range, wave shuffles scan the per-thread sums, one LDS exchange
// combines the waves.
template <int THREADS>
MOESQ_DEV void block_exclusive_scan(const int32_t* vals, int32_t E, int32_t* out, int32_t* wsum) {
  constexpr int WAVES = THREADS / 64;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int per = (E + THREADS - 1) / THREADS;
  const int lo = min(E, tid * per), hi = min(E, lo + per);
  int sum = 0;
  for (int i = lo; i < hi; i++) sum += vals[i];
  int incl = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int v = 0; v < WAVES; v++) before += (v < w) ? wsum[v] : 0;
  int run = before + incl - sum;
  for (int i = lo; i < hi; i++) {
    out[i] = run;
    run += vals[i];
  }
  if (tid == THREADS - 1) {
    int tot = 0;
#pragma unroll
    for (int v = 0; v < WAVES; v++) tot += wsum[v];
    out[E] = tot;
  }
  __syncthreads();
}
