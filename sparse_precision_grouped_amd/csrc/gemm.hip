// Grouped sparse NVFP4 GEMM for gfx950 (paper Section 2 and Section 3.4 "Grouped sparse GEMM
// execution": Y_e^T = W_e X_e^T per expert in one launch, the sparse weights on the left operand,
// block scales applied inside the product, alpha_e = 1/(gamma_w,e gamma_a,e) on the fp32
// accumulator; Appendix D.1: token counts read on the device, each expert gets ceil(N_e/T_N)
// token tiles, only the last tile of an expert touches padding).
//
// MI355X design:
//  - The paired-4:8 weights feed v_smfmac_f32_16x16x64_f16 (2:4 structured-sparse MFMA) after an
//    even/odd de-interleave of every 8-group, which turns each of the six paired patterns into a
//    valid 2:4 pattern; the pair mask becomes the sparse index operand (two steps' 16-bit index
//    words per VGPR, picked by the instruction's abid field). E2M1 codes are expanded with the
//    gfx950 FP4->f16 convert and multiplied by the UE4M3 block scale (FP8->f16 convert) in f16:
//    e2m1 * e4m3 has at most 6 significant bits, so every operand is exact and the only rounding
//    is the fp32 accumulation. No lookup tables: all decoding is VALU work in registers.
//  - Weights are read from the kernel layout built at load time (prepack_kernel): units of four
//    16-row x 256-K fragments, in which lane (row r, chunk c) finds its 16 packed bytes per
//    fragment and its index codes and scale codes of all four fragments side by side, so a wave
//    reads a 5632-byte unit with six buffer loads. The lane covers K
//    [64c + 16s, +16) at step s of the super-step; the activation (B) operand follows the same K
//    mapping. Buffer loads past an expert's last token return zero, which pads partial tiles.
//  - Decode (few tokens per expert): weight streaming. One workgroup = 16*MF weight rows of one
//    expert; its 4 waves split K and reduce through LDS in a fixed order (deterministic).
//  - Prefill: persistent 512 x 128 tiles (8 waves x 4 m-fragments x 16 rows, 8 n-fragments x 16
//    tokens); the activation tile of each super-step is staged once into LDS (f16, de-interleaved:
//    decoded from the NVFP4 codes, or loaded straight from the quantizer's f16 copy) and shared by
//    the eight waves; the weights go from global memory straight to registers.
//  - The gate_up GEMM of the MLP fuses SwiGLU and the NVFP4 requantization of h in its epilogue:
//    a wave owns the gate rows and the matching up rows of 32 intermediate columns, which is one
//    32-element scale block per token.
#include "common.h"
#include "launch.h"

#include <stdlib.h>

namespace moesq {

MOESQ_DEV f16x16 concat_x(u32x4 lo, u32x4 hi) {
  typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
  u32x8 v;
  v.s0 = lo.x; v.s1 = lo.y; v.s2 = lo.z; v.s3 = lo.w;
  v.s4 = hi.x; v.s5 = hi.y; v.s6 = hi.z; v.s7 = hi.w;
  return __builtin_bit_cast(f16x16, v);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Store 4 consecutive outputs scaled by alpha: fp32, or bf16 rounded to nearest even by the gfx950
// packed convert.
MOESQ_DEV void store4(void* y, int64_t off, f32x4 v, float alpha, int bf16) {
  if (bf16) {
    const bf16x2 lo = __builtin_convertvector((f32x2){v.x * alpha, v.y * alpha}, bf16x2);
    const bf16x2 hi = __builtin_convertvector((f32x2){v.z * alpha, v.w * alpha}, bf16x2);
    uint2 o;
    o.x = __builtin_bit_cast(uint32_t, lo);
    o.y = __builtin_bit_cast(uint32_t, hi);
    *(uint2*)((uint16_t*)y + off) = o;
  } else {
    float4 o;
    o.x = v.x * alpha; o.y = v.y * alpha; o.z = v.z * alpha; o.w = v.w * alpha;
    *(float4*)((float*)y + off) = o;
  }
}

// ============================================================== operand stages (registers) =====
typedef __amdgpu_buffer_rsrc_t rsrc_t;

MOESQ_DEV rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// s_waitcnt operand that waits until at most n (< 16) vector-memory operations are outstanding and does
// not wait on the other counters (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int vmcnt_only(int n) { return (n & 15) | (7 << 4) | (15 << 8); }

// Workgroup barrier after the caller's own s_waitcnt: the empty asm statements keep the compiler from
// moving memory accesses across it, and no fence is emitted, so loads still in flight stay in flight (a
// fence with direct-to-LDS loads outstanding makes the compiler wait for every vector-memory operation).
MOESQ_DEV void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroup barrier that orders LDS accesses only: global loads and stores issued before it stay in
// flight (a plain __syncthreads waits for every outstanding memory operation of the wave).
MOESQ_DEV void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// One 256-K super-step of MF A fragments (16 rows each) for one lane. sw[f] holds fragment f's two
// scale codes in its low half (load_w, the weight-streaming kernel's loads), or, from the tiled kernel's
// half-stage loads, the loaded word itself with the codes in its high half for odd f (a freshly loaded
// word is then not touched until it is used, so its load is not waited for early).
template <int MF>
struct WStage {
  u32x4 pk[MF];
  uint32_t mk[MF];
  uint32_t sw[MF];
};

// Where a wave's MF fragments live in the kernel layout: units of 4 fragments (64 rows) per
// super-step, kGroupBytes each, super-steps of one 64-row group consecutive. g0/g1: byte offset of
// the group's super-step 0 within the expert; j0/j1: first fragment used in that group. Without SPLIT
// the MF (2 or 4) fragments are consecutive from (g0, j0); with SPLIT (MF = 4) fragments 0-1 come
// from (g0, j0) and 2-3 from (g1, j1), as in the gate_up tile (gate rows, then the matching up rows).
struct WSrc {
  uint32_t g0, g1;
  int j0, j1;
};

// Cache policy of the weight-streaming kernel's packed-code loads: non-temporal. Each packed byte is
// read once per launch; the hint measured 7-8% faster for c1 and the c3 gate_up GEMM and 3% for the
// decode-sized MLP. The index and scale codes keep the default policy: the MLP's workgroup pairs share
// their cache lines through L2, and non-temporal loads there measured slower for the MLP.
constexpr int kPackedPolicy = 2;  // the nt bit of the buffer-load cache-policy operand

// Two consecutive fragments (j, j + 1) of a unit into slots f, f + 1: two 16-byte packed loads, one
// 8-byte index-code load and one 4-byte scale load (lane offsets go in the per-lane operand).
template <int MF>
MOESQ_DEV void load_w_pair(WStage<MF>& st, int f, rsrc_t rw, uint32_t go, int j, int lane) {
  st.pk[f] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(go + 1024u * j + 16u * lane), 0, kPackedPolicy));
  st.pk[f + 1] =
      __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(go + 1024u * (j + 1) + 16u * lane), 0, kPackedPolicy));
  const auto m = __builtin_amdgcn_raw_buffer_load_b64(rw, (int)(go + 4096u + 16u * lane + 4u * j), 0, 0);
  st.mk[f] = m[0];
  st.mk[f + 1] = m[1];
  const uint32_t sc = __builtin_amdgcn_raw_buffer_load_b32(rw, (int)(go + 5120u + 8u * lane + 2u * j), 0, 0);
  st.sw[f] = sc;
  st.sw[f + 1] = sc >> 16;
}

template <int MF, bool SPLIT>
MOESQ_DEV void load_w(WStage<MF>& st, rsrc_t rw, const WSrc& src, int lane, int ss) {
  static_assert(MF == 2 || MF == 4, "fragments per wave");
  const uint32_t go = src.g0 + (uint32_t)ss * kGroupBytes;
  if (MF == 4 && !SPLIT) {
#pragma unroll
    for (int j = 0; j < 4; j++)
      st.pk[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(go + 1024u * j + 16u * lane), 0, kPackedPolicy));
    const u32x4 m = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(go + 4096u + 16u * lane), 0, 0));
    st.mk[0] = m.x; st.mk[1] = m.y; st.mk[2] = m.z; st.mk[3] = m.w;
    const auto sc = __builtin_amdgcn_raw_buffer_load_b64(rw, (int)(go + 5120u + 8u * lane), 0, 0);
    st.sw[0] = sc[0]; st.sw[1] = sc[0] >> 16; st.sw[2] = sc[1]; st.sw[3] = sc[1] >> 16;
  } else {
    load_w_pair(st, 0, rw, go, src.j0, lane);
    if (MF == 4) load_w_pair(st, 2, rw, src.g1 + (uint32_t)ss * kGroupBytes, src.j1, lane);
  }
}

// Per-fragment metadata of one super-step: sparse index words (steps 0/2 and 1/3) and the block
// scales of steps 0-1 and 2-3 as f16x2 pairs.
struct WMeta {
  uint32_t i02, i13;
  f16x2 s01, s23;
};

template <int MF>
MOESQ_DEV WMeta w_meta(const WStage<MF>& w, int f, bool odd_high = false) {
  WMeta m;
  sparse_index_words(w.mk[f], m.i02, m.i13);
  e4m3_pair_f16x2(w.sw[f], m.s01, m.s23, odd_high && (f & 1) != 0);
  return m;
}

// A operand of step s (0..3) for m-fragment f: the kernel layout's nibble order makes each FP4
// convert produce one de-interleaved operand register directly.
template <int MF>
MOESQ_DEV f16x8 w_frag(const WStage<MF>& w, const WMeta& m, int f, int s) {
  const f16x2 sc = s < 2 ? m.s01 : m.s23;
  const uint32_t wd = s == 0 ? w.pk[f].x : s == 1 ? w.pk[f].y : s == 2 ? w.pk[f].z : w.pk[f].w;
  u32x4 o;
  o.x = f16x2_bits(MOESQ_CVT_FP4(wd, 0) * sc);
  o.y = f16x2_bits(MOESQ_CVT_FP4(wd, 1) * sc);
  o.z = f16x2_bits(MOESQ_CVT_FP4(wd, 2) * sc);
  o.w = f16x2_bits(MOESQ_CVT_FP4(wd, 3) * sc);
  return __builtin_bit_cast(f16x8, o);
}

// One sparse MFMA of step S (a compile-time constant): the index word's half is chosen by
// abid = S / 2.
template <int S>
MOESQ_DEV f32x4 smfmac_step(f16x8 A, f16x16 B, f32x4 C, const WMeta& m) {
  return __builtin_amdgcn_smfmac_f32_16x16x64_f16(A, B, C, (int)((S & 1) ? m.i13 : m.i02), 0, S >> 1);
}

// Activation operand of one lane for one super-step (decode kernel): for each of the 4 K-steps two
// 8-groups (codes) and the two block-scale pairs. Rows past the expert's tokens read as zero.
struct XStage {
  uint32_t bc[8];
  uint32_t bs0, bs1;
};

MOESQ_DEV void load_x(XStage& st, rsrc_t rq, rsrc_t rs, uint32_t voq, uint32_t vos, int ss) {
#pragma unroll
  for (int s = 0; s < 4; s++) {
    st.bc[2 * s] = __builtin_amdgcn_raw_buffer_load_b32(rq, (int)(voq + 128u * ss + 8u * s), 0, 0);
    st.bc[2 * s + 1] = __builtin_amdgcn_raw_buffer_load_b32(rq, (int)(voq + 128u * ss + 64u + 8u * s), 0, 0);
  }
  st.bs0 = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)(vos + 8u * ss), 0, 0);
  st.bs1 = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)(vos + 8u * ss + 4u), 0, 0);
}

template <int S, int MF>
MOESQ_DEV void x_step(f32x4 (&acc)[MF], const WStage<MF>& w, const WMeta (&m)[MF], const XStage& x, f16x2 a01,
                      f16x2 a23, f16x2 b01, f16x2 b23) {
  const f16x16 B = concat_x(decode_x_group(x.bc[2 * S], S < 2 ? a01 : a23),
                            decode_x_group(x.bc[2 * S + 1], S < 2 ? b01 : b23));
#pragma unroll
  for (int f = 0; f < MF; f++) acc[f] = smfmac_step<S>(w_frag(w, m[f], f, S), B, acc[f], m[f]);
}

template <int MF>
MOESQ_DEV void mma_superstep_x(f32x4 (&acc)[MF], const WStage<MF>& w, const XStage& x) {
  WMeta m[MF];
#pragma unroll
  for (int f = 0; f < MF; f++) m[f] = w_meta(w, f);
  f16x2 a01, a23, b01, b23;
  e4m3_pair_f16x2(x.bs0, a01, a23);
  e4m3_pair_f16x2(x.bs1, b01, b23);
  x_step<0>(acc, w, m, x, a01, a23, b01, b23);
  x_step<1>(acc, w, m, x, a01, a23, b01, b23);
  x_step<2>(acc, w, m, x, a01, a23, b01, b23);
  x_step<3>(acc, w, m, x, a01, a23, b01, b23);
}

// f16 operand copy (xk) for the decode kernel: the lane's two 8-groups of step s are the 16-byte chunks
// g and g + 16 of the super-step with g = 8 (c >> 1) + (c & 1) + 2 s (the same K mapping as the NVFP4
// path), so a step is two 16-byte loads and no decoding.
struct XKStage {
  u32x4 lo[4], hi[4];
};

MOESQ_DEV void load_xk(XKStage& st, rsrc_t rx, uint32_t vox, int ss) {
#pragma unroll
  for (int s = 0; s < 4; s++) {
    st.lo[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(vox + 512u * ss + 32u * s), 0, 0));
    st.hi[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(vox + 512u * ss + 32u * s + 256u), 0, 0));
  }
}

template <int S, int MF>
MOESQ_DEV void xk_step(f32x4 (&acc)[MF], const WStage<MF>& w, const WMeta (&m)[MF], const XKStage& x) {
  const f16x16 B = concat_x(x.lo[S], x.hi[S]);
#pragma unroll
  for (int f = 0; f < MF; f++) acc[f] = smfmac_step<S>(w_frag(w, m[f], f, S), B, acc[f], m[f]);
}

template <int MF>
MOESQ_DEV void mma_superstep_xk(f32x4 (&acc)[MF], const WStage<MF>& w, const XKStage& x) {
  WMeta m[MF];
#pragma unroll
  for (int f = 0; f < MF; f++) m[f] = w_meta(w, f);
  xk_step<0>(acc, w, m, x);
  xk_step<1>(acc, w, m, x);
  xk_step<2>(acc, w, m, x);
  xk_step<3>(acc, w, m, x);
}

// The activation stage of the decode kernel: NVFP4 codes (decoded in registers) or the f16 copy.
template <bool XK>
struct DStage;
template <>
struct DStage<false> {
  XStage x;
  MOESQ_DEV void load(rsrc_t rq, rsrc_t rs, uint32_t voq, uint32_t vos, uint32_t, int ss) { load_x(x, rq, rs, voq, vos, ss); }
};
template <>
struct DStage<true> {
  XKStage x;
  MOESQ_DEV void load(rsrc_t rq, rsrc_t, uint32_t, uint32_t, uint32_t vox, int ss) { load_xk(x, rq, vox, ss); }
};

// The rows of expert e: [off, off + ne). Prefix layout: offsets[e] .. offsets[e+1]. Capacity layout
// (cap > 0, offsets holds the token counts): rows e * cap .. + min(count, cap) of a buffer with a fixed
// per-expert capacity; the remaining rows of the expert are padding and are neither read nor written.
MOESQ_DEV void expert_rows(const GemmArgs& a, int e, int& off, int& ne) {
  if (a.cap > 0) {
    off = e * a.cap;
    ne = min(a.offsets[e], a.cap);
  } else {
    off = a.offsets[e];
    ne = a.offsets[e + 1] - off;
  }
}

// gamma_w of expert e for rows in half h (0: rows < N/2, 1: rows >= N/2): one scale per expert, or a
// (gate, up) pair when the weights carry split tensor scales.
MOESQ_DEV float wscale(const GemmArgs& a, int e, int h) { return a.gsplit ? a.gscale[2 * e + h] : a.gscale[e]; }

MOESQ_DEV uint32_t expert_kl_bytes(int N, int K) { return (uint32_t)(N / 16) * (uint32_t)(K / 256) * kFragBytes; }

// ============================================================== dense NVFP4 control operand =====
// The dense control (unpruned NVFP4, one UE4M3 scale per 32 K) runs the same kernels with the dense
// v_mfma_f32_16x16x32_f16: per 64-K step and 16-row fragment, two MFMAs over the 8-groups g (lo) and
// g + 16 (hi) that the sparse step covers with one 2:4 MFMA. Layout (moesq_prepack_dense_weights):
// per expert, 64-row group and 256-K super-step a kDenseUnitBytes unit; fragment j's lane l owns the
// 32 bytes [2048 j + 32 l, +32) = code words (S0 lo, S0 hi, S1 lo, S1 hi, S2 lo, S2 hi, S3 lo, S3 hi),
// each 8-group with its nibbles in the operand order (0, 2, 4, 6, 1, 3, 5, 7), and the 4 bytes
// [8192 + 16 l + 4 j, +4) = block-scale codes (steps 0-1 lo, 0-1 hi, 2-3 lo, 2-3 hi).
constexpr int kDenseUnitBytes = 9216;

template <int MF>
struct DWStage {
  u32x4 c0[MF], c1[MF];  // code words of steps 0-1 and 2-3
  uint32_t sc[MF];       // scale codes
};

template <int MF>
MOESQ_DEV void load_dw(DWStage<MF>& st, rsrc_t rw, uint32_t g0, int j0, int lane, int ss) {
  static_assert(MF == 2 || MF == 4, "fragments per wave");
  const uint32_t go = g0 + (uint32_t)ss * kDenseUnitBytes;
#pragma unroll
  for (int f = 0; f < MF; f++) {
    const uint32_t o = go + 2048u * (j0 + f) + 32u * lane;
    st.c0[f] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)o, 0, 0));
    st.c1[f] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(o + 16u), 0, 0));
  }
  if (MF == 4) {
    const u32x4 m = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(go + 8192u + 16u * lane), 0, 0));
    st.sc[0] = m.x; st.sc[1] = m.y; st.sc[2] = m.z; st.sc[3] = m.w;
  } else {
    const auto m = __builtin_amdgcn_raw_buffer_load_b64(rw, (int)(go + 8192u + 16u * lane + 4u * j0), 0, 0);
    st.sc[0] = m[0]; st.sc[1] = m[1];
  }
}

// One dense A operand (8 f16) from a code word in operand nibble order, scaled by sc.
MOESQ_DEV f16x8 dense_frag(uint32_t wd, f16x2 sc) {
  u32x4 o;
  o.x = f16x2_bits(MOESQ_CVT_FP4(wd, 0) * sc);
  o.y = f16x2_bits(MOESQ_CVT_FP4(wd, 1) * sc);
  o.z = f16x2_bits(MOESQ_CVT_FP4(wd, 2) * sc);
  o.w = f16x2_bits(MOESQ_CVT_FP4(wd, 3) * sc);
  return __builtin_bit_cast(f16x8, o);
}

struct DMeta {
  f16x2 lo01, hi01, lo23, hi23;
};

template <int MF>
MOESQ_DEV DMeta dense_meta(const DWStage<MF>& w, int f) {
  DMeta m;
  e4m3_pair_f16x2(w.sc[f], m.lo01, m.hi01);
  e4m3_pair_f16x2(w.sc[f], m.lo23, m.hi23, true);
  return m;
}

// Step S of fragment f against the activation operand halves (blo: 8-group g, bhi: g + 16).
template <int S, int MF>
MOESQ_DEV f32x4 dense_step(const DWStage<MF>& w, const DMeta& m, int f, u32x4 blo, u32x4 bhi, f32x4 acc) {
  const u32x4 cw = S < 2 ? w.c0[f] : w.c1[f];
  const uint32_t wlo = (S & 1) ? cw.z : cw.x, whi = (S & 1) ? cw.w : cw.y;
  const f16x8 alo = dense_frag(wlo, S < 2 ? m.lo01 : m.lo23);
  const f16x8 ahi = dense_frag(whi, S < 2 ? m.hi01 : m.hi23);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, __builtin_bit_cast(f16x8, blo), acc, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, __builtin_bit_cast(f16x8, bhi), acc, 0, 0, 0);
}

template <int S, int MF>
MOESQ_DEV void dense_x_step(f32x4 (&acc)[MF], const DWStage<MF>& w, const DMeta (&m)[MF], const XStage& x,
                            f16x2 a01, f16x2 a23, f16x2 b01, f16x2 b23) {
  const u32x4 blo = decode_x_group(x.bc[2 * S], S < 2 ? a01 : a23);
  const u32x4 bhi = decode_x_group(x.bc[2 * S + 1], S < 2 ? b01 : b23);
#pragma unroll
  for (int f = 0; f < MF; f++) acc[f] = dense_step<S>(w, m[f], f, blo, bhi, acc[f]);
}

template <int MF>
MOESQ_DEV void dense_superstep_x(f32x4 (&acc)[MF], const DWStage<MF>& w, const XStage& x) {
  DMeta m[MF];
#pragma unroll
  for (int f = 0; f < MF; f++) m[f] = dense_meta(w, f);
  f16x2 a01, a23, b01, b23;
  e4m3_pair_f16x2(x.bs0, a01, a23);
  e4m3_pair_f16x2(x.bs1, b01, b23);
  dense_x_step<0>(acc, w, m, x, a01, a23, b01, b23);
  dense_x_step<1>(acc, w, m, x, a01, a23, b01, b23);
  dense_x_step<2>(acc, w, m, x, a01, a23, b01, b23);
  dense_x_step<3>(acc, w, m, x, a01, a23, b01, b23);
}

template <int MF>
MOESQ_DEV void dense_superstep_xk(f32x4 (&acc)[MF], const DWStage<MF>& w, const XKStage& x) {
  DMeta m[MF];
#pragma unroll
  for (int f = 0; f < MF; f++) m[f] = dense_meta(w, f);
#pragma unroll
  for (int f = 0; f < MF; f++) {
    acc[f] = dense_step<0>(w, m[f], f, x.lo[0], x.hi[0], acc[f]);
    acc[f] = dense_step<1>(w, m[f], f, x.lo[1], x.hi[1], acc[f]);
    acc[f] = dense_step<2>(w, m[f], f, x.lo[2], x.hi[2], acc[f]);
    acc[f] = dense_step<3>(w, m[f], f, x.lo[3], x.hi[3], acc[f]);
  }
}

MOESQ_DEV uint32_t expert_dense_bytes(int N, int K) { return (uint32_t)(N / 64) * (uint32_t)(K / 256) * kDenseUnitBytes; }

// Weight stage of the decode kernel: the sparse layout (WStage) or the dense control (DWStage).
template <int MF, bool DENSE, bool SPLIT = false>
struct WS;
template <int MF, bool SPLIT>
struct WS<MF, false, SPLIT> {
  WStage<MF> w;
  MOESQ_DEV void load(rsrc_t rw, const WSrc& src, int lane, int ss) { load_w<MF, SPLIT>(w, rw, src, lane, ss); }
};
template <int MF>
struct WS<MF, true, false> {
  DWStage<MF> w;
  MOESQ_DEV void load(rsrc_t rw, const WSrc& src, int lane, int ss) { load_dw<MF>(w, rw, src.g0, src.j0, lane, ss); }
};

template <int MF, bool SPLIT>
MOESQ_DEV void stage_mma(f32x4 (&acc)[MF], const WS<MF, false, SPLIT>& w, const DStage<false>& x) { mma_superstep_x(acc, w.w, x.x); }
template <int MF, bool SPLIT>
MOESQ_DEV void stage_mma(f32x4 (&acc)[MF], const WS<MF, false, SPLIT>& w, const DStage<true>& x) { mma_superstep_xk(acc, w.w, x.x); }
template <int MF>
MOESQ_DEV void stage_mma(f32x4 (&acc)[MF], const WS<MF, true>& w, const DStage<false>& x) { dense_superstep_x(acc, w.w, x.x); }
template <int MF>
MOESQ_DEV void stage_mma(f32x4 (&acc)[MF], const WS<MF, true>& w, const DStage<true>& x) { dense_superstep_xk(acc, w.w, x.x); }

// Epilogue forms of the GEMM kernels, fixed at compile time so that the production kernels carry no
// dump or calibration code (the weight-streaming MLP kernel runs at its register cap).
constexpr int kEpiPlain = 0;    // plain GEMM output (alpha_e, fp32 or bf16 store)
constexpr int kEpiMlp = 1;      // gate_up of the MLP: SwiGLU + NVFP4 requantization of h
constexpr int kEpiMlpDump = 2;  // kEpiMlp plus the fp32 gate_up and h dumps (GemmArgs::dump / hdump)
constexpr int kEpiCalib = 3;    // gate_up + SwiGLU, per-expert amax(h) only (GemmArgs::amax_h)

// MLP gate_up epilogue for one token (permuted row p; tv: the row is a real token): g0, g1 are the two
// gate fragments and u0, u1 the matching up fragments of the 32 intermediate columns [ib, ib + 32);
// lane (r16, cc) holds columns 16 f + 4 cc .. + 3 of fragment f. h = SiLU(g) * u in fp32 (the optional
// fp32 dumps keep g and u, and h; alpha and alpha_u are the gate and up alpha_e, equal unless the weights
// carry split tensor scales), then the NVFP4 requantization of the 32-block with the expert's gamma_h
// (amax over the 4 lanes cc = 0..3: xor 16, 32), and the h codes, block scale and optional f16 copy.
// Returns the block's amax(h) for a real token (0 otherwise); in calibration (EPI = kEpiCalib) nothing
// is written and gh is not used.
template <int EPI>
MOESQ_DEV float mlp_epilogue_token(const GemmArgs& a, int64_t p, bool tv, int ib, int cc, float alpha, float alpha_u,
                                   float gh, f32x4 g0, f32x4 g1, f32x4 u0, f32x4 u1) {
  const int N = a.N, I = N / 2;
  const f32x4 gg[2] = {g0, g1}, uu[2] = {u0, u1};
  float h[8];
#pragma unroll
  for (int f = 0; f < 2; f++) {
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const float g = gg[f][r] * alpha;
      const float u = uu[f][r] * alpha_u;
      h[4 * f + r] = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;  // SiLU(g) u (fast exp and reciprocal)
    }
    if (EPI == kEpiMlpDump && tv && a.dump) {
      const int64_t rowo = p * N;
      float4 gv, uv;
      gv.x = gg[f][0] * alpha; gv.y = gg[f][1] * alpha; gv.z = gg[f][2] * alpha; gv.w = gg[f][3] * alpha;
      uv.x = uu[f][0] * alpha_u; uv.y = uu[f][1] * alpha_u; uv.z = uu[f][2] * alpha_u; uv.w = uu[f][3] * alpha_u;
      *(float4*)(a.dump + rowo + ib + 16 * f + 4 * cc) = gv;
      *(float4*)(a.dump + rowo + I + ib + 16 * f + 4 * cc) = uv;
    }
    if (EPI == kEpiMlpDump && tv && a.hdump) {
      float4 hv;
      hv.x = h[4 * f]; hv.y = h[4 * f + 1]; hv.z = h[4 * f + 2]; hv.w = h[4 * f + 3];
      *(float4*)(a.hdump + p * I + ib + 16 * f + 4 * cc) = hv;
    }
  }
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i++) am = __builtin_fmaxf(am, __builtin_fabsf(h[i]));
  am = __builtin_fmaxf(am, __shfl_xor(am, 16));
  am = __builtin_fmaxf(am, __shfl_xor(am, 32));
  if (EPI == kEpiCalib) return tv ? am : 0.0f;
  const float t = gh * am;
  const float uq = t / 6.0f;
  const uint32_t sc = e4m3_encode(uq);
  const float sv = e4m3_value(sc) / gh;
  if (tv) {
    f16x2 s01, s01b;
    e4m3_pair_f16x2(sc, s01, s01b);
    // E2M1(h / sv) of the correctly rounded quotients (e2m1_codes4); a block with a huge or non-finite
    // amax takes the plain division and encoder
    const float r = sv != 0.0f ? 1.0f / sv : 0.0f;
    const bool fast = am * r < 1e30f;
    uint32_t cw[2];
#pragma unroll
    for (int f = 0; f < 2; f++) {
      uint32_t codes = 0u;
      if (sv != 0.0f) {
        if (fast) {
          codes = e2m1_codes4(h[4 * f], h[4 * f + 1], h[4 * f + 2], h[4 * f + 3], sv, r);
        } else {
#pragma unroll
          for (int i = 0; i < 4; i++) codes |= e2m1_encode(h[4 * f + i] / sv) << (4 * i);
        }
      }
      cw[f] = codes;
      const int i0 = ib + 16 * f + 4 * cc;  // 4 consecutive intermediate columns: half (cc & 1) of an 8-group
      if (a.h_k) {
        // f16 copy in the de-interleaved group order (a0,a2,a4,a6,a1,a3,a5,a7): this lane holds
        // a[4h..4h+3] (h = cc & 1) and writes words h ((a4h, a4h+2)) and 2 + h ((a4h+1, a4h+3)).
        const uint32_t v01 = f16x2_bits(MOESQ_CVT_FP4(codes, 0) * s01);  // (v0, v1)
        const uint32_t v23 = f16x2_bits(MOESQ_CVT_FP4(codes, 1) * s01);  // (v2, v3)
        uint8_t* grp = (uint8_t*)a.h_k + (p * I + (i0 & ~7)) * 2;
        *(uint32_t*)(grp + 4 * (cc & 1)) = __builtin_amdgcn_perm(v23, v01, 0x05040100u);
        *(uint32_t*)(grp + 8 + 4 * (cc & 1)) = __builtin_amdgcn_perm(v23, v01, 0x07060302u);
      }
    }
    // The two lanes of a lane-row pair (cc = 2m, 2m + 1; same token) swap halves: the even lane then
    // holds the 8 codes of columns ib + 4 cc .. + 7 of the first 16, the odd lane those of columns
    // ib + 16 + 4 (cc - 1) .. + 7, and each stores them as one 4-byte word.
    const auto pr = __builtin_amdgcn_permlane16_swap(cw[0], cw[1], false, false);
    const int g0 = (cc & 1) ? ib + 16 + 4 * (cc - 1) : ib + 4 * cc;
    *(uint32_t*)(a.h_q + p * (I / 2) + g0 / 2) = (pr[0] & 0xFFFFu) | (pr[1] << 16);
    if (cc == 0) a.h_s[p * (I / 32) + ib / 32] = (uint8_t)sc;
  }
  return tv ? am : 0.0f;
}

// Calibration: the largest of the wave's per-token block amax values goes to the expert's word by one
// device atomic max on its float bits (non-negative floats order like their bit patterns, so the result
// does not depend on the order of the atomics).
MOESQ_DEV void calib_amax_commit(uint32_t* amax_h, int e, float m) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) m = __builtin_fmaxf(m, __shfl_xor(m, d));
  if ((threadIdx.x & 63) == 0 && m > 0.0f) atomicMax(&amax_h[e], __float_as_uint(m));
}

// ============================================================================ decode kernel =====
// Weight streaming for few tokens per expert. A workgroup of KS * RG waves covers 16*MF*RG weight rows
// of one expert: RG row groups of 16*MF rows, each split over KS waves along K (wave kw takes
// super-steps kw, kw + KS, ...). The KS partial sums of a row group are added in wave order through
// LDS (deterministic). Each wave keeps two super-steps of operands in flight (register double
// buffering). Experts with more than 16 tokens loop over 16-token blocks.
// grid (N / (16*MF*RG), E).
// MLP (the gate_up GEMM of the routed-expert MLP, N = 2I): workgroup x takes gate rows [32 x, +32) and
// the matching up rows [I + 32 x, +32) (fragments 0-1 and 2-3), so after the K reduction one wave holds
// the gate and up sums of 32 intermediate columns, one 32-block per token: SwiGLU and the NVFP4
// requantization of h run in the same epilogue as the tiled kernel's.
// Weight streaming here is bound by the bytes a CU keeps in flight, so the register budget is capped
// at 168 VGPRs for 3 waves per SIMD (no spills). The f16-operand forms of the dense control and of the
// MLP epilogue need more with two activation stages, so they hold one: each step's activations are
// reloaded right after that step's MFMAs, while the weights stay double-buffered.
template <int MF, int KS, int RG, bool XK, bool DENSE, int MLP = kEpiPlain>
__global__ __launch_bounds__(64 * KS * RG) __attribute__((amdgpu_waves_per_eu(3, 3))) void gemm_decode_kernel(GemmArgs a) {
  // the f16-operand forms of the dense control and of the MLP epilogue hold one activation stage
  constexpr bool kOneX = (DENSE || MLP) && XK;
  static_assert(!MLP || (MF == 4 && RG == 1 && KS > 1 && !DENSE), "MLP epilogue: 32 gate + 32 up rows per workgroup");
  __shared__ f32x4 red[KS > 1 ? KS * RG : 1][MF][64];
  const int e = blockIdx.y;
  int off, ne;
  expert_rows(a, e, off, ne);
  if (ne <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, c = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw = w % KS, rg = w / KS;
  const int K = a.K, N = a.N, nss = K / 256;
  const int rb0 = (blockIdx.x * RG + rg) * MF;
  const uint32_t ekl = DENSE ? expert_dense_bytes(N, K) : expert_kl_bytes(N, K);
  const rsrc_t rw = make_rsrc(a.kl + (size_t)e * ekl, ekl);
  WSrc src;
  // MLP: workgroups 2m and 2m+1 read the two halves of the same 64-row units' mask and scale lines;
  // when gridDim.x is a multiple of 16 the blocks are renumbered so that such a pair is dispatched 8
  // apart, i.e. to the same XCD (workgroups go to the XCDs round-robin), and shares its L2 lines.
  const int bx = (MLP && gridDim.x % 16 == 0)
                     ? (int)((blockIdx.x & ~15u) + 2 * (blockIdx.x & 7u) + ((blockIdx.x >> 3) & 1u))
                     : (int)blockIdx.x;
  if (MLP) {
    const int rgate = 2 * bx, rup = N / 32 + 2 * bx;  // 16-row blocks of the gate / up rows
    src.g0 = (uint32_t)(rgate / 4) * (uint32_t)nss * kGroupBytes;
    src.j0 = rgate % 4;
    src.g1 = (uint32_t)(rup / 4) * (uint32_t)nss * kGroupBytes;
    src.j1 = rup % 4;
  } else {
    src.g0 = (uint32_t)(rb0 / 4) * (uint32_t)nss * (DENSE ? kDenseUnitBytes : kGroupBytes);
    src.j0 = rb0 % 4;
    src.g1 = 0;
    src.j1 = 0;
  }
  const rsrc_t rq = XK ? make_rsrc((const uint8_t*)a.xk + (size_t)off * K * 2, (uint32_t)ne * K * 2)
                      : make_rsrc(a.q + (size_t)off * (K / 2), (uint32_t)ne * (K / 2));
  const rsrc_t rs = make_rsrc(a.s + (size_t)off * (K / 32), (uint32_t)ne * (K / 32));
  const int n0 = rb0 * 16;
  // alpha_e = 1/(gamma_w gamma_a); the MLP's gate rows take the first and its up rows the second
  // tensor scale, a plain wave the scale of its row half
  const float alpha = 1.0f / (wscale(a, e, MLP ? 0 : (n0 >= N / 2)) * a.gamma_a[e]);
  const float alpha_u = MLP ? 1.0f / (wscale(a, e, 1) * a.gamma_a[e]) : alpha;
  for (int tb = 0; tb < ne; tb += 16) {
    f32x4 acc[MF];
#pragma unroll
    for (int f = 0; f < MF; f++) acc[f] = (f32x4){0.f, 0.f, 0.f, 0.f};
    const int tok = tb + r16;
    const bool tv = tok < ne;
    // byte offsets of the lane's first activation group (step 0) and its block scales
    const uint32_t voq = (uint32_t)tok * (K / 2) + 32u * (c >> 1) + 4u * (c & 1);
    const uint32_t vos = (uint32_t)tok * (K / 32) + 2u * (c >> 1);
    const uint32_t vox = (uint32_t)tok * (uint32_t)(2 * K) + 16u * (8u * (c >> 1) + (c & 1));
    WS<MF, DENSE, (MLP != kEpiPlain)> w0, w1;
    DStage<XK> x0, x1;
    int ss = kw;
    if (ss < nss) {
      w0.load(rw, src, lane, ss);
      x0.load(rq, rs, voq, vos, vox, ss);
    }
    if constexpr (kOneX) {
      // one activation stage, reloaded as soon as a step has used it; the weights stay double-buffered
      while (ss < nss) {
        const int s1 = ss + KS, s2 = ss + 2 * KS;
        if (s1 < nss) w1.load(rw, src, lane, s1);
        stage_mma(acc, w0, x0);
        if (s1 < nss) x0.load(rq, rs, voq, vos, vox, s1);
        if (s2 < nss) w0.load(rw, src, lane, s2);
        if (s1 < nss) stage_mma(acc, w1, x0);
        if (s2 < nss) x0.load(rq, rs, voq, vos, vox, s2);
        ss = s2;
      }
    } else {
      while (ss < nss) {
        const int s1 = ss + KS, s2 = ss + 2 * KS;
        if (s1 < nss) {
          w1.load(rw, src, lane, s1);
          x1.load(rq, rs, voq, vos, vox, s1);
        }
        stage_mma(acc, w0, x0);
        if (s2 < nss) {
          w0.load(rw, src, lane, s2);
          x0.load(rq, rs, voq, vos, vox, s2);
        }
        if (s1 < nss) stage_mma(acc, w1, x1);
        ss = s2;
      }
    }
    if (KS == 1) {
      if (tv) {
#pragma unroll
        for (int f = 0; f < MF; f++) store4(a.y, (int64_t)(off + tok) * N + n0 + 16 * f + 4 * c, acc[f], alpha, a.y_bf16);
      }
    } else {
#pragma unroll
      for (int f = 0; f < MF; f++) red[rg * KS + kw][f][lane] = acc[f];
      __syncthreads();
      if (MLP) {
        if (kw == 0) {
          f32x4 sum[4];
#pragma unroll
          for (int f = 0; f < 4; f++) {
            sum[f] = red[0][f][lane];
#pragma unroll
            for (int v = 1; v < KS; v++) sum[f] = sum[f] + red[v][f][lane];
          }
          const float gh = MLP == kEpiCalib ? 1.0f : a.gamma_h[e];
          const float am = mlp_epilogue_token<MLP>(a, off + tok, tv, 32 * bx, c, alpha, alpha_u, gh, sum[0], sum[1],
                                                   sum[2], sum[3]);
          // calibration: one atomic max per 16-token block (nothing carried across the block loop)
          if (MLP == kEpiCalib) calib_amax_commit(a.amax_h, e, am);
        }
      } else {
        for (int f = kw; f < MF; f += KS) {
          f32x4 sum = red[rg * KS][f][lane];
#pragma unroll
          for (int v = 1; v < KS; v++) sum = sum + red[rg * KS + v][f][lane];
          if (tv) store4(a.y, (int64_t)(off + tok) * N + n0 + 16 * f + 4 * c, sum, alpha, a.y_bf16);
        }
      }
      __syncthreads();
    }
  }
}

// ==================================================== dispatch + GEMM in one launch (decode) =====
// Small decode batches: the routing, the activation quantization and the weight-streaming GEMM of one
// layer in a single launch (the work of route_quantize_kernel followed by gemm_decode_kernel<4, 4, 1,
// true>, with the same results). Workgroup (x, e) ranks all T*k ids itself to find expert e's count,
// offset and slots in slot order, issues its first weight loads, then quantizes the expert's tokens
// (up to kDispTok per pass) into LDS as the f16 operand while those loads are in flight, and runs the
// decode kernel's K-split MMA loop and fixed-order reduction with B read from LDS. The workgroups of
// row block 0 also write the routing tables and the q / s (/ xk) rows of their expert, so every output
// of the two-call path is produced.
constexpr int kDispTok = 8;          // tokens per pass (LDS rows)
constexpr int kDispMaxSlots = 1024;  // T*k
constexpr int kDispMaxK = 2048;

struct DispArgs {
  const int32_t* ids;
  int32_t n, k;  // slots T*k, top-k
  const void* x;
  int32_t x_bf16;
  int64_t ld_x;
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_slot;
  int32_t* slot_pos;
  int32_t* dev_status;
  uint8_t* q;
  uint8_t* s;
  uint8_t* xk;  // optional f16 copy of the quantized rows
};

MOESQ_DEV void lds_xk(XKStage& st, const uint8_t* brow, bool tv, int ss) {
#pragma unroll
  for (int s = 0; s < 4; s++) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    st.lo[s] = tv ? *(const u32x4*)(brow + 512 * ss + 32 * s) : z;
    st.hi[s] = tv ? *(const u32x4*)(brow + 512 * ss + 32 * s + 256) : z;
  }
}

// The 8 token values of quantization item gi (row i = gi / gpr of the pass, 8-group gi % gpr), or zeros.
MOESQ_DEV void load_token8(const DispArgs& d, const int32_t* list, int tb, int gpr, int gi, int nq, float v[8]) {
#pragma unroll
  for (int j = 0; j < 8; j++) v[j] = 0.0f;
  if (gi >= nq) return;
  const int i = gi / gpr, ch = gi - i * gpr;
  const int64_t t = list[tb + i] / d.k;
  if (d.x_bf16) {
    const uint4 raw = *(const uint4*)((const uint16_t*)d.x + t * d.ld_x + 8 * ch);
    const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int j = 0; j < 4; j++) {
      v[2 * j] = bf16_bits_to_f32(wd[j] & 0xFFFFu);
      v[2 * j + 1] = bf16_bits_to_f32(wd[j] >> 16);
    }
  } else {
    const float4 x0 = *(const float4*)((const float*)d.x + t * d.ld_x + 8 * ch);
    const float4 x1 = *(const float4*)((const float*)d.x + t * d.ld_x + 8 * ch + 4);
    v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w;
    v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
  }
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void dispatch_gemm_kernel(GemmArgs a,
                                                                                                     DispArgs d) {
  constexpr int MF = 4, KS = 4, R = kDispMaxSlots / 256;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_act[];  // kDispTok rows of 2K + 16 bytes; then the reduction
  __shared__ int32_t list[kDispMaxSlots];                            // expert e's slots in slot order
  __shared__ int32_t ceq[R][4], clt[R][4];
  const int e = blockIdx.y, bx = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int E = a.E, K = a.K, N = a.N, nss = K / 256;
  // ---- routing of expert e
  int idv[R];
#pragma unroll
  for (int r = 0; r < R; r++) {
    const int f = tid + 256 * r;
    idv[r] = f < d.n ? d.ids[f] : -1;
  }
  uint64_t meq[R];
#pragma unroll
  for (int r = 0; r < R; r++) {
    const bool valid = idv[r] >= 0 && idv[r] < E;
    meq[r] = __ballot(idv[r] == e);
    const uint64_t mlt = __ballot(valid && idv[r] < e);
    if (lane == 0) {
      ceq[r][w] = __builtin_popcountll(meq[r]);
      clt[r][w] = __builtin_popcountll(mlt);
    }
  }
  __syncthreads();
  int ne = 0, off = 0;
  int base[R];
#pragma unroll
  for (int r = 0; r < R; r++) {
#pragma unroll
    for (int v = 0; v < 4; v++) {
      if (v == w) base[r] = ne;
      ne += ceq[r][v];
      off += clt[r][v];
    }
  }
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int r = 0; r < R; r++) {
    if (idv[r] == e) {
      const int f = tid + 256 * r;
      const int rank = base[r] + __builtin_popcountll(meq[r] & below);
      list[rank] = f;
      if (bx == 0) {
        d.sorted_slot[off + rank] = f;
        d.slot_pos[f] = off + rank;
      }
    }
  }
  if (bx == 0) {
    if (tid == 0) {
      d.counts[e] = ne;
      d.offsets[e] = off;
      if (e == E - 1) d.offsets[E] = off + ne;  // all valid slots
    }
    if (e == 0) {
#pragma unroll
      for (int r = 0; r < R; r++) {
        const int f = tid + 256 * r;
        if (f < d.n && !(idv[r] >= 0 && idv[r] < E)) {
          d.slot_pos[f] = -1;
          if (d.dev_status) *d.dev_status = MOESQ_ERR_INVALID_ARG;
        }
      }
    }
  }
  __syncthreads();
  if (ne == 0) return;
  // ---- weights and the K-split MMA, as gemm_decode_kernel<4, 4, 1>
  const int kw = w, rb0 = bx * MF, n0 = rb0 * 16;
  const int r16 = lane & 15, c = lane >> 4;
  const uint32_t ekl = expert_kl_bytes(N, K);
  const rsrc_t rw = make_rsrc(a.kl + (size_t)e * ekl, ekl);
  WSrc src;
  src.g0 = (uint32_t)(rb0 / 4) * (uint32_t)nss * kGroupBytes;
  src.j0 = 0;
  src.g1 = 0;
  src.j1 = 0;
  const float ga = a.gamma_a[e];
  const float alpha = 1.0f / (wscale(a, e, n0 >= N / 2) * ga);
  const int rowb = 2 * K + 16;  // LDS row stride of the f16 activations
  const int gpr = K / 8;        // 8-groups per row
  const uint8_t* brow = lds_act + r16 * rowb + 16 * (8 * (c >> 1) + (c & 1));
  for (int tb = 0; tb < ne; tb += kDispTok) {
    const int nb = min(kDispTok, ne - tb);
    const int nq = nb * gpr;
    // this thread's first 8 token values, loaded before the weights: waiting for them then does not
    // wait for the weight loads (vector-memory counters complete in issue order)
    float v[8];
    load_token8(d, list, tb, gpr, tid, nq, v);
    WS<MF, false> w0, w1;
    int ss = kw;
    if (ss < nss) w0.load(rw, src, lane, ss);
    if (ss + KS < nss) w1.load(rw, src, lane, ss + KS);
    // quantize the pass's tokens (as quantize_token_copies: 4 lanes per 32-block) into LDS
    for (int gi0 = 0; gi0 < nq; gi0 += 256) {
      const int gi = gi0 + tid;
      const bool gv = gi < nq;
      const int i = gv ? gi / gpr : 0, ch = gi - i * gpr;
      if (gi0 > 0) load_token8(d, list, tb, gpr, gi, nq, v);
      uint32_t codes, sc;
      quant8_block4(v, ga, codes, sc);
      f16x2 sv, unused;
      e4m3_pair_f16x2(sc, sv, unused);
      const u32x4 xv = decode_x_group(codes, sv);
      if (gv) {
        *(u32x4*)(lds_act + i * rowb + 16 * ch) = xv;
        if (bx == 0) {
          const int64_t p = off + tb + i;
          *(uint32_t*)(d.q + p * (K / 2) + 4 * ch) = codes;
          if ((lane & 3) == 0) d.s[p * (K / 32) + ch / 4] = (uint8_t)sc;
          if (d.xk) *(u32x4*)(d.xk + (p * K + 8 * ch) * 2) = xv;
        }
      }
    }
    __syncthreads();
    f32x4 acc[MF];
#pragma unroll
    for (int f = 0; f < MF; f++) acc[f] = (f32x4){0.f, 0.f, 0.f, 0.f};
    const bool tv = r16 < nb;
    while (ss < nss) {
      const int s1 = ss + KS, s2 = ss + 2 * KS, s3 = ss + 3 * KS;
      {
        XKStage xs;
        lds_xk(xs, brow, tv, ss);
        mma_superstep_xk(acc, w0.w, xs);
      }
      if (s2 < nss) w0.load(rw, src, lane, s2);
      if (s1 < nss) {
        XKStage xs;
        lds_xk(xs, brow, tv, s1);
        mma_superstep_xk(acc, w1.w, xs);
        if (s3 < nss) w1.load(rw, src, lane, s3);
      }
      ss = s2;
    }
    // fixed-order K reduction through LDS (reusing the activation rows)
    __syncthreads();
    f32x4* red = (f32x4*)lds_act;  // [KS][MF][64]
#pragma unroll
    for (int f = 0; f < MF; f++) red[(kw * MF + f) * 64 + lane] = acc[f];
    __syncthreads();
    for (int f = kw; f < MF; f += KS) {
      f32x4 sum = red[f * 64 + lane];
#pragma unroll
      for (int v = 1; v < KS; v++) sum = sum + red[(v * MF + f) * 64 + lane];
      if (tv) store4(a.y, (int64_t)(off + tb + r16) * N + n0 + 16 * f + 4 * c, sum, alpha, a.y_bf16);
    }
    __syncthreads();
  }
}

// One launch only where it is faster than the two: every workgroup of an expert repeats the
// quantization of that expert's tokens, which outweighs the saved launch once the batch has more
// than about one routed row per two experts (measured at E = 128, K = 2048, N = 1536, top-8:
// 16.6 vs 17.7 us at T*k = 32, 22.0 vs 22.6 us at T*k = 64, 30.6 vs 27.7 us at T*k = 128).
bool dispatch_gemm_fused(int64_t T, int32_t k, int32_t E, int32_t K) {
  const int64_t n = T * k;
  return T > 0 && n <= kDispMaxSlots && 2 * n <= (int64_t)E && K <= kDispMaxK && E <= kMaxExpertsRoute;
}

int launch_dispatch_gemm(hipStream_t st, const GemmArgs& a, const int32_t* ids, int64_t T, int32_t k, const void* x,
                         bool x_bf16, int64_t ld_x, int32_t* counts, int32_t* offsets, int32_t* sorted_slot,
                         int32_t* slot_pos, int32_t* dev_status, uint8_t* q, uint8_t* s, void* xk) {
  DispArgs d{};
  d.ids = ids; d.n = (int32_t)(T * k); d.k = k;
  d.x = x; d.x_bf16 = x_bf16; d.ld_x = ld_x;
  d.counts = counts; d.offsets = offsets; d.sorted_slot = sorted_slot; d.slot_pos = slot_pos;
  d.dev_status = dev_status; d.q = q; d.s = s; d.xk = (uint8_t*)xk;
  const size_t lds = (size_t)max(kDispTok * (2 * a.K + 16), 4 * 4 * 64 * 16);
  hipLaunchKernelGGL(dispatch_gemm_kernel, dim3(a.N / 64, a.E), dim3(256), lds, st, a, d);
  return hipGetLastError() == hipSuccess ? MOESQ_OK : MOESQ_ERR_HIP;
}

// ============================================================================= tiled kernel =====
// Prefill-sized problems. A workgroup of 8 waves computes 512 weight rows x 128 tokens of one expert
// (MLP gate_up: 256 gate rows and the matching 256 up rows); a wave owns 64 rows (4 m-fragments)
// and all 128 tokens (8 n-fragments), so each decoded weight operand feeds 8 MFMAs and each staged
// activation operand is shared by all 8 waves. Token tiles past an expert's last token skip their
// empty 16-token fragments.
constexpr int kTileTok = 128;                          // T_N
constexpr int kTileNF = kTileTok / 16;                 // n-fragments per wave
constexpr int kTileThreads = 512;                      // 8 waves
constexpr int kPfGroups = 32;                          // 8-element groups per 256-K super-step
constexpr int kBTileBytes = kTileTok * kPfGroups * 16;  // 65536 B: one super-step of f16 activations

// Activation tile (B) in LDS, both paths: 16-byte chunk (token r, 8-group g of the super-step) at
// 16 * (32 r + (g ^ (r & 31))). The XOR swizzle keeps the 16 rows read by one B fragment, and the 16
// tokens written by one staging store, on distinct banks.
MOESQ_DEV uint8_t* b_chunk(uint8_t* Bs, int r, int g) { return Bs + 16 * (32 * r + (g ^ (r & 31))); }
MOESQ_DEV const uint8_t* b_chunk(const uint8_t* Bs, int r, int g) { return Bs + 16 * (32 * r + (g ^ (r & 31))); }

// Activation staging of one super-step from NVFP4 codes: thread (token, quarter of the super-step)
// reads 32 code bytes (8 groups = 64 K) and their two block scales and decodes them to f16
// (de-interleaved) into LDS.
struct PStage {
  u32x4 cw0, cw1;
  uint32_t sc2;
};

MOESQ_DEV void load_p(PStage& st, rsrc_t rq, rsrc_t rs, uint32_t voq, uint32_t vos, int ss) {
  st.cw0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)(voq + 128u * ss), 0, 0));
  st.cw1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)(voq + 128u * ss + 16u), 0, 0));
  st.sc2 = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)(vos + 8u * ss), 0, 0);
}

// Decode the staged codes of token `tok`, groups 8 qtr + G0 .. 8 qtr + G1 - 1, into the swizzled tile.
template <int G0, int G1>
MOESQ_DEV void stage_p_part(const PStage& st, uint8_t* Bs, int tok, int qtr) {
  f16x2 s0, s1;
  e4m3_pair_f16x2(st.sc2, s0, s1);
  const uint32_t cw[8] = {st.cw0.x, st.cw0.y, st.cw0.z, st.cw0.w, st.cw1.x, st.cw1.y, st.cw1.z, st.cw1.w};
#pragma unroll
  for (int i = G0; i < G1; i++) *(u32x4*)b_chunk(Bs, tok, 8 * qtr + i) = decode_x_group(cw[i], i < 4 ? s0 : s1);
}

MOESQ_DEV void stage_p(const PStage& st, uint8_t* Bs, int tok, int qtr) { stage_p_part<0, 8>(st, Bs, tok, qtr); }

// One K-step (64 K) of the wave's MF x NF fragments. The n-fragments go in blocks of G; a block
// whose first token lies past the expert's last token (n >= nv, wave uniform) is skipped, so a
// partial token tile costs about its own size.
#ifndef MOESQ_TILE_SKIP_G
#define MOESQ_TILE_SKIP_G 4
#endif
template <int S, int MF, int NF, bool XK>
MOESQ_DEV void lds_step(f32x4 (&acc)[MF][NF], const WStage<MF>& w, const WMeta (&m)[MF], const uint8_t* Bs, int r16,
                        int c, int nv) {
  constexpr int G = MOESQ_TILE_SKIP_G;
  f16x8 A[MF];
#pragma unroll
  for (int f = 0; f < MF; f++) A[f] = w_frag(w, m[f], f, S);
  const int g1 = 8 * (c >> 1) + 2 * S + (c & 1);
#pragma unroll
  for (int n0 = 0; n0 < NF; n0 += G) {
    if (G == NF || n0 < nv) {
      // the next n-fragment's B is read from LDS while this one's MFMAs issue
      f16x16 Bn = concat_x(*(const u32x4*)b_chunk(Bs, n0 * 16 + r16, g1), *(const u32x4*)b_chunk(Bs, n0 * 16 + r16, g1 + 16));
#pragma unroll
      for (int n = n0; n < n0 + G; n++) {
        const f16x16 B = Bn;
        if (n + 1 < n0 + G) {
          const int r = (n + 1) * 16 + r16;
          Bn = concat_x(*(const u32x4*)b_chunk(Bs, r, g1), *(const u32x4*)b_chunk(Bs, r, g1 + 16));
        }
#pragma unroll
        for (int f = 0; f < MF; f++) acc[f][n] = smfmac_step<S>(A[f], B, acc[f][n], m[f]);
      }
    }
  }
}

template <int MF, int NF, bool XK>
MOESQ_DEV void mma_superstep_lds(f32x4 (&acc)[MF][NF], const WStage<MF>& w, const uint8_t* Bs, int r16, int c,
                                 int nv) {
  WMeta m[MF];
#pragma unroll
  for (int f = 0; f < MF; f++) m[f] = w_meta(w, f);
  lds_step<0, MF, NF, XK>(acc, w, m, Bs, r16, c, nv);
  lds_step<1, MF, NF, XK>(acc, w, m, Bs, r16, c, nv);
  lds_step<2, MF, NF, XK>(acc, w, m, Bs, r16, c, nv);
  lds_step<3, MF, NF, XK>(acc, w, m, Bs, r16, c, nv);
}

// Dense control: step S in two halves (8-groups g and g + 16), each a decoded A operand per fragment
// against the staged activations, one dense MFMA per (fragment, n-fragment).
template <int S, int MF, int NF>
MOESQ_DEV void dense_lds_step(f32x4 (&acc)[MF][NF], const DWStage<MF>& w, const DMeta (&m)[MF], const uint8_t* Bs,
                              int r16, int c, int nv) {
  constexpr int G = MOESQ_TILE_SKIP_G;
  const int g1 = 8 * (c >> 1) + 2 * S + (c & 1);
#pragma unroll
  for (int h = 0; h < 2; h++) {
    f16x8 A[MF];
#pragma unroll
    for (int f = 0; f < MF; f++) {
      const u32x4 cw = S < 2 ? w.c0[f] : w.c1[f];
      const uint32_t wd = h == 0 ? ((S & 1) ? cw.z : cw.x) : ((S & 1) ? cw.w : cw.y);
      const f16x2 sc = h == 0 ? (S < 2 ? m[f].lo01 : m[f].lo23) : (S < 2 ? m[f].hi01 : m[f].hi23);
      A[f] = dense_frag(wd, sc);
    }
#pragma unroll
    for (int n0 = 0; n0 < NF; n0 += G) {
      if (G == NF || n0 < nv) {
#pragma unroll
        for (int n = n0; n < n0 + G; n++) {
          const f16x8 B = __builtin_bit_cast(f16x8, *(const u32x4*)b_chunk(Bs, n * 16 + r16, g1 + 16 * h));
#pragma unroll
          for (int f = 0; f < MF; f++) acc[f][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[f], B, acc[f][n], 0, 0, 0);
        }
      }
    }
  }
}

template <int MF, int NF>
MOESQ_DEV void dense_superstep_lds(f32x4 (&acc)[MF][NF], const DWStage<MF>& w, const uint8_t* Bs, int r16, int c,
                                   int nv) {
  DMeta m[MF];
#pragma unroll
  for (int f = 0; f < MF; f++) m[f] = dense_meta(w, f);
  dense_lds_step<0, MF, NF>(acc, w, m, Bs, r16, c, nv);
  dense_lds_step<1, MF, NF>(acc, w, m, Bs, r16, c, nv);
  dense_lds_step<2, MF, NF>(acc, w, m, Bs, r16, c, nv);
  dense_lds_step<3, MF, NF>(acc, w, m, Bs, r16, c, nv);
}

// Weight stage of the tiled kernel: the sparse layout or the dense control.
// The sparse weights of a super-step in two halves: half 0 = the packed bytes of steps 0-1 of every
// fragment (8 of the lane's 16 bytes) plus the super-step's index and scale codes, half 1 = the packed
// bytes of steps 2-3. Half 0 of the next super-step is loaded as soon as steps 0-1 have decoded theirs
// (the index and scale codes live on in the decoded metadata), half 1 after steps 2-3: each load has
// half a super-step of MFMAs to arrive in, with no more registers than one full stage.
template <int MF, bool SPLIT>
MOESQ_DEV void load_w_half0(WStage<MF>& st, rsrc_t rw, const WSrc& src, int lane, int ss) {
  const uint32_t go = src.g0 + (uint32_t)ss * kGroupBytes;
  auto pk01 = [&](int f, uint32_t g, int j) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(rw, (int)(g + 1024u * j + 16u * lane), 0, 0);
    st.pk[f].x = v[0];
    st.pk[f].y = v[1];
  };
  if (MF == 4 && !SPLIT) {
#pragma unroll
    for (int j = 0; j < 4; j++) pk01(j, go, j);
    const u32x4 m = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(go + 4096u + 16u * lane), 0, 0));
    st.mk[0] = m.x; st.mk[1] = m.y; st.mk[2] = m.z; st.mk[3] = m.w;
    const auto sc = __builtin_amdgcn_raw_buffer_load_b64(rw, (int)(go + 5120u + 8u * lane), 0, 0);
    st.sw[0] = sc[0]; st.sw[1] = sc[0]; st.sw[2] = sc[1]; st.sw[3] = sc[1];
  } else {
#pragma unroll
    for (int h = 0; h < (MF == 4 ? 2 : 1); h++) {
      const uint32_t g = (h == 0 ? src.g0 : src.g1) + (uint32_t)ss * kGroupBytes;
      const int j = h == 0 ? src.j0 : src.j1;
      pk01(2 * h, g, j);
      pk01(2 * h + 1, g, j + 1);
      const auto m = __builtin_amdgcn_raw_buffer_load_b64(rw, (int)(g + 4096u + 16u * lane + 4u * j), 0, 0);
      st.mk[2 * h] = m[0];
      st.mk[2 * h + 1] = m[1];
      const uint32_t sc = __builtin_amdgcn_raw_buffer_load_b32(rw, (int)(g + 5120u + 8u * lane + 2u * j), 0, 0);
      st.sw[2 * h] = sc;
      st.sw[2 * h + 1] = sc;
    }
  }
}

template <int MF, bool SPLIT>
MOESQ_DEV void load_w_half1(WStage<MF>& st, rsrc_t rw, const WSrc& src, int lane, int ss) {
#pragma unroll
  for (int f = 0; f < MF; f++) {
    const bool second = SPLIT && f >= 2;
    const uint32_t g = (second ? src.g1 : src.g0) + (uint32_t)ss * kGroupBytes;
    const int j = SPLIT ? (second ? src.j1 + f - 2 : src.j0 + f) : src.j0 + f;
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(rw, (int)(g + 1024u * j + 16u * lane + 8u), 0, 0);
    st.pk[f].z = v[0];
    st.pk[f].w = v[1];
  }
}

// Weight stage of the tiled kernel, driven as two halves: load0 / load1 fetch a super-step's halves,
// half<0> runs steps 0-1 (decoding the super-step's metadata first) and half<1> steps 2-3. kLoads1 is
// the number of vector-memory loads load1 issues per wave.
template <int MF, bool MLP, bool DENSE>
struct TWS;
template <int MF, bool MLP>
struct TWS<MF, MLP, false> {
  static constexpr int kLoads1 = MF;
  WStage<MF> w;
  WMeta m[MF];
  MOESQ_DEV void load0(rsrc_t rw, const WSrc& src, int lane, int ss) { load_w_half0<MF, MLP>(w, rw, src, lane, ss); }
  MOESQ_DEV void load1(rsrc_t rw, const WSrc& src, int lane, int ss) { load_w_half1<MF, MLP>(w, rw, src, lane, ss); }
  // the super-step's index words and block scales, from half 0 (before the next B prefetch is issued, so
  // that waiting for half 0 does not also wait for that prefetch)
  MOESQ_DEV void meta() {
#pragma unroll
    for (int f = 0; f < MF; f++) {
      m[f] = w_meta(w, f, true);
      // computed here, not sunk past the prefetch issued next by the scheduler
      asm volatile("" ::"v"(m[f].i02), "v"(m[f].i13), "v"(f16x2_bits(m[f].s01)), "v"(f16x2_bits(m[f].s23)));
    }
  }
  // With the NVFP4 activation codes of the next step (p, loaded at the start of this one), the halves
  // also decode them into the other LDS tile Bn: half of the groups after step 1, the rest after step
  // 2. This VALU work then runs beside the MFMAs that the other wave of the SIMD issues, instead of in
  // a phase of its own in which both waves stage.
  template <int H, int NF, bool XK>
  MOESQ_DEV void half(f32x4 (&acc)[MF][NF], const uint8_t* Bs, int r16, int c, int nv, const PStage* p, uint8_t* Bn,
                      int tok, int qtr) {
    if (H == 0) {
      lds_step<0, MF, NF, XK>(acc, w, m, Bs, r16, c, nv);
      lds_step<1, MF, NF, XK>(acc, w, m, Bs, r16, c, nv);
      if (!XK) stage_p_part<0, 4>(*p, Bn, tok, qtr);
    } else {
      lds_step<2, MF, NF, XK>(acc, w, m, Bs, r16, c, nv);
      if (!XK) stage_p_part<4, 8>(*p, Bn, tok, qtr);
      lds_step<3, MF, NF, XK>(acc, w, m, Bs, r16, c, nv);
    }
  }
};
// The dense control keeps one stage: the whole super-step in half 0, loaded after it.
template <int MF, bool MLP>
struct TWS<MF, MLP, true> {
  static constexpr int kLoads1 = 0;
  DWStage<MF> w;
  MOESQ_DEV void load0(rsrc_t rw, const WSrc& src, int lane, int ss) { load_dw<MF>(w, rw, src.g0, src.j0, lane, ss); }
  MOESQ_DEV void load1(rsrc_t, const WSrc&, int, int) {}
  MOESQ_DEV void meta() {}
  template <int H, int NF, bool XK>
  MOESQ_DEV void half(f32x4 (&acc)[MF][NF], const uint8_t* Bs, int r16, int c, int nv, const PStage*, uint8_t*, int,
                      int) {
    if (H == 0) dense_superstep_lds<MF, NF>(acc, w, Bs, r16, c, nv);
  }
};

// The tile list in LDS: the full token tiles first (exclusive prefix full_pre[0..E] of the per-expert
// counts floor(n_e / kTileTok), E+1 entries), then the experts' partial last tiles, largest first
// (plist[0..P): the experts ordered by the partial tile's 16-token fragment count, descending, then by
// expert; plist[E] = P). Also each expert's first row off_l[e] and row count ne_l[e] (E entries), and its
// epilogue scalars scal_l[3E]: alpha_e of the rows below N/2 [0, E), of the rows from N/2 [E, 2E) (the
// same unless the weights carry split tensor scales; the MLP's gate and up rows), and gamma_h [2E, 3E)
// for the MLP. Read once per workgroup here, so that the per-tile work reads LDS, not global memory (a
// vector load there makes the wave wait for every load in flight, the prefetches included).
// part: LDS scratch of THREADS ints.
template <int THREADS>
MOESQ_DEV void build_tile_prefix(const GemmArgs& a, int32_t* full_pre, int32_t* off_l, int32_t* ne_l, float* scal_l,
                                 int32_t* plist, int32_t* part) {
  constexpr int PER_LANE = THREADS / 64;
  const int tid = threadIdx.x;
  const int E = a.E;
  for (int i = tid; i < E; i += THREADS) {
    int off, ne;
    expert_rows(a, i, off, ne);
    off_l[i] = off;
    ne_l[i] = max(ne, 0);
    const float ga = a.gamma_a[i];
    scal_l[i] = 1.0f / (wscale(a, i, 0) * ga);
    scal_l[E + i] = 1.0f / (wscale(a, i, 1) * ga);
    scal_l[2 * E + i] = a.gamma_h ? a.gamma_h[i] : 1.0f;
  }
  __syncthreads();
  const int per = (E + THREADS - 1) / THREADS;
  const int lo = min(E, tid * per), hi = min(E, lo + per);
  int sum = 0;
  for (int e = lo; e < hi; e++) sum += ne_l[e] / kTileTok;
  part[tid] = sum;
  if (tid >= THREADS - 64) {
    // the last wave lists the partial tiles: one ballot per 64 experts and fragment count
    const int lane = tid & 63;
    int base = 0;
    for (int b = kTileTok / 16; b >= 1; b--) {
      for (int e0 = 0; e0 < E; e0 += 64) {
        const int e = e0 + lane;
        const int r = e < E ? ne_l[e] % kTileTok : 0;
        const bool m = r > 0 && (r + 15) / 16 == b;
        const uint64_t bal = __ballot(m);
        if (m) plist[base + __popcll(bal & ((1ull << lane) - 1ull))] = e;
        base += __popcll(bal);
      }
    }
    if (lane == 0) plist[E] = base;
  }
  __syncthreads();
  if (tid < 64) {  // wave 0 scans the partial sums (PER_LANE per lane)
    int v[PER_LANE], s = 0;
#pragma unroll
    for (int i = 0; i < PER_LANE; i++) { v[i] = part[PER_LANE * tid + i]; s += v[i]; }
    int incl = s;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d);
      if (tid >= d) incl += o;
    }
    int run = incl - s;
#pragma unroll
    for (int i = 0; i < PER_LANE; i++) { part[PER_LANE * tid + i] = run; run += v[i]; }
  }
  __syncthreads();
  int run = part[tid];
  for (int e = lo; e < hi; e++) {
    full_pre[e] = run;
    run += ne_l[e] / kTileTok;
  }
  if (hi == E && lo < hi) full_pre[E] = run;
  __syncthreads();
}

// One output tile of the persistent schedule and the per-tile operand addressing (all wave uniform).
struct TileEpi {  // what the MMA and the epilogue of a tile read
  int e, off, ne, tb, rb, nv;
  float alpha;
};
template <int MF>
struct TileCtx : TileEpi {
  rsrc_t rw;          // expert's weights (kernel layout)
  WSrc src;           // the wave's m-fragments in the kernel layout
  rsrc_t rq, rs;      // expert's activation codes / scales (FP4 path) or f16 activations (rq, f16 path)
};

// Tile t of the list: the full token tiles ordered expert -> token tile -> row block (row block
// fastest: workgroups of one XCD that run neighbouring tiles share the activation tile in L2), then the
// partial last tiles in plist order, each with its RB row blocks.
template <int MF, bool MLP, bool XK, bool DENSE>
MOESQ_DEV TileCtx<MF> make_tile(const GemmArgs& a, const int32_t* full_pre, const int32_t* off_l, const int32_t* ne_l,
                                const float* scal_l, const int32_t* plist, const uint16_t* lut, int RB, int t, int w) {
  TileCtx<MF> c;
  const int TA = __builtin_amdgcn_readfirstlane(full_pre[a.E]) * RB;
  if (t < TA) {
    const int u = t / RB;  // full token tile u, row block t % RB
    if (lut) {
      c.e = __builtin_amdgcn_readfirstlane((int)lut[u]);
    } else {
      int lo = 0, hi = a.E - 1;  // largest e with full_pre[e] * RB <= t
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (full_pre[mid] * RB <= t) lo = mid; else hi = mid - 1;
      }
      c.e = __builtin_amdgcn_readfirstlane(lo);
    }
    c.tb = __builtin_amdgcn_readfirstlane((u - full_pre[c.e]) * kTileTok);
    c.rb = __builtin_amdgcn_readfirstlane(t - u * RB);
  } else {
    const int u = t - TA;
    c.e = __builtin_amdgcn_readfirstlane(plist[u / RB]);
    c.tb = __builtin_amdgcn_readfirstlane((ne_l[c.e] / kTileTok) * kTileTok);
    c.rb = __builtin_amdgcn_readfirstlane(u % RB);
  }
  c.off = __builtin_amdgcn_readfirstlane(off_l[c.e]);
  c.ne = __builtin_amdgcn_readfirstlane(ne_l[c.e]);
  c.nv = min(kTileNF, (c.ne - c.tb + 15) / 16);
  const int K = a.K, N = a.N, nss = K / 256;
  const uint32_t ekl = DENSE ? expert_dense_bytes(N, K) : expert_kl_bytes(N, K);
  c.rw = make_rsrc(a.kl + (size_t)c.e * ekl, ekl);
  if (MLP) {
    const int rg = (c.rb * 256 + 32 * w) / 16, ru = (N / 2 + c.rb * 256 + 32 * w) / 16;  // gate / up 16-row blocks
    c.src.g0 = __builtin_amdgcn_readfirstlane((uint32_t)(rg / 4) * (uint32_t)nss * kGroupBytes);
    c.src.j0 = __builtin_amdgcn_readfirstlane(rg % 4);
    c.src.g1 = __builtin_amdgcn_readfirstlane((uint32_t)(ru / 4) * (uint32_t)nss * kGroupBytes);
    c.src.j1 = __builtin_amdgcn_readfirstlane(ru % 4);
  } else {
    const int rbf = min(c.rb * 512 + 64 * w, N - 64) / 16;
    c.src.g0 = __builtin_amdgcn_readfirstlane((uint32_t)(rbf / 4) * (uint32_t)nss *
                                              (uint32_t)(DENSE ? kDenseUnitBytes : kGroupBytes));
    c.src.j0 = 0;
    c.src.g1 = 0;
    c.src.j1 = 0;
  }
  // alpha_e: the MLP tile's gate and up rows take the two tensor scales, a plain wave its row half's
  const int half = MLP ? 0 : (min(c.rb * 512 + 64 * w, N - 64) >= N / 2);
  c.alpha = scal_l[half * a.E + c.e];
  if (XK) {
    c.rq = make_rsrc((const uint8_t*)a.xk + (size_t)c.off * K * 2, (uint32_t)c.ne * K * 2);
    c.rs = c.rq;
  } else {
    c.rq = make_rsrc(a.q + (size_t)c.off * (K / 2), (uint32_t)c.ne * (K / 2));
    c.rs = make_rsrc(a.s + (size_t)c.off * (K / 32), (uint32_t)c.ne * (K / 32));
  }
  return c;
}

// Per-lane parts of the activation addresses. FP4 path: token = lane + 64 (w & 1), quarter w / 2.
// f16 path: the wave's 8 direct-to-LDS chunk loads j = 0..7 fill chunks q = (8 w + j) * 64 + lane of
// the swizzled tile, chunk q holding token r = q / 32 = 16 w + 2 j + h (h = lane / 32), group
// (q % 32) ^ (r % 32). Its source offset r 2K + 16 (pq ^ (r % 32)) (pq = lane % 32) splits into this
// lane's part xl = h 2K + 16 (pq ^ 16 (w & 1) ^ h), xor 32 j, plus the uniform (16 w + 2 j) 2K (for
// K % 256 == 0 the bit fields do not overlap), so each load costs one xor and one add.
struct BAddr {
  uint32_t tok, qtr, xl;
};

MOESQ_DEV BAddr make_baddr(int w, int lane, int K) {
  BAddr b;
  b.tok = (uint32_t)(lane + 64 * (w & 1));
  b.qtr = (uint32_t)(w >> 1);
  const uint32_t h = (uint32_t)lane >> 5, pq = (uint32_t)lane & 31u;
  b.xl = h * (uint32_t)(2 * K) + 16u * (pq ^ (16u * (uint32_t)(w & 1)) ^ h);
  return b;
}

// Issue the activation operand of super-step ss of tile c: f16 path = 8 direct-to-LDS loads per wave
// (wave w fills chunks [512 w, 512 w + 512) of the swizzled tile); FP4 path = register loads.
template <int MF, bool XK>
MOESQ_DEV void issue_b(const TileCtx<MF>& c, int ss, uint8_t* Bs, PStage& p, int w, int lane, const BAddr& ba, int K) {
  if (XK) {
    const uint32_t ub = ((uint32_t)c.tb + 16u * (uint32_t)w) * (uint32_t)(2 * K) + 512u * ss;
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const uint32_t vo = (ba.xl ^ (32u * (uint32_t)j)) + (ub + (uint32_t)j * (uint32_t)(4 * K));
#if defined(__HIP_DEVICE_COMPILE__)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rq, (__attribute__((address_space(3))) void*)(Bs + (8 * w + j) * 1024),
                                               16, (int)vo, 0, 0, 0);
#else
      (void)vo;
#endif
    }
  } else {
    const uint32_t t = (uint32_t)c.tb + ba.tok;
    load_p(p, c.rq, c.rs, t * (K / 2) + 32u * ba.qtr, t * (K / 32) + 2u * ba.qtr, ss);
  }
}

MOESQ_DEV void stage_b(const PStage& p, uint8_t* Bs, const BAddr& ba) { stage_p(p, Bs, (int)ba.tok, (int)ba.qtr); }

// Epilogue of a finished tile.
template <int MF, int NF, int MLP>
MOESQ_DEV void tile_epilogue(const GemmArgs& a, const TileEpi& c, f32x4 (&acc)[MF][NF], int w, int r16, int cc,
                             const float* scal_l) {
  const int N = a.N;
  const float alpha = c.alpha;
  if (!MLP) {
    const int n0 = c.rb * 512 + 64 * w;
    if (n0 >= N) return;
    // Lane (r16, cc) holds columns 16 f + 4 cc .. + 3 of token r16 for every fragment f. A permlane16
    // swap between lane rows cc = 2i and 2i + 1 gives each lane 8 consecutive columns of one fragment
    // (even cc: fragment f, columns 16 f + 4 cc ..; odd cc: fragment f + 1, columns 16 (f+1) + 4 (cc-1)
    // ..), so every store writes 16 (bf16) or 32 (fp32) contiguous bytes.
    const int odd = cc & 1;
#pragma unroll
    for (int n = 0; n < NF; n++) {
      const int tok = c.tb + n * 16 + r16;
      const bool tv = tok < c.ne;
      const int64_t rowo = (int64_t)(c.off + tok) * N + n0;
#pragma unroll
      for (int f = 0; f < MF; f += 2) {
        const int col = odd ? 16 * (f + 1) + 4 * (cc - 1) : 16 * f + 4 * cc;
        if (a.y_bf16) {
          const bf16x2 x0 = __builtin_convertvector((f32x2){acc[f][n].x * alpha, acc[f][n].y * alpha}, bf16x2);
          const bf16x2 x1 = __builtin_convertvector((f32x2){acc[f][n].z * alpha, acc[f][n].w * alpha}, bf16x2);
          const bf16x2 y0 = __builtin_convertvector((f32x2){acc[f + 1][n].x * alpha, acc[f + 1][n].y * alpha}, bf16x2);
          const bf16x2 y1 = __builtin_convertvector((f32x2){acc[f + 1][n].z * alpha, acc[f + 1][n].w * alpha}, bf16x2);
          const auto s0 = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x0), __builtin_bit_cast(uint32_t, y0),
                                                           false, false);
          const auto s1 = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x1), __builtin_bit_cast(uint32_t, y1),
                                                           false, false);
          if (tv) *(u32x4*)((uint16_t*)a.y + rowo + col) = (u32x4){s0[0], s1[0], s0[1], s1[1]};
        } else {
          uint32_t xv[4], yv[4];
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[f][n][i] * alpha),
                                                             __float_as_uint(acc[f + 1][n][i] * alpha), false, false);
            xv[i] = sw[0];
            yv[i] = sw[1];
          }
          if (tv) {
            u32x4* dst = (u32x4*)((float*)a.y + rowo + col);
            dst[0] = (u32x4){xv[0], xv[1], xv[2], xv[3]};
            dst[1] = (u32x4){yv[0], yv[1], yv[2], yv[3]};
          }
        }
      }
    }
    return;
  }
  const int ib = c.rb * 256 + 32 * w;  // first intermediate column of this wave (one 32-block)
  const float alpha_u = scal_l[a.E + c.e];  // the up rows' alpha_e
  const float gh = scal_l[2 * a.E + c.e];
  float amx = 0.0f;
#pragma unroll
  for (int n = 0; n < NF; n++) {
    if (n >= c.nv) break;
    const int tok = c.tb + n * 16 + r16;
    amx = __builtin_fmaxf(amx, mlp_epilogue_token<MLP>(a, c.off + tok, tok < c.ne, ib, cc, alpha, alpha_u, gh,
                                                       acc[0][n], acc[1][n], acc[2][n], acc[3][n]));
  }
  if (MLP == kEpiCalib) calib_amax_commit(a.amax_h, c.e, amx);
}

// Persistent tiled kernel, one 8-wave workgroup per CU. The grid holds 8*J workgroups; the tile list
// (full token tiles, then the partial ones, largest first) is dealt to the XCDs in groups of J
// consecutive tiles, slot j of XCD x handling tiles x J + j, + 8 J, ... The super-steps of all the workgroup's tiles form one
// pipeline: while step i computes, the activations (LDS) of step i+1 -- possibly the first step of
// the next tile -- are in flight, and its weights are loaded into the one register stage as soon as
// step i's MFMAs have read it; one barrier per step. (One weight stage measured as fast as two; the
// registers it frees hold the B read-ahead of the sparse kernels and the dense control's larger stage.)
template <int MLP, bool XK, bool DENSE = false>
__global__ __launch_bounds__(kTileThreads, 1) void gemm_tile_kernel(GemmArgs a) {
  constexpr int MF = 4, NF = kTileNF;
  constexpr int BBYTES = kBTileBytes;
  extern __shared__ __align__(16) uint8_t dyn[];
  __shared__ int32_t part[kTileThreads];
  const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, cc = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint8_t* Bs0 = dyn;                                    // two activation tiles
  uint8_t* Bs1 = dyn + BBYTES;
  int32_t* full_pre = (int32_t*)(dyn + 2 * BBYTES);      // [E+1]
  int32_t* off_l = full_pre + a.E + 1;                   // [E+1]
  int32_t* ne_l = off_l + a.E + 1;                       // [E]
  float* scal_l = (float*)(ne_l + a.E);                  // [3E]
  int32_t* plist = (int32_t*)(scal_l + 3 * a.E);         // [E+1]
  build_tile_prefix<kTileThreads>(a, full_pre, off_l, ne_l, scal_l, plist, part);
  // the expert of every full token tile, when the table fits (lut_cap entries): one LDS read per tile
  // switch instead of a binary search over full_pre
  const uint16_t* lut = nullptr;
  if (full_pre[a.E] <= a.lut_cap) {
    uint16_t* l = (uint16_t*)(plist + a.E + 1);
    for (int e = threadIdx.x; e < a.E; e += kTileThreads)
      for (int u = full_pre[e]; u < full_pre[e + 1]; u++) l[u] = (uint16_t)e;
    __syncthreads();
    lut = l;
  }
  const int K = a.K, nss = K / 256;
  const int RB = MLP ? a.N / 512 : (a.N + 511) / 512;   // MLP: 256 gate + 256 up rows per tile
  const int T = (full_pre[a.E] + plist[a.E]) * RB;
  // groups of J consecutive tiles are dealt to the 8 XCDs in turn (workgroup x + 8 j runs on XCD x):
  // slot j of XCD x takes tiles (8 k + x) J + j, k = 0, 1, ... Neighbouring tiles still run side by side
  // on one XCD, and every XCD gets a share of the full tiles and of the cheaper partial tiles at the end.
  const int J = gridDim.x >> 3, x = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int tend = T;
  int t = x * J + j;
  if (t >= tend) return;
  const BAddr ba = make_baddr(w, lane, K);

  f32x4 acc[MF][NF];
#pragma unroll
  for (int f = 0; f < MF; f++)
#pragma unroll
    for (int n = 0; n < NF; n++) acc[f][n] = (f32x4){0.f, 0.f, 0.f, 0.f};

  constexpr bool kMlp = MLP != kEpiPlain;
  // nxt: the tile of the step whose operands are loaded next (the current tile until its last step);
  // cur: the MMA and epilogue fields of the step being computed
  TileCtx<MF> nxt = make_tile<MF, kMlp, XK, DENSE>(a, full_pre, off_l, ne_l, scal_l, plist, lut, RB, t, w);
  TileEpi cur = nxt;
  TWS<MF, kMlp, DENSE> wc;
  PStage p;
  wc.load0(nxt.rw, nxt.src, lane, 0);
  wc.load1(nxt.rw, nxt.src, lane, 0);
  issue_b<MF, XK>(nxt, 0, Bs0, p, w, lane, ba, K);
  if (!XK) stage_b(p, Bs0, ba);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int ss = 0;
  uint32_t bsel = 0;  // which LDS tile holds the current step
  while (true) {
    // coordinates of the next step
    int ss_n = ss + 1, t_n = t;
    if (ss_n == nss) {
      ss_n = 0;
      t_n = t + 8 * J;
    }
    const bool has_n = t_n < tend;
    if (has_n && ss_n == 0) nxt = make_tile<MF, kMlp, XK, DENSE>(a, full_pre, off_l, ne_l, scal_l, plist, lut, RB, t_n, w);
    uint8_t* Bc = bsel ? Bs1 : Bs0;
    uint8_t* Bn = bsel ? Bs0 : Bs1;
    // The prefetches below are issued on every super-step, the last one too (there they read the current
    // tile's first super-step again: in range, and never used), so that no branch around them leaves the
    // compiler's wait bookkeeping unsure of how many loads are in flight.
    wc.meta();
    issue_b<MF, XK>(nxt, ss_n, Bn, p, w, lane, ba, K);
    wc.template half<0, NF, XK>(acc, Bc, r16, cc, cur.nv, &p, Bn, (int)ba.tok, (int)ba.qtr);
    wc.load0(nxt.rw, nxt.src, lane, ss_n);  // half 0 of the next super-step, its registers read
    wc.template half<1, NF, XK>(acc, Bc, r16, cc, cur.nv, &p, Bn, (int)ba.tok, (int)ba.qtr);
    const bool tile_end = ss == nss - 1;
    if (tile_end) {
      tile_epilogue<MF, NF, MLP>(a, cur, acc, w, r16, cc, scal_l);
#pragma unroll
      for (int f = 0; f < MF; f++)
#pragma unroll
        for (int n = 0; n < NF; n++) acc[f][n] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
    wc.load1(nxt.rw, nxt.src, lane, ss_n);
    if (!XK && DENSE) stage_b(p, Bn, ba);  // the sparse weight stage decodes it inside its halves
    if (XK) {
      // the direct-to-LDS loads of the next step (issued first) must have landed; the kLoads1 weight
      // loads issued last may stay in flight. Loads complete in issue order, so waiting until at most
      // kLoads1 vector-memory operations are outstanding is enough; after an epilogue (stores in flight,
      // which need not complete in order with the loads) everything is waited for.
      // (The direct-to-LDS data is in LDS once its load is counted complete, and every wave's LDS reads
      // of the current tile completed before it got here: a bare barrier suffices.)
      if (tile_end || !has_n) __builtin_amdgcn_s_waitcnt(0);
      else __builtin_amdgcn_s_waitcnt(vmcnt_only(TWS<MF, kMlp, DENSE>::kLoads1));
      bare_barrier();
    } else {
      lds_barrier();  // epilogue stores may still be in flight
    }
    if (!has_n) break;
    cur = nxt;
    t = t_n;
    ss = ss_n;
    bsel ^= 1u;
  }
}

static size_t tile_tables_bytes(int E) { return 2 * (size_t)kBTileBytes + (3 * (size_t)(E + 1) + 4 * (size_t)E) * 4; }
// Entries of the full-token-tile table: one per possible full tile (rows / kTileTok), as far as the LDS
// left beside the tile tables and the kernel's static LDS holds them (0: the kernel searches full_pre).
static int tile_lut_cap(int E, int64_t rows) {
  const int64_t room = (160 * 1024 - (int64_t)tile_tables_bytes(E) - kTileThreads * 4) / 2;
  return (int)std::max<int64_t>(0, std::min<int64_t>(rows / kTileTok, room & ~(int64_t)1));
}
static size_t tile_lds_bytes(int E, int lut_cap) { return tile_tables_bytes(E) + (size_t)(lut_cap + 1) / 2 * 4; }
// the tile tables of the largest expert count the GEMM calls accept fit one workgroup's 160 KiB of LDS
static_assert(2 * kBTileBytes + (3 * (kMaxExpertsGemm + 1) + 4 * kMaxExpertsGemm) * 4 + kTileThreads * 4 <= 160 * 1024,
              "tile tables for kMaxExpertsGemm experts exceed the LDS");

static int device_cu_count() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cus[dev] = v;
  }
  return cus[dev];
}

// Decode variants (MF, KS, RG); the default is picked by measurement, the environment variable
// MOESQ_DECODE_VARIANT overrides it for tuning.
static int decode_variant_default() {
  static int v = -1;
  if (v < 0) {
    const char* e = getenv("MOESQ_DECODE_VARIANT");
    v = e ? atoi(e) : 0;
    if (v < 0 || v > 7) v = 0;
  }
  return v;
}

template <int MF, int KS, int RG, bool DENSE = false>
static bool launch_decode(hipStream_t st, const GemmArgs& a) {
  constexpr int rows = 16 * MF * RG;
  if (a.N % rows != 0) return false;
  if (a.xk)
    hipLaunchKernelGGL((gemm_decode_kernel<MF, KS, RG, true, DENSE>), dim3(a.N / rows, a.E), dim3(64 * KS * RG), 0, st,
                       a);
  else
    hipLaunchKernelGGL((gemm_decode_kernel<MF, KS, RG, false, DENSE>), dim3(a.N / rows, a.E), dim3(64 * KS * RG), 0,
                       st, a);
  return true;
}

int launch_gemm_variant(hipStream_t st, const GemmArgs& a, int64_t rows, int variant) {
  if (rows == 0) return MOESQ_OK;
  // the gate_up GEMM of the MLP: its epilogue form
  const int epi = a.amax_h ? kEpiCalib : (a.dump || a.hdump) ? kEpiMlpDump : a.gamma_h ? kEpiMlp : kEpiPlain;
  if (variant == 0 && epi != kEpiPlain) {
    // MLP gate_up by weight streaming: 32 gate + 32 up rows per workgroup
    const dim3 grid(a.N / 64, a.E), block(256);
    if (a.xk) {
      if (epi == kEpiMlp) hipLaunchKernelGGL((gemm_decode_kernel<4, 4, 1, true, false, kEpiMlp>), grid, block, 0, st, a);
      else if (epi == kEpiMlpDump)
        hipLaunchKernelGGL((gemm_decode_kernel<4, 4, 1, true, false, kEpiMlpDump>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((gemm_decode_kernel<4, 4, 1, true, false, kEpiCalib>), grid, block, 0, st, a);
    } else {
      if (epi == kEpiMlp) hipLaunchKernelGGL((gemm_decode_kernel<4, 4, 1, false, false, kEpiMlp>), grid, block, 0, st, a);
      else if (epi == kEpiMlpDump)
        hipLaunchKernelGGL((gemm_decode_kernel<4, 4, 1, false, false, kEpiMlpDump>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((gemm_decode_kernel<4, 4, 1, false, false, kEpiCalib>), grid, block, 0, st, a);
    }
  } else if (variant == 0) {
    bool ok = false;
    switch (decode_variant_default()) {
      case 2: ok = launch_decode<4, 1, 4>(st, a); break;
      case 3: ok = launch_decode<4, 8, 1>(st, a); break;
      case 4: ok = launch_decode<2, 8, 1>(st, a); break;
      case 5: ok = launch_decode<2, 4, 1>(st, a); break;
      case 6: ok = launch_decode<4, 2, 2>(st, a); break;
      case 7: ok = launch_decode<2, 4, 2>(st, a); break;
      default: break;
    }
    if (!ok) launch_decode<4, 4, 1>(st, a);  // N % 64 == 0 always holds
  } else {
    // persistent grid: one 8-wave workgroup per CU, a multiple of the 8 XCDs
    const int grid = 8 * ((device_cu_count() + 7) / 8);
    const bool xk = a.xk != nullptr;
    GemmArgs at = a;
    at.lut_cap = tile_lut_cap(a.E, rows);
    const size_t lds = tile_lds_bytes(a.E, at.lut_cap);
    const dim3 g(grid), b(kTileThreads);
    if (xk) {
      switch (epi) {
        case kEpiMlp: hipLaunchKernelGGL((gemm_tile_kernel<kEpiMlp, true>), g, b, lds, st, at); break;
        case kEpiMlpDump: hipLaunchKernelGGL((gemm_tile_kernel<kEpiMlpDump, true>), g, b, lds, st, at); break;
        case kEpiCalib: hipLaunchKernelGGL((gemm_tile_kernel<kEpiCalib, true>), g, b, lds, st, at); break;
        default: hipLaunchKernelGGL((gemm_tile_kernel<kEpiPlain, true>), g, b, lds, st, at); break;
      }
    } else {
      switch (epi) {
        case kEpiMlp: hipLaunchKernelGGL((gemm_tile_kernel<kEpiMlp, false>), g, b, lds, st, at); break;
        case kEpiMlpDump: hipLaunchKernelGGL((gemm_tile_kernel<kEpiMlpDump, false>), g, b, lds, st, at); break;
        case kEpiCalib: hipLaunchKernelGGL((gemm_tile_kernel<kEpiCalib, false>), g, b, lds, st, at); break;
        default: hipLaunchKernelGGL((gemm_tile_kernel<kEpiPlain, false>), g, b, lds, st, at); break;
      }
    }
  }
  return hipGetLastError() == hipSuccess ? MOESQ_OK : MOESQ_ERR_HIP;
}

// Dense control: variant 0 = weight streaming, otherwise the tiled kernel (no MLP epilogue).
int launch_dense_gemm(hipStream_t st, const GemmArgs& a, int64_t rows, int variant) {
  if (rows == 0) return MOESQ_OK;
  if (variant == 0) {
    launch_decode<4, 4, 1, true>(st, a);
  } else {
    const int grid = 8 * ((device_cu_count() + 7) / 8);
    GemmArgs at = a;
    at.lut_cap = tile_lut_cap(a.E, rows);
    const size_t lds = tile_lds_bytes(a.E, at.lut_cap);
    if (a.xk) hipLaunchKernelGGL((gemm_tile_kernel<kEpiPlain, true, true>), dim3(grid), dim3(kTileThreads), lds, st, at);
    else hipLaunchKernelGGL((gemm_tile_kernel<kEpiPlain, false, true>), dim3(grid), dim3(kTileThreads), lds, st, at);
  }
  return hipGetLastError() == hipSuccess ? MOESQ_OK : MOESQ_ERR_HIP;
}

// gamma_h[e] = Eq. 5 of the expert's amax(h) (float bits); 1 for an expert without tokens (amax 0).
__global__ void calib_gamma_kernel(const uint32_t* __restrict__ amax_bits, float* __restrict__ gamma_h, int32_t E) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e < E) gamma_h[e] = global_scale_from_amax(__uint_as_float(amax_bits[e]));
}

__global__ void zero_u32_kernel(uint32_t* p, int32_t n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

int launch_calibrate_h(hipStream_t st, GemmArgs a, int64_t rows, int variant, uint32_t* amax_bits, float* gamma_h) {
  const unsigned nb = (unsigned)((a.E + 255) / 256);
  // a fill kernel, not a memset: the call may be captured in a graph
  hipLaunchKernelGGL(zero_u32_kernel, dim3(nb), dim3(256), 0, st, amax_bits, a.E);
  a.gamma_h = nullptr;
  a.amax_h = amax_bits;
  a.h_q = nullptr; a.h_s = nullptr; a.h_k = nullptr;
  int rc = launch_gemm_variant(st, a, rows, variant);
  if (rc != MOESQ_OK) return rc;
  hipLaunchKernelGGL(calib_gamma_kernel, dim3(nb), dim3(256), 0, st, amax_bits, gamma_h, a.E);
  return hipGetLastError() == hipSuccess ? MOESQ_OK : MOESQ_ERR_HIP;
}

int launch_gemm(hipStream_t st, const GemmArgs& a, int64_t rows) {
  // Few tokens per expert: weight streaming; otherwise the tiled kernel. The MLP epilogue lives in
  // the tiled kernel.
  const bool decode = a.gamma_h == nullptr && rows <= (int64_t)16 * a.E;
  return launch_gemm_variant(st, a, rows, decode ? 0 : 1);
}

}  // namespace moesq
