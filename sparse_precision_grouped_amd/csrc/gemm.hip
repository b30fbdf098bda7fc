// Grouped sparse NVFP4 GEMM for gfx950 (paper Section 2 and Section 3.4 "Grouped sparse GEMM
// execution": Y_e^T = W_e X_e^T per expert in one launch, the sparse weights on the left operand,
// block scales applied inside the product, alpha_e = 1/(gamma_w,e gamma_a,e) on the fp32
// accumulator; Appendix D.1: token counts read on the device, each expert gets ceil(N_e/T_N)
// token tiles, only the last tile of an expert touches padding).
//
// MI355X design:
//  - The paired-4:8 weights feed v_smfmac_f32_16x16x64_f16 (2:4 structured-sparse MFMA) after an
//    even/odd de-interleave of every 8-group, which turns each of the six paired patterns into a
//    valid 2:4 pattern; the pair mask becomes the sparse index operand (an LDS table, mask byte ->
//    16-bit index word). E2M1 codes are expanded with the gfx950 FP4->f16 convert and multiplied
//    by the UE4M3 block scale in f16: e2m1 * e4m3 has at most 6 significant bits, so every operand
//    is exact and the only rounding is the fp32 accumulation.
//  - K is traversed in super-steps of 256: lane (row r, chunk c) of an A fragment reads 16
//    contiguous packed bytes, 4 mask bytes and 2 scale bytes of one row (one 128-bit load plus two
//    small loads straight from the pair-bitmask storage, no repacking), and covers K
//    [64c + 16s, +16) at step s. The activation (B) operand follows the same K mapping.
//  - Decode (few tokens per expert): weight streaming. One workgroup = 64 weight rows of one
//    expert; its 4 waves split K and reduce through LDS in a fixed order (deterministic).
//  - Prefill: 256 x 64 tiles (4 waves x 4 m-fragments x 16 rows, 4 n-fragments x 16 tokens);
//    the activation tile of each super-step is decoded once into LDS (f16, de-interleaved) and
//    shared by the four waves; the weights go from global memory straight to registers.
//  - The gate_up GEMM of the MLP fuses SwiGLU and the NVFP4 requantization of h in its epilogue:
//    a wave owns the gate rows and the matching up rows of 32 intermediate columns, which is one
//    32-element scale block per token.
#include "common.h"
#include "launch.h"

namespace moesq {

// LDS tables: mask byte (two pair nibbles) -> 16-bit sparse index word; UE4M3 code -> f16x2 (v, v).
struct DecodeTables {
  uint16_t idx[256];
  uint32_t scl[256];
};

MOESQ_DEV void init_tables(DecodeTables& t) {
  for (int i = threadIdx.x; i < 256; i += blockDim.x) {
    t.idx[i] = (uint16_t)pair_index_word((uint32_t)i);
    t.scl[i] = e4m3_f16x2_bits((uint32_t)i);
  }
}

MOESQ_DEV f16x16 concat_x(u32x4 lo, u32x4 hi) {
  typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
  u32x8 v;
  v.s0 = lo.x; v.s1 = lo.y; v.s2 = lo.z; v.s3 = lo.w;
  v.s4 = hi.x; v.s5 = hi.y; v.s6 = hi.z; v.s7 = hi.w;
  return __builtin_bit_cast(f16x16, v);
}

MOESQ_DEV void store4(void* y, int64_t off, f32x4 v, float alpha, int bf16) {
  if (bf16) {
    uint2 o;
    o.x = f32_to_bf16_bits(v.x * alpha) | (f32_to_bf16_bits(v.y * alpha) << 16);
    o.y = f32_to_bf16_bits(v.z * alpha) | (f32_to_bf16_bits(v.w * alpha) << 16);
    *(uint2*)((uint16_t*)y + off) = o;
  } else {
    float4 o;
    o.x = v.x * alpha; o.y = v.y * alpha; o.z = v.z * alpha; o.w = v.w * alpha;
    *(float4*)((float*)y + off) = o;
  }
}

// ============================================================================ decode kernel =====
// grid (N / (16*MF), E), 256 threads. Wave w takes super-steps ss = w, w+4, ...; the 4 partial
// accumulators are summed in wave order. Experts with more than 16 tokens loop over 16-token
// blocks re-reading their weights (cache-resident after the first pass).
template <int MF>
__global__ __launch_bounds__(256) void gemm_decode_kernel(GemmArgs a) {
  __shared__ DecodeTables tab;
  __shared__ f32x4 red[4][MF][64];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r16 = lane & 15, c = lane >> 4;
  const int e = blockIdx.y;
  init_tables(tab);
  const int off = a.offsets[e];
  const int ne = a.offsets[e + 1] - off;
  __syncthreads();
  if (ne <= 0) return;
  const int K = a.K, nss = K / 256;
  const int n0 = blockIdx.x * (16 * MF);
  const int64_t row0 = (int64_t)e * a.N + n0 + r16;
  const uint8_t* P = a.packed + row0 * (K / 4) + 16 * c;
  const uint8_t* M = a.mask + row0 * (K / 16) + 4 * c;
  const uint8_t* S = a.wscale + row0 * (K / 32) + 2 * c;
  const int64_t fP = 16 * (int64_t)(K / 4), fM = 16 * (int64_t)(K / 16), fS = 16 * (int64_t)(K / 32);
  const float alpha = 1.0f / (a.gscale[e] * a.gamma_a[e]);
  const int gB = 32 * (c >> 1) + 4 * (c & 1);  // byte offset of the lane's first activation group (step 0)
  for (int tb = 0; tb < ne; tb += 16) {
    f32x4 acc[MF];
#pragma unroll
    for (int f = 0; f < MF; f++) acc[f] = (f32x4){0.f, 0.f, 0.f, 0.f};
    const int tok = tb + r16;
    const bool tv = tok < ne;
    const uint8_t* Q = a.q + (int64_t)(off + (tv ? tok : 0)) * (K / 2) + gB;
    const uint8_t* SA = a.s + (int64_t)(off + (tv ? tok : 0)) * (K / 32) + 2 * (c >> 1);
    for (int ss = w; ss < nss; ss += 4) {
      u32x4 pk[MF];
      uint32_t mk[MF], sw[MF];
#pragma unroll
      for (int f = 0; f < MF; f++) {
        pk[f] = *(const u32x4*)(P + f * fP + 64 * ss);
        mk[f] = *(const uint32_t*)(M + f * fM + 16 * ss);
        sw[f] = *(const uint16_t*)(S + f * fS + 8 * ss);
      }
      uint32_t bc[8];
      uint32_t bs0 = 0u, bs1 = 0u;
      if (tv) {
#pragma unroll
        for (int s = 0; s < 4; s++) {
          bc[2 * s] = *(const uint32_t*)(Q + 128 * ss + 8 * s);
          bc[2 * s + 1] = *(const uint32_t*)(Q + 128 * ss + 64 + 8 * s);
        }
        bs0 = *(const uint16_t*)(SA + 8 * ss);
        bs1 = *(const uint16_t*)(SA + 8 * ss + 4);
      } else {
#pragma unroll
        for (int i = 0; i < 8; i++) bc[i] = 0u;
      }
#pragma unroll
      for (int s = 0; s < 4; s++) {
        const f16x2 sb1 = bits_f16x2(tab.scl[(bs0 >> (8 * (s >> 1))) & 0xFFu]);
        const f16x2 sb2 = bits_f16x2(tab.scl[(bs1 >> (8 * (s >> 1))) & 0xFFu]);
        const f16x16 B = concat_x(decode_x_group(bc[2 * s], sb1), decode_x_group(bc[2 * s + 1], sb2));
#pragma unroll
        for (int f = 0; f < MF; f++) {
          const f16x2 scw = bits_f16x2(tab.scl[(sw[f] >> (8 * (s >> 1))) & 0xFFu]);
          const uint32_t wd = s == 0 ? pk[f].x : s == 1 ? pk[f].y : s == 2 ? pk[f].z : pk[f].w;
          const f16x8 A = decode_w_step(wd, scw);
          const int idx = tab.idx[(mk[f] >> (8 * s)) & 0xFFu];
          acc[f] = __builtin_amdgcn_smfmac_f32_16x16x64_f16(A, B, acc[f], idx, 0, 0);
        }
      }
    }
#pragma unroll
    for (int f = 0; f < MF; f++) red[w][f][lane] = acc[f];
    __syncthreads();
    for (int f = w; f < MF; f += 4) {
      f32x4 sum = red[0][f][lane];
      sum = sum + red[1][f][lane];
      sum = sum + red[2][f][lane];
      sum = sum + red[3][f][lane];
      if (tv) store4(a.y, (int64_t)(off + tok) * a.N + n0 + 16 * f + 4 * c, sum, alpha, a.y_bf16);
    }
    __syncthreads();
  }
}

// =========================================================================== prefill kernel =====
constexpr int kPfTokens = 64;                 // T_N
constexpr int kPfGroups = 32;                 // 8-element groups per 256-K super-step
constexpr int kPfRowBytes = kPfGroups * 16 + 16;  // decoded f16 groups of one token (+ pad)

// Tile table: tile_pre[e] = sum over e' < e of ceil(n_e' / 64), built in LDS by every workgroup.
MOESQ_DEV void build_tile_prefix(const int32_t* __restrict__ offsets, int E, int32_t* tile_pre, int32_t* part) {
  const int tid = threadIdx.x;
  const int per = (E + 255) / 256;
  const int lo = min(E, tid * per), hi = min(E, lo + per);
  int sum = 0;
  for (int e = lo; e < hi; e++) sum += (offsets[e + 1] - offsets[e] + kPfTokens - 1) / kPfTokens;
  part[tid] = sum;
  __syncthreads();
  if (tid < 64) {  // wave 0 scans the 256 partial sums (4 per lane)
    int v[4], s = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) { v[i] = part[4 * tid + i]; s += v[i]; }
    int incl = s;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d);
      if (tid >= d) incl += o;
    }
    int run = incl - s;
#pragma unroll
    for (int i = 0; i < 4; i++) { part[4 * tid + i] = run; run += v[i]; }
  }
  __syncthreads();
  int run = part[tid];
  for (int e = lo; e < hi; e++) {
    tile_pre[e] = run;
    run += (offsets[e + 1] - offsets[e] + kPfTokens - 1) / kPfTokens;
  }
  if (hi == E && lo < hi) tile_pre[E] = run;
  if (E == 0 && tid == 0) tile_pre[0] = 0;
  __syncthreads();
}

template <bool MLP>
__global__ __launch_bounds__(256) void gemm_prefill_kernel(GemmArgs a) {
  constexpr int MF = 4, NF = 4;
  extern __shared__ __align__(16) uint8_t dyn[];
  __shared__ DecodeTables tab;
  __shared__ int32_t part[256];
  __shared__ int32_t tinfo[2];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r16 = lane & 15, c = lane >> 4;
  int32_t* tile_pre = (int32_t*)dyn;                               // [E+1]
  uint8_t* Bs = dyn + (((a.E + 1) * 4 + 15) / 16) * 16;           // [64][kPfRowBytes]
  init_tables(tab);
  build_tile_prefix(a.offsets, a.E, tile_pre, part);
  const int ty = blockIdx.y;
  if (tid == 0) {
    int e = -1;
    if (ty < tile_pre[a.E]) {
      int lo = 0, hi = a.E - 1;  // largest e with tile_pre[e] <= ty
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tile_pre[mid] <= ty) lo = mid; else hi = mid - 1;
      }
      e = lo;
    }
    tinfo[0] = e;
    tinfo[1] = e >= 0 ? ty - tile_pre[e] : 0;
  }
  __syncthreads();
  const int e = tinfo[0];
  if (e < 0) return;
  const int tb = tinfo[1] * kPfTokens;
  const int off = a.offsets[e];
  const int ne = a.offsets[e + 1] - off;
  const int K = a.K, N = a.N, nss = K / 256;

  // weight rows of this wave's m-fragments
  int64_t rowf[MF];
  bool wave_on = true;
  if (MLP) {
    const int I = N / 2;
    const int i0 = blockIdx.x * 128 + 32 * w;
#pragma unroll
    for (int f = 0; f < MF; f++) rowf[f] = (int64_t)e * N + (f < 2 ? 0 : I) + i0 + 16 * (f & 1) + r16;
  } else {
    const int n0 = blockIdx.x * 256 + 64 * w;
    wave_on = n0 < N;
#pragma unroll
    for (int f = 0; f < MF; f++) rowf[f] = (int64_t)e * N + (wave_on ? n0 + 16 * f : 0) + r16;
  }
  const float alpha = 1.0f / (a.gscale[e] * a.gamma_a[e]);

  f32x4 acc[MF][NF];
#pragma unroll
  for (int f = 0; f < MF; f++)
#pragma unroll
    for (int n = 0; n < NF; n++) acc[f][n] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // activation staging role: token tt, groups 8*part4 .. +8 of the super-step
  const int tt = tid >> 2, part4 = tid & 3;
  const bool st_valid = tb + tt < ne;
  const uint8_t* Qs = a.q + (int64_t)(off + (st_valid ? tb + tt : 0)) * (K / 2) + 32 * part4;
  const uint8_t* Ss = a.s + (int64_t)(off + (st_valid ? tb + tt : 0)) * (K / 32) + 2 * part4;
  uint8_t* Bw = Bs + tt * kPfRowBytes + part4 * 8 * 16;

  for (int ss = 0; ss < nss; ss++) {
    u32x4 pk[MF];
    uint32_t mk[MF], sw[MF];
    if (wave_on) {
#pragma unroll
      for (int f = 0; f < MF; f++) {
        pk[f] = *(const u32x4*)(a.packed + rowf[f] * (K / 4) + 64 * ss + 16 * c);
        mk[f] = *(const uint32_t*)(a.mask + rowf[f] * (K / 16) + 16 * ss + 4 * c);
        sw[f] = *(const uint16_t*)(a.wscale + rowf[f] * (K / 32) + 8 * ss + 2 * c);
      }
    }
    // stage + decode the activation tile of this super-step
    {
      u32x4 cw0 = (u32x4){0u, 0u, 0u, 0u}, cw1 = cw0;
      uint32_t sc2 = 0u;
      if (st_valid) {
        cw0 = *(const u32x4*)(Qs + 128 * ss);
        cw1 = *(const u32x4*)(Qs + 128 * ss + 16);
        sc2 = *(const uint16_t*)(Ss + 8 * ss);
      }
      const f16x2 s0 = bits_f16x2(tab.scl[sc2 & 0xFFu]);
      const f16x2 s1 = bits_f16x2(tab.scl[sc2 >> 8]);
      const uint32_t cws[8] = {cw0.x, cw0.y, cw0.z, cw0.w, cw1.x, cw1.y, cw1.z, cw1.w};
#pragma unroll
      for (int g = 0; g < 8; g++) *(u32x4*)(Bw + 16 * g) = decode_x_group(cws[g], g < 4 ? s0 : s1);
    }
    __syncthreads();
    if (wave_on) {
#pragma unroll
      for (int s = 0; s < 4; s++) {
        f16x8 A[MF];
        int idx[MF];
#pragma unroll
        for (int f = 0; f < MF; f++) {
          const f16x2 scw = bits_f16x2(tab.scl[(sw[f] >> (8 * (s >> 1))) & 0xFFu]);
          const uint32_t wd = s == 0 ? pk[f].x : s == 1 ? pk[f].y : s == 2 ? pk[f].z : pk[f].w;
          A[f] = decode_w_step(wd, scw);
          idx[f] = tab.idx[(mk[f] >> (8 * s)) & 0xFFu];
        }
        const int g1 = 8 * (c >> 1) + 2 * s + (c & 1);
#pragma unroll
        for (int n = 0; n < NF; n++) {
          const uint8_t* br = Bs + (n * 16 + r16) * kPfRowBytes;
          const f16x16 B = concat_x(*(const u32x4*)(br + 16 * g1), *(const u32x4*)(br + 16 * (g1 + 16)));
#pragma unroll
          for (int f = 0; f < MF; f++)
            acc[f][n] = __builtin_amdgcn_smfmac_f32_16x16x64_f16(A[f], B, acc[f][n], idx[f], 0, 0);
        }
      }
    }
    __syncthreads();
  }

  if (!wave_on) return;
  if (!MLP) {
    const int n0 = blockIdx.x * 256 + 64 * w;
#pragma unroll
    for (int n = 0; n < NF; n++) {
      const int tok = tb + n * 16 + r16;
      if (tok >= ne) continue;
#pragma unroll
      for (int f = 0; f < MF; f++) store4(a.y, (int64_t)(off + tok) * N + n0 + 16 * f + 4 * c, acc[f][n], alpha, a.y_bf16);
    }
  } else {
    const int I = N / 2;
    const int ib = blockIdx.x * 128 + 32 * w;  // first intermediate column of this wave (32-block)
    const float gh = a.gamma_h[e];
#pragma unroll
    for (int n = 0; n < NF; n++) {
      const int tok = tb + n * 16 + r16;
      const bool tv = tok < ne;
      float h[8];
#pragma unroll
      for (int f = 0; f < 2; f++) {
#pragma unroll
        for (int r = 0; r < 4; r++) {
          const float g = acc[f][n][r] * alpha;
          const float u = acc[f + 2][n][r] * alpha;
          h[4 * f + r] = g / (1.0f + __expf(-g)) * u;
        }
        if (tv && a.dump) {
          const int64_t rowo = (int64_t)(off + tok) * N;
          float4 gv, uv;
          gv.x = acc[f][n][0] * alpha; gv.y = acc[f][n][1] * alpha; gv.z = acc[f][n][2] * alpha; gv.w = acc[f][n][3] * alpha;
          uv.x = acc[f + 2][n][0] * alpha; uv.y = acc[f + 2][n][1] * alpha; uv.z = acc[f + 2][n][2] * alpha;
          uv.w = acc[f + 2][n][3] * alpha;
          *(float4*)(a.dump + rowo + ib + 16 * f + 4 * c) = gv;
          *(float4*)(a.dump + rowo + I + ib + 16 * f + 4 * c) = uv;
        }
      }
      // requantize: the 32-block of this token is spread over the 4 lanes c = 0..3 (xor 16, 32)
      float am = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; i++) am = __builtin_fmaxf(am, __builtin_fabsf(h[i]));
      am = __builtin_fmaxf(am, __shfl_xor(am, 16));
      am = __builtin_fmaxf(am, __shfl_xor(am, 32));
      const float t = gh * am;
      const float uq = t / 6.0f;
      const uint32_t sc = e4m3_encode(uq);
      const float sv = e4m3_value(sc) / gh;
      if (tv) {
        const int64_t p = off + tok;
#pragma unroll
        for (int f = 0; f < 2; f++) {
          uint32_t codes = 0u;
          if (sv != 0.0f) {
#pragma unroll
            for (int r = 0; r < 4; r++) codes |= e2m1_encode(h[4 * f + r] / sv) << (4 * r);
          }
          *(uint16_t*)(a.h_q + p * (I / 2) + (ib + 16 * f + 4 * c) / 2) = (uint16_t)codes;
        }
        if (c == 0) a.h_s[p * (I / 32) + ib / 32] = (uint8_t)sc;
      }
    }
  }
}

static size_t prefill_lds_bytes(int E) { return (size_t)(((E + 1) * 4 + 15) / 16) * 16 + (size_t)kPfTokens * kPfRowBytes; }

int launch_gemm_variant(hipStream_t st, const GemmArgs& a, int64_t rows, int variant) {
  if (rows == 0) return MOESQ_OK;
  if (variant == 0) {
    hipLaunchKernelGGL(gemm_decode_kernel<4>, dim3(a.N / 64, a.E), dim3(256), 0, st, a);
  } else {
    const int64_t tiles = (rows + kPfTokens - 1) / kPfTokens + a.E;
    const size_t lds = prefill_lds_bytes(a.E);
    if (a.gamma_h) {
      hipLaunchKernelGGL(gemm_prefill_kernel<true>, dim3(a.N / 256, (unsigned)tiles), dim3(256), lds, st, a);
    } else {
      hipLaunchKernelGGL(gemm_prefill_kernel<false>, dim3((a.N + 255) / 256, (unsigned)tiles), dim3(256), lds, st,
                         a);
    }
  }
  return hipGetLastError() == hipSuccess ? MOESQ_OK : MOESQ_ERR_HIP;
}

int launch_gemm(hipStream_t st, const GemmArgs& a, int64_t rows) {
  // Few tokens per expert: weight streaming; otherwise the tiled kernel. The MLP epilogue lives in
  // the tiled kernel.
  const bool decode = a.gamma_h == nullptr && rows <= (int64_t)16 * a.E;
  return launch_gemm_variant(st, a, rows, decode ? 0 : 1);
}

}  // namespace moesq
