// Router-weighted unpermute + combine (paper Appendix D.1, token combination): out[t] is the sum
// over the k routed copies of token t, in slot order j = 0..k-1, of topk_w[t][j] times that copy's
// expert output row; fp32 accumulation, no atomics (deterministic).
#include "common.h"
#include "launch.h"

namespace moesq {

constexpr int kCombineThreads = 128;  // 7168 / 8 = 7 x 128: no idle lanes at the Kimi hidden size
constexpr int kCombineUnroll = 8;     // routed copies whose rows are in flight together

// One copy's 8-column row segment: 16 bytes of bf16 or 32 bytes of fp32, loaded raw.
template <bool YBF16>
struct Row8 {
  uint4 r[YBF16 ? 1 : 2];
};

// bf16 rows are read with the non-temporal hint: each is read once, and the hint measured 11% faster
// at the Kimi prefill size (c4 combine 202 -> 179 us); fp32 rows measured no better with it.
template <bool YBF16>
MOESQ_DEV Row8<YBF16> combine_load(const void* __restrict__ y, int64_t p, int32_t H, int col) {
  Row8<YBF16> o;
  if (YBF16) {
    const u32x4 v = __builtin_nontemporal_load((const u32x4*)((const uint16_t*)y + p * H + col));
    o.r[0] = make_uint4(v.x, v.y, v.z, v.w);
  } else {
    o.r[0] = *(const uint4*)((const float*)y + p * H + col);
    o.r[YBF16 ? 0 : 1] = *(const uint4*)((const float*)y + p * H + col + 4);
  }
  return o;
}

template <bool YBF16>
MOESQ_DEV void combine_values(const Row8<YBF16>& o, float v[8]) {
  if (YBF16) {
    const uint32_t wd[4] = {o.r[0].x, o.r[0].y, o.r[0].z, o.r[0].w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[2 * i] = bf16_bits_to_f32(wd[i] & 0xFFFFu);
      v[2 * i + 1] = bf16_bits_to_f32(wd[i] >> 16);
    }
  } else {
    const uint4 a = o.r[0], b = o.r[YBF16 ? 0 : 1];
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y); v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y); v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
  }
}

// grid (ceil(H/8/128), T); each thread owns 8 consecutive output columns of one token. The copies are
// taken kCombineUnroll at a time: their (uniform) slots and weights first, then all their row loads
// (a copy with no row loads a row of the group that has one, and is not added), then the
// multiply-adds in slot order, so the sum is the same as one copy after another.
template <bool YBF16>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const void* __restrict__ y,
                                                                  const int32_t* __restrict__ slot_pos,
                                                                  const float* __restrict__ topk_w, int32_t k,
                                                                  int32_t H, void* __restrict__ out, int out_bf16) {
  const int64_t t = blockIdx.y;
  const int col = 8 * (blockIdx.x * kCombineThreads + threadIdx.x);
  if (col >= H) return;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; i++) acc[i] = 0.0f;
  for (int j0 = 0; j0 < k; j0 += kCombineUnroll) {
    int32_t p[kCombineUnroll];
    float wt[kCombineUnroll];
    int32_t pany = -1;
#pragma unroll
    for (int u = 0; u < kCombineUnroll; u++) {
      const int j = j0 + u;
      p[u] = j < k ? slot_pos[t * k + j] : -1;
      wt[u] = j < k ? topk_w[t * k + j] : 0.0f;
      pany = max(pany, p[u]);
    }
    if (pany < 0) continue;  // no copy of this group has a row
    Row8<YBF16> raw[kCombineUnroll];
#pragma unroll
    for (int u = 0; u < kCombineUnroll; u++) raw[u] = combine_load<YBF16>(y, p[u] >= 0 ? p[u] : pany, H, col);
#pragma unroll
    for (int u = 0; u < kCombineUnroll; u++) {
      if (p[u] < 0) continue;  // a copy with no row (invalid id, or over capacity)
      float v[8];
      combine_values<YBF16>(raw[u], v);
#pragma unroll
      for (int i = 0; i < 8; i++) acc[i] = acc[i] + wt[u] * v[i];
    }
  }
  if (out_bf16) {
    uint4 o;
    o.x = f32_to_bf16_bits(acc[0]) | (f32_to_bf16_bits(acc[1]) << 16);
    o.y = f32_to_bf16_bits(acc[2]) | (f32_to_bf16_bits(acc[3]) << 16);
    o.z = f32_to_bf16_bits(acc[4]) | (f32_to_bf16_bits(acc[5]) << 16);
    o.w = f32_to_bf16_bits(acc[6]) | (f32_to_bf16_bits(acc[7]) << 16);
    *(uint4*)((uint16_t*)out + t * H + col) = o;
  } else {
    float4 a, b;
    a.x = acc[0]; a.y = acc[1]; a.z = acc[2]; a.w = acc[3];
    b.x = acc[4]; b.y = acc[5]; b.z = acc[6]; b.w = acc[7];
    *(float4*)((float*)out + t * H + col) = a;
    *(float4*)((float*)out + t * H + col + 4) = b;
  }
}

int launch_combine(hipStream_t st, const void* y, bool y_bf16, const int32_t* slot_pos, const float* w, int64_t T,
                   int32_t k, int32_t H, void* out, bool out_bf16) {
  if (T == 0) return MOESQ_OK;
  const int gx = (H / 8 + kCombineThreads - 1) / kCombineThreads;
  if (y_bf16)
    hipLaunchKernelGGL(combine_kernel<true>, dim3(gx, (unsigned)T), dim3(kCombineThreads), 0, st, y, slot_pos, w, k, H, out,
                       (int)out_bf16);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3(gx, (unsigned)T), dim3(kCombineThreads), 0, st, y, slot_pos, w, k, H, out,
                       (int)out_bf16);
  return hipGetLastError() == hipSuccess ? MOESQ_OK : MOESQ_ERR_HIP;
}

}  // namespace moesq
