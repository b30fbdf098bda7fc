// Router-weighted unpermute + combine (paper Appendix D.1, token combination): out[t] is the sum
// over the k routed copies of token t, in slot order j = 0..k-1, of topk_w[t][j] times that copy's
// expert output row; fp32 accumulation, no atomics (deterministic).
#include "common.h"
#include "launch.h"

namespace moesq {

// grid (ceil(H/8/256), T); each thread owns 8 consecutive output columns of one token.
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y, int y_bf16,
                                                      const int32_t* __restrict__ slot_pos,
                                                      const float* __restrict__ topk_w, int32_t k, int32_t H,
                                                      void* __restrict__ out, int out_bf16) {
  const int64_t t = blockIdx.y;
  const int col = 8 * (blockIdx.x * 256 + threadIdx.x);
  if (col >= H) return;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; i++) acc[i] = 0.0f;
  for (int j = 0; j < k; j++) {
    const int32_t p = slot_pos[t * k + j];
    if (p < 0) continue;
    const float wt = topk_w[t * k + j];
    float v[8];
    if (y_bf16) {
      const uint4 raw = *(const uint4*)((const uint16_t*)y + (int64_t)p * H + col);
      const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int i = 0; i < 4; i++) {
        v[2 * i] = bf16_bits_to_f32(wd[i] & 0xFFFFu);
        v[2 * i + 1] = bf16_bits_to_f32(wd[i] >> 16);
      }
    } else {
      const float4 a = *(const float4*)((const float*)y + (int64_t)p * H + col);
      const float4 b = *(const float4*)((const float*)y + (int64_t)p * H + col + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
#pragma unroll
    for (int i = 0; i < 8; i++) acc[i] = acc[i] + wt * v[i];
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
  const int gx = (H / 8 + 255) / 256;
  hipLaunchKernelGGL(combine_kernel, dim3(gx, (unsigned)T), dim3(256), 0, st, y, (int)y_bf16, slot_pos, w, k, H,
                     out, (int)out_bf16);
  return hipGetLastError() == hipSuccess ? MOESQ_OK : MOESQ_ERR_HIP;
}

}  // namespace moesq
