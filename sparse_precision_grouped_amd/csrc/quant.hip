// NVFP4 quantization kernels:
//  - dispatch + dynamic activation quantization (paper Section 3.4 and Appendix D.1: 32-element
//    blocks at run time, fused with token dispatch; Eq. 3 + Eq. 5 with the expert's tensor scale);
//  - weight compression to paired-4:8 NVFP4 in pair-bitmask v1 storage (setup; Section 3.4 last
//    paragraph, Appendix A; model card "Sparse storage layout");
//  - pair-bitmask v1 -> dense NVFP4 unpacking (the model card's lossless round trip).
#include "common.h"
#include "launch.h"

namespace moesq {

// max |x| over the 8-groups g = first, first + stride, ... < n of a [rows][ld] tensor with gpr 8-groups
// per row (K % 8 == 0, ld % 8 == 0, 16-byte aligned): U independent loads in flight per round (an index
// past the end re-reads the last group, which leaves the max unchanged).
template <int U, bool BF16>
MOESQ_DEV float amax_groups_t(const void* __restrict__ x, int32_t n, int32_t gpr, int64_t ld, int32_t first,
                              int32_t stride) {
  float m = 0.0f;
  for (int32_t g0 = first; g0 < n; g0 += U * stride) {
    // addresses first, then every load, then the reductions, so the U loads are in flight together
    int64_t off[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int32_t g = min(g0 + u * stride, n - 1);
      const int32_t r = g / gpr;
      off[u] = (int64_t)r * ld + 8 * (int64_t)(g - r * gpr);
    }
    if (BF16) {
      uint4 raw[U];
#pragma unroll
      for (int u = 0; u < U; u++) raw[u] = *(const uint4*)((const uint16_t*)x + off[u]);
#pragma unroll
      for (int u = 0; u < U; u++) {
        const uint32_t wd[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
        for (int j = 0; j < 4; j++) {
          m = __builtin_fmaxf(m, __builtin_fabsf(bf16_bits_to_f32(wd[j] & 0xFFFFu)));
          m = __builtin_fmaxf(m, __builtin_fabsf(bf16_bits_to_f32(wd[j] >> 16)));
        }
      }
    } else {
      float4 a[U], b[U];
#pragma unroll
      for (int u = 0; u < U; u++) {
        a[u] = *(const float4*)((const float*)x + off[u]);
        b[u] = *(const float4*)((const float*)x + off[u] + 4);
      }
#pragma unroll
      for (int u = 0; u < U; u++) {
        m = __builtin_fmaxf(m, __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(a[u].x), __builtin_fabsf(a[u].y)),
                                               __builtin_fmaxf(__builtin_fabsf(a[u].z), __builtin_fabsf(a[u].w))));
        m = __builtin_fmaxf(m, __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(b[u].x), __builtin_fabsf(b[u].y)),
                                               __builtin_fmaxf(__builtin_fabsf(b[u].z), __builtin_fabsf(b[u].w))));
      }
    }
  }
  return m;
}

template <int U>
MOESQ_DEV float amax_groups(const void* __restrict__ x, int x_bf16, int32_t n, int32_t gpr, int64_t ld, int32_t first,
                            int32_t stride) {
  return x_bf16 ? amax_groups_t<U, true>(x, n, gpr, ld, first, stride)
                : amax_groups_t<U, false>(x, n, gpr, ld, first, stride);
}

// Workgroup-wide max of m (256 threads; wmax: 4 floats of LDS).
MOESQ_DEV float block_max256(float m, float* wmax) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, d));
  if (lane == 0) wmax[w] = m;
  __syncthreads();
  return __builtin_fmaxf(__builtin_fmaxf(wmax[0], wmax[1]), __builtin_fmaxf(wmax[2], wmax[3]));
}

// This thread's share of the amax of |x| over rows [0, T) x [0, K) scanned by one workgroup of 256
// threads (16 loads in flight); block_max256 of it gives the tensor's amax.
MOESQ_DEV float thread_amax(const void* __restrict__ x, int x_bf16, int64_t T, int32_t K, int64_t ld_x) {
  return amax_groups<16>(x, x_bf16, (int32_t)(T * (K / 8)), K / 8, ld_x, threadIdx.x, 256);
}

// Fused dispatch + quantization: one workgroup per token. Its waves take the token's 512-element
// chunks (wave w: chunks w, w+4, ...), read them once, quantize them (a lane holds 8 consecutive
// values, four lanes per 32-block, block amax by a 4-lane max reduction) and write the codes to every
// permuted row the token is routed to. The codes depend on the row's expert only through its tensor
// scale, so they are recomputed only when that scale changes between consecutive copies.
constexpr int kQuantMaxE = 4096;
constexpr int kQuantMaxK = 512;

// NT: load with the non-temporal hint (token rows read once, from a token matrix too large to stay
// in the caches).
template <bool NT = false>
MOESQ_DEV void load_chunk(const void* __restrict__ x, int x_bf16, int64_t t, int64_t ld_x, int ch, bool valid,
                          float v[8]) {
#pragma unroll
  for (int i = 0; i < 8; i++) v[i] = 0.0f;
  if (!valid) return;
  if (x_bf16) {
    const u32x4* src = (const u32x4*)((const uint16_t*)x + t * ld_x + 8 * ch);
    const u32x4 raw = NT ? __builtin_nontemporal_load(src) : *src;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[2 * i] = bf16_bits_to_f32(raw[i] & 0xFFFFu);
      v[2 * i + 1] = bf16_bits_to_f32(raw[i] >> 16);
    }
  } else {
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    const f32x4v* src = (const f32x4v*)((const float*)x + t * ld_x + 8 * ch);
    const f32x4v a = NT ? __builtin_nontemporal_load(src) : src[0];
    const f32x4v b = NT ? __builtin_nontemporal_load(src + 1) : src[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// Quantize token t's row (this wave's first chunk already in v) and write the codes to the nk
// permuted rows dst[0..nk) (LDS; negative = skipped), each with its expert's tensor scale gam[j].
template <bool NT = false>
MOESQ_DEV void quantize_token_copies(const void* __restrict__ x, int x_bf16, int64_t t, int32_t K, int64_t ld_x,
                                     float v[8], int nk, const int32_t* dst, const float* gam,
                                     uint8_t* __restrict__ q, uint8_t* __restrict__ s, uint8_t* __restrict__ xk) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nchunk = (K + 511) / 512;
  for (int chunk = w; chunk < nchunk; chunk += 4) {
    const int ch = chunk * 64 + lane;  // 8-value group index within the row
    const bool valid = ch < K / 8;
    if (chunk != w) load_chunk<NT>(x, x_bf16, t, ld_x, ch, valid, v);
    bool have = false;
    float gq = 0.0f;
    uint32_t codes = 0u, sc = 0u;
    u32x4 xv = {0u, 0u, 0u, 0u};
    for (int j = 0; j < nk; j++) {
      const int32_t p = dst[j];
      if (p < 0) continue;
      const float g = gam[j];
      if (!have || g != gq) {
        quant8_block4(v, g, codes, sc);
        if (xk) {
          // the same values dequantized (exact in f16), in the GEMM's de-interleaved group order
          f16x2 sv, unused;
          e4m3_pair_f16x2(sc, sv, unused);
          xv = decode_x_group(codes, sv);
        }
        gq = g;
        have = true;
      }
      if (valid) {
        *(uint32_t*)(q + (int64_t)p * (K / 2) + 4 * ch) = codes;
        if ((lane & 3) == 0) s[(int64_t)p * (K / 32) + ch / 4] = (uint8_t)sc;
        if (xk) *(u32x4*)(xk + ((int64_t)p * K + 8 * ch) * 2) = xv;
      }
    }
  }
}

template <bool NT>
__global__ __launch_bounds__(256) void quantize_kernel(const void* __restrict__ x, int x_bf16, int64_t T, int32_t K,
                                                       int64_t ld_x, const int32_t* __restrict__ slot_pos, int32_t k,
                                                       const float* __restrict__ gamma,
                                                       const int32_t* __restrict__ offsets, int32_t E,
                                                       uint8_t* __restrict__ q, uint8_t* __restrict__ s,
                                                       uint8_t* __restrict__ xk, int32_t cap) {
  __shared__ int32_t off_l[kQuantMaxE + 1];
  __shared__ int32_t dst[kQuantMaxK];
  __shared__ float gam[kQuantMaxK];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t t = blockIdx.x;
  const int nk = slot_pos ? k : 1;
  const int nchunk = (K + 511) / 512;
  // the independent loads first: this wave's first chunk of the row, the token's destinations, the
  // expert offsets
  float v[8];
  load_chunk<NT>(x, x_bf16, t, ld_x, w * 64 + lane, w < nchunk && w * 64 + lane < K / 8, v);
  int32_t p0 = tid < nk ? (slot_pos ? slot_pos[t * k + tid] : (int32_t)t) : -1;
  if (offsets) {
    for (int i = tid; i <= E; i += 256) off_l[i] = offsets[i];
    __syncthreads();
  }
  for (int j = tid; j < nk; j += 256) {
    int32_t p = j == tid ? p0 : (slot_pos ? slot_pos[t * k + j] : (int32_t)t);
    float g = gamma[0];
    if (p >= 0 && offsets) {
      if (p >= off_l[E]) {
        p = -1;  // not a routed row
      } else {
        int lo = 0, hi = E - 1;  // largest e with offsets[e] <= p
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (off_l[mid] <= p) lo = mid; else hi = mid - 1;
        }
        g = gamma[lo];
      }
    } else if (p >= 0 && cap > 0) {
      g = gamma[p / cap];  // capacity layout: expert e owns rows [e cap, (e + 1) cap)
    }
    dst[j] = p;
    gam[j] = g;
  }
  __syncthreads();
  quantize_token_copies<NT>(x, x_bf16, t, K, ld_x, v, nk, dst, gam, q, s, xk);
}

int launch_quantize(hipStream_t st, const void* x, bool x_bf16, int64_t T, int32_t K, int64_t ld_x,
                    const int32_t* slot_pos, int32_t k, const float* gamma, const int32_t* offsets, int32_t E,
                    uint8_t* q, uint8_t* s, void* xk, int32_t cap) {
  if (T == 0) return MOESQ_OK;
  // A token matrix of more than 64 MiB is read with the non-temporal hint: at the Kimi prefill size
  // (235 MB of fp32 tokens) that measured 12% faster (108 -> 95 us); at 34 MB (c2) the default policy
  // was faster (18.4 vs 19.8 us), the rows staying in the caches.
  if ((int64_t)T * ld_x * (x_bf16 ? 2 : 4) > ((int64_t)64 << 20))
    hipLaunchKernelGGL(quantize_kernel<true>, dim3((unsigned)T), dim3(256), 0, st, x, (int)x_bf16, T, K, ld_x, slot_pos, k,
                       gamma, offsets, E, q, s, (uint8_t*)xk, cap);
  else
    hipLaunchKernelGGL(quantize_kernel<false>, dim3((unsigned)T), dim3(256), 0, st, x, (int)x_bf16, T, K, ld_x, slot_pos,
                       k, gamma, offsets, E, q, s, (uint8_t*)xk, cap);
  return hipGetLastError() == hipSuccess ? MOESQ_OK : MOESQ_ERR_HIP;
}

// Capacity layout ([P] Appendix D.1: activations and outputs batched with a fixed per-expert capacity,
// so expert e's operands sit at a fixed stride): slot f of expert e with stable rank r among that
// expert's slots goes to row e * cap + r, or nowhere (-1) when r >= cap; invalid ids stay -1.
__global__ __launch_bounds__(256) void capacity_slots_kernel(const int32_t* __restrict__ ids, int64_t n, int32_t cap,
                                                             const int32_t* __restrict__ offsets,
                                                             const int32_t* __restrict__ slot_pos_prefix,
                                                             int32_t* __restrict__ slot_pos) {
  const int64_t f = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (f >= n) return;
  const int32_t p = slot_pos_prefix[f];
  int32_t out = -1;
  if (p >= 0) {
    const int32_t e = ids[f];
    const int32_t r = p - offsets[e];
    if (r < cap) out = e * cap + r;
  }
  slot_pos[f] = out;
}

int launch_capacity_slots(hipStream_t st, const int32_t* ids, int64_t n, int32_t E, int32_t cap, const int32_t* offsets,
                          const int32_t* slot_pos_prefix, int32_t* slot_pos) {
  (void)E;
  if (n == 0) return MOESQ_OK;
  hipLaunchKernelGGL(capacity_slots_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, ids, n, cap, offsets,
                     slot_pos_prefix, slot_pos);
  return hipGetLastError() == hipSuccess ? MOESQ_OK : MOESQ_ERR_HIP;
}

// Routing fused into the quantizer for decode-sized batches (T*k <= kRouteSingleMax, k <=
// kFusedRouteMaxK): every workgroup (one per token) reads all T*k ids, builds the expert histogram
// and its exclusive prefix in LDS, and places only its own token's k copies: row = offsets[e] +
// the number of earlier slots with expert e, counted with wave ballots. The results equal those of
// the routing kernels followed by quantize_kernel, with one launch and no dependent read of
// slot_pos / offsets from global memory.
__global__ __launch_bounds__(256) void route_quantize_kernel(
    const int32_t* __restrict__ ids, int32_t k, int32_t E, const void* __restrict__ x, int x_bf16, int32_t K,
    int64_t ld_x, const float* __restrict__ gamma, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_slot, int32_t* __restrict__ slot_pos, int32_t* dev_status, uint8_t* __restrict__ q,
    uint8_t* __restrict__ s, uint8_t* __restrict__ xk, float* __restrict__ gamma_out) {
  __shared__ int32_t hist[kMaxExpertsRoute];
  __shared__ float wmax[4];
  __shared__ int32_t pos[kMaxExpertsRoute + 1];
  __shared__ float gam_all[kMaxExpertsRoute];  // all tensor scales: no load that waits on an id
  __shared__ int32_t wsum[4];
  __shared__ int32_t mine[kFusedRouteMaxK];
  __shared__ int32_t wcnt[4][kFusedRouteMaxK];  // per wave: earlier slots with copy j's expert
  __shared__ int32_t dst[kFusedRouteMaxK];
  __shared__ float gam[kFusedRouteMaxK];
  constexpr int R = kRouteSingleMax / 256;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t t = blockIdx.x;
  const int64_t n = (int64_t)gridDim.x * k;
  const int64_t f0 = t * k;  // this token's first slot
  const int nchunk = (K + 511) / 512;
  float v[8];
  load_chunk(x, x_bf16, t, ld_x, w * 64 + lane, w < nchunk && w * 64 + lane < K / 8, v);
  int ev[R];
#pragma unroll
  for (int r = 0; r < R; r++) {
    const int64_t f = tid + (int64_t)r * 256;
    ev[r] = f < n ? ids[f] : -1;
  }
  // dynamic tensor scale: this thread's part of the amax over all T x K values, loaded together with
  // the ids (every workgroup scans the whole tensor itself; max is order-free, so all agree)
  const float am_part = gamma_out ? thread_amax(x, x_bf16, gridDim.x, K, ld_x) : 0.0f;
  int e_my = -1;
  if (tid < k) {
    e_my = ids[f0 + tid];
    if (e_my < 0 || e_my >= E) e_my = -1;
  }
  for (int i = tid; i < E; i += 256) {
    hist[i] = 0;
    if (!gamma_out) gam_all[i] = gamma[i];
  }
  if (gamma_out) {
    // Eq. 5 from the tensor amax; workgroup 0 publishes it as the per-expert scales the GEMM reads
    const float g = global_scale_from_amax(block_max256(am_part, wmax));
    for (int i = tid; i < E; i += 256) {
      gam_all[i] = g;
      if (blockIdx.x == 0) gamma_out[i] = g;
    }
  }
  if (tid < k) mine[tid] = e_my;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; r++)
    if (ev[r] >= 0 && ev[r] < E) atomicAdd(&hist[ev[r]], 1);
  __syncthreads();
  block_exclusive_scan<256>(hist, E, pos, wsum);
  if (blockIdx.x == 0) {
    for (int i = tid; i <= E; i += 256) {
      offsets[i] = pos[i];
      if (i < E) counts[i] = hist[i];
    }
  }
  // rank of copy j = number of slots f < f0 + j routed to the same expert: each wave counts its own
  // slots with ballots (only rounds holding such slots take part) for 8 copies at a time, and the
  // wave counts are added after one barrier
  const int nr = (int)((f0 + k + 255) / 256);
  for (int j0 = 0; j0 < k; j0 += 8) {
    int ej[8];
#pragma unroll
    for (int u = 0; u < 8; u++) ej[u] = j0 + u < k ? mine[j0 + u] : -1;  // uniform over the workgroup
#pragma unroll
    for (int u = 0; u < 8; u++) {
      if (ej[u] < 0) continue;
      int c = 0;
#pragma unroll
      for (int r = 0; r < R; r++)
        if (r < nr) c += __builtin_popcountll(__ballot(ev[r] == ej[u] && tid + (int64_t)r * 256 < f0 + j0 + u));
      if (lane == 0) wcnt[w][j0 + u] = c;
    }
  }
  __syncthreads();
  if (tid < k) {
    int32_t p = -1;
    if (e_my >= 0) {
      p = pos[e_my] + wcnt[0][tid] + wcnt[1][tid] + wcnt[2][tid] + wcnt[3][tid];
      sorted_slot[p] = (int32_t)(f0 + tid);
    } else if (dev_status) {
      *dev_status = MOESQ_ERR_INVALID_ARG;
    }
    slot_pos[f0 + tid] = p;
    dst[tid] = p;
    gam[tid] = e_my >= 0 ? gam_all[e_my] : 0.0f;
  }
  __syncthreads();
  quantize_token_copies(x, x_bf16, t, K, ld_x, v, k, dst, gam, q, s, xk);
}

bool route_quantize_fused(int64_t T, int32_t k, int32_t E) {
  return T > 0 && T * k <= kRouteSingleMax && k <= kFusedRouteMaxK && E <= kMaxExpertsRoute;
}

bool route_quantize_dyn_fused(int64_t T, int32_t k, int32_t E, int32_t K, bool x_bf16) {
  return route_quantize_fused(T, k, E) && T * K * (x_bf16 ? 2 : 4) <= kDynScaleMaxBytes;
}

int launch_route_quantize(hipStream_t st, const int32_t* ids, int64_t T, int32_t k, int32_t E, const void* x,
                          bool x_bf16, int32_t K, int64_t ld_x, const float* gamma, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_slot, int32_t* slot_pos, void* ws, int32_t* dev_status,
                          uint8_t* q, uint8_t* s, void* xk, float* gamma_out) {
  const bool one = gamma_out ? route_quantize_dyn_fused(T, k, E, K, x_bf16) : route_quantize_fused(T, k, E);
  if (!one) {
    if (gamma_out) {
      // amax pre-pass: Eq. 5 over the whole tensor, broadcast to the E per-expert scales
      const int rc = launch_global_scale(st, x, x_bf16, T, K, ld_x, gamma_out, E);
      if (rc != MOESQ_OK) return rc;
      gamma = gamma_out;
    }
    if (route_quantize_fused(T, k, E)) {
      hipLaunchKernelGGL(route_quantize_kernel, dim3((unsigned)T), dim3(256), 0, st, ids, k, E, x, (int)x_bf16, K,
                         ld_x, gamma, counts, offsets, sorted_slot, slot_pos, dev_status, q, s, (uint8_t*)xk,
                         (float*)nullptr);
      return hipGetLastError() == hipSuccess ? MOESQ_OK : MOESQ_ERR_HIP;
    }
    const int rc = launch_route(st, ids, T * k, E, counts, offsets, sorted_slot, slot_pos, ws, dev_status);
    if (rc != MOESQ_OK) return rc;
    return launch_quantize(st, x, x_bf16, T, K, ld_x, slot_pos, k, gamma, offsets, E, q, s, xk);
  }
  hipLaunchKernelGGL(route_quantize_kernel, dim3((unsigned)T), dim3(256), 0, st, ids, k, E, x, (int)x_bf16, K, ld_x,
                     gamma, counts, offsets, sorted_slot, slot_pos, dev_status, q, s, (uint8_t*)xk, gamma_out);
  return hipGetLastError() == hipSuccess ? MOESQ_OK : MOESQ_ERR_HIP;
}

// ------------------------------------------------------------------ weight compression ----------
// Paired-4:8 pruning of one 8-group in place: keep the two pairs with the largest L2 norm (fp64
// norms, ties to the lower pair index), zero the other two.
MOESQ_DEV void prune_group(float v[8]) {
  double nrm[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const double a = (double)v[2 * i], b = (double)v[2 * i + 1];
    const double aa = a * a, bb = b * b;
    nrm[i] = aa + bb;
  }
  int first = 0;
#pragma unroll
  for (int i = 1; i < 4; i++)
    if (nrm[i] > nrm[first]) first = i;
  int second = first == 0 ? 1 : 0;
#pragma unroll
  for (int i = 0; i < 4; i++)
    if (i != first && nrm[i] > nrm[second]) second = i;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    if (i != first && i != second) {
      v[2 * i] = 0.0f;
      v[2 * i + 1] = 0.0f;
    }
  }
}

__global__ void zero_words_kernel(uint32_t* p, int32_t n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// Per expert amax of the pruned weights, as ordered float bits (max of non-negative floats equals
// max of their bit patterns, so the atomic result does not depend on order).
__global__ __launch_bounds__(256) void compress_amax_kernel(const float* __restrict__ w, int32_t N, int32_t K,
                                                            uint32_t* __restrict__ amax_bits) {
  const int e = blockIdx.y;
  const int64_t ngroups = (int64_t)N * K / 8;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  float m = 0.0f;
  if (g < ngroups) {
    const float* src = w + (int64_t)e * N * K + 8 * g;
    const float4 a = *(const float4*)src, b = *(const float4*)(src + 4);
    float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    prune_group(v);
#pragma unroll
    for (int i = 0; i < 8; i++) m = __builtin_fmaxf(m, __builtin_fabsf(v[i]));
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, d));
  if ((threadIdx.x & 63) == 0 && m > 0.0f) atomicMax(&amax_bits[e], __float_as_uint(m));
}

// One thread per 32-element block of a weight row: prune its four 8-groups, quantize (Eq. 3 + 5
// with the expert's tensor scale), form dense NVFP4 bytes, and store them as pair-bitmask v1.
__global__ __launch_bounds__(256) void compress_pack_kernel(const float* __restrict__ w, int32_t N, int32_t K,
                                                            const uint32_t* __restrict__ amax_bits,
                                                            uint8_t* __restrict__ packed, uint8_t* __restrict__ mask,
                                                            uint8_t* __restrict__ scale, float* __restrict__ gscale,
                                                            int32_t* dev_status) {
  const int e = blockIdx.y;
  const int64_t nblocks = (int64_t)N * (K / 32);
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const float gamma = global_scale_from_amax(__uint_as_float(amax_bits[e]));
  if (i == 0) gscale[e] = gamma;
  if (i >= nblocks) return;
  const float* src = w + (int64_t)e * N * K + 32 * i;
  float v[32];
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const float4 a = *(const float4*)(src + 4 * j);
    v[4 * j] = a.x; v[4 * j + 1] = a.y; v[4 * j + 2] = a.z; v[4 * j + 3] = a.w;
  }
#pragma unroll
  for (int gi = 0; gi < 4; gi++) prune_group(v + 8 * gi);
  float am = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; j++) am = __builtin_fmaxf(am, __builtin_fabsf(v[j]));
  const float t = gamma * am;
  const float u = t / 6.0f;
  const uint32_t sc = e4m3_encode(u);
  const float sv = e4m3_value(sc) / gamma;
  uint8_t dense[16];
#pragma unroll
  for (int j = 0; j < 16; j++) {
    uint32_t c0 = 0u, c1 = 0u;
    if (sv != 0.0f) {
      c0 = e2m1_encode(v[2 * j] / sv);
      c1 = e2m1_encode(v[2 * j + 1] / sv);
    }
    dense[j] = (uint8_t)(c0 | (c1 << 4));
  }
  uint8_t pk[8];
  uint32_t nibs = 0u;
  bool bad = false;
#pragma unroll
  for (int c = 0; c < 4; c++) {
    uint32_t nib = 0u, cnt = 0u;
#pragma unroll
    for (int b = 0; b < 4; b++)
      if (dense[4 * c + b] != 0) { nib |= 1u << b; cnt++; }
    if (cnt > 2u) { bad = true; nib = 0u; cnt = 0u; }
#pragma unroll
    for (int b = 0; b < 4; b++)
      if (cnt < 2u && !(nib & (1u << b))) { nib |= 1u << b; cnt++; }
    int o = 0;
#pragma unroll
    for (int b = 0; b < 4; b++)
      if (nib & (1u << b)) { pk[2 * c + (o & 1)] = dense[4 * c + b]; o++; }
    nibs |= nib << (4 * c);
  }
  if (bad && dev_status) *dev_status = MOESQ_ERR_PATTERN;
  const int64_t row = i / (K / 32), b = i % (K / 32);
  const int64_t rbase = (int64_t)e * N + row;
  uint2 pw;
  pw.x = (uint32_t)pk[0] | ((uint32_t)pk[1] << 8) | ((uint32_t)pk[2] << 16) | ((uint32_t)pk[3] << 24);
  pw.y = (uint32_t)pk[4] | ((uint32_t)pk[5] << 8) | ((uint32_t)pk[6] << 16) | ((uint32_t)pk[7] << 24);
  *(uint2*)(packed + rbase * (K / 4) + 8 * b) = pw;
  *(uint16_t*)(mask + rbase * (K / 16) + 2 * b) = (uint16_t)nibs;
  scale[rbase * (K / 32) + b] = (uint8_t)sc;
}

int launch_compress(hipStream_t st, const float* w, int32_t E, int32_t N, int32_t K, uint8_t* packed, uint8_t* mask,
                    uint8_t* scale, float* gscale, void* ws, int32_t* dev_status) {
  uint32_t* amax = (uint32_t*)ws;
  hipLaunchKernelGGL(zero_words_kernel, dim3((E + 255) / 256), dim3(256), 0, st, amax, E);
  const int64_t ngroups = (int64_t)N * K / 8;
  hipLaunchKernelGGL(compress_amax_kernel, dim3((unsigned)((ngroups + 255) / 256), E), dim3(256), 0, st, w, N, K,
                     amax);
  const int64_t nblocks = (int64_t)N * (K / 32);
  hipLaunchKernelGGL(compress_pack_kernel, dim3((unsigned)((nblocks + 255) / 256), E), dim3(256), 0, st, w, N, K,
                     amax, packed, mask, scale, gscale, dev_status);
  return hipGetLastError() == hipSuccess ? MOESQ_OK : MOESQ_ERR_HIP;
}

// ------------------------------------------------------------------ unpack ------------------------
__global__ __launch_bounds__(256) void unpack_kernel(const uint8_t* __restrict__ packed,
                                                     const uint8_t* __restrict__ mask, int64_t nchunks,
                                                     uint8_t* __restrict__ dense, int32_t* dev_status) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= nchunks) return;
  const uint32_t mb = mask[c >> 1];
  const uint32_t nib = (c & 1) ? (mb >> 4) : (mb & 15u);
  if (__builtin_popcount(nib) != 2 && dev_status) *dev_status = MOESQ_ERR_PATTERN;
  const uint32_t b0 = packed[2 * c], b1 = packed[2 * c + 1];
  uint32_t out = 0u;
  int o = 0;
#pragma unroll
  for (int b = 0; b < 4; b++) {
    if ((nib & (1u << b)) && o < 2) {
      out |= (o == 0 ? b0 : b1) << (8 * b);
      o++;
    }
  }
  *(uint32_t*)(dense + 4 * c) = out;
}

int launch_unpack(hipStream_t st, const uint8_t* packed, const uint8_t* mask, int32_t E, int32_t N, int32_t K,
                  uint8_t* dense, int32_t* dev_status) {
  // Chunks of consecutive rows are contiguous in all three arrays, so the [E][N] rows flatten.
  const int64_t nchunks = (int64_t)E * N * (K / 8);
  if (nchunks == 0) return MOESQ_OK;
  hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)((nchunks + 255) / 256)), dim3(256), 0, st, packed, mask, nchunks,
                     dense, dev_status);
  return hipGetLastError() == hipSuccess ? MOESQ_OK : MOESQ_ERR_HIP;
}

// ------------------------------------------------------------------ kernel layout -----------------
// Load-time repack of pair-bitmask v1 weights into the GEMM's fragment layout (same bytes, 2.75
// bits per weight). Fragment (e, rb, ss) covers rows 16rb..16rb+15 and K [256ss, +256) and holds,
// for lane l = 16c + r (row 16rb + r, K [256ss + 64c, +64)):
//   [16 l, +16)        the 16 packed bytes of the lane's eight 8-groups, each group's two kept
//                      bytes (b0, b1) rewritten as (lo b0 | lo b1 << 4, hi b0 | hi b1 << 4), so one
//                      FP4->f16 convert yields a de-interleaved 2:4 operand register;
//   [1024 + 4 l, +4)   the sparse-index codes (i | j << 2 of the kept pairs i < j) of the eight
//                      groups, one nibble each, in the group order 0, 2, 4, 6, 1, 3, 5, 7;
//   [1280 + 2 l, +2)   the 2 UE4M3 block-scale codes.
// Fragments are stored e-major, then rb, then ss, so one wave streams K with contiguous reads.
__global__ __launch_bounds__(256) void prepack_kernel(const uint8_t* __restrict__ packed,
                                                      const uint8_t* __restrict__ mask,
                                                      const uint8_t* __restrict__ scale, int32_t N, int32_t K,
                                                      int64_t nfrag, uint8_t* __restrict__ kl) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nfrag * 64) return;
  const int64_t frag = i >> 6;
  const int l = (int)(i & 63), r = l & 15, c = l >> 4;
  const int nss = K / 256;
  const int64_t ss = frag % nss;
  const int64_t rowblk = frag / nss;               // e * (N/16) + rb
  const int64_t row = rowblk * 16 + r;             // e * N + 16 rb + r
  const uint4 pk = *(const uint4*)(packed + row * (K / 4) + 64 * ss + 16 * c);
  const uint32_t w[4] = {pk.x, pk.y, pk.z, pk.w};
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    // two groups per word: bytes (b0, b1) of group 0 and (b2, b3) of group 1
    const uint32_t lo = w[j] & 0x0F0F0F0Fu, hi = (w[j] >> 4) & 0x0F0F0F0Fu;
    // lo holds (lo b0, lo b1, lo b2, lo b3) in the low nibbles of bytes 0..3; pack pairs of bytes
    const uint32_t l01 = (lo & 0xFFu) | ((lo >> 4) & 0xF0u);           // lo b0 | lo b1 << 4
    const uint32_t h01 = (hi & 0xFFu) | ((hi >> 4) & 0xF0u);
    const uint32_t l23 = ((lo >> 16) & 0xFFu) | ((lo >> 20) & 0xF0u);
    const uint32_t h23 = ((hi >> 16) & 0xFFu) | ((hi >> 20) & 0xF0u);
    o[j] = l01 | (h01 << 8) | (l23 << 16) | (h23 << 24);
  }
  // group of 4 fragments (64 rows) per super-step: fragment j = rowblk % 4
  const int j = (int)(rowblk & 3);
  uint8_t* F = kl + ((rowblk >> 2) * nss + ss) * (int64_t)kGroupBytes;
  *(uint4*)(F + 1024 * j + 16 * l) = make_uint4(o[0], o[1], o[2], o[3]);
  const uint32_t mk = *(const uint32_t*)(mask + row * (K / 16) + 16 * ss + 4 * c);
  uint32_t codes = 0u;
#pragma unroll
  for (int k = 0; k < 8; k++) {
    const int g = (k < 4) ? 2 * k : 2 * (k - 4) + 1;
    codes |= pair_index_code((mk >> (4 * g)) & 15u) << (4 * k);
  }
  *(uint32_t*)(F + 4096 + 16 * l + 4 * j) = codes;
  *(uint16_t*)(F + 5120 + 8 * l + 2 * j) = *(const uint16_t*)(scale + row * (K / 32) + 8 * ss + 2 * c);
}

int launch_prepack(hipStream_t st, const uint8_t* packed, const uint8_t* mask, const uint8_t* scale, int32_t E,
                   int32_t N, int32_t K, uint8_t* kl) {
  const int64_t nfrag = (int64_t)E * (N / 16) * (K / 256);
  if (nfrag == 0) return MOESQ_OK;
  hipLaunchKernelGGL(prepack_kernel, dim3((unsigned)((nfrag * 64 + 255) / 256)), dim3(256), 0, st, packed, mask, scale,
                     N, K, nfrag, kl);
  return hipGetLastError() == hipSuccess ? MOESQ_OK : MOESQ_ERR_HIP;
}

// Dense NVFP4 control layout (the unpruned counterpart of prepack_kernel's layout): per expert,
// 64-row group and 256-K super-step a 9216-byte unit. Fragment j's lane l = 16c + r owns the 32 bytes
// [2048 j + 32 l, +32): the code words of its 8-groups g(S, h) = 8 (c>>1) + 2 S + (c&1) + 16 h in the
// order (S0 h0, S0 h1, S1 h0, ..., S3 h1), each word's nibbles reordered to (0, 2, 4, 6, 1, 3, 5, 7);
// and the 4 bytes [8192 + 16 l + 4 j, +4): the scale codes of blocks 2q, 4+2q, 2q+1, 5+2q (q = c>>1)
// of the super-step.
constexpr int kDenseUnit = 9216;

MOESQ_DEV uint32_t operand_nibble_order(uint32_t w) {
  uint32_t o = 0u;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int src = i < 4 ? 2 * i : 2 * (i - 4) + 1;
    o |= ((w >> (4 * src)) & 15u) << (4 * i);
  }
  return o;
}

__global__ __launch_bounds__(256) void prepack_dense_kernel(const uint8_t* __restrict__ codes,
                                                            const uint8_t* __restrict__ scales, int32_t N, int32_t K,
                                                            int64_t nfrag, uint8_t* __restrict__ kl) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nfrag * 64) return;
  const int64_t frag = i >> 6;
  const int l = (int)(i & 63), r = l & 15, c = l >> 4, q = c >> 1;
  const int nss = K / 256;
  const int64_t ss = frag % nss;
  const int64_t rowblk = frag / nss;   // e * (N/16) + rb
  const int64_t row = rowblk * 16 + r;
  const int j = (int)(rowblk & 3);
  uint8_t* U = kl + ((rowblk >> 2) * nss + ss) * (int64_t)kDenseUnit;
  const uint8_t* src = codes + row * (K / 2) + 128 * ss;
  uint32_t o[8];
#pragma unroll
  for (int S = 0; S < 4; S++)
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const int g = 8 * q + 2 * S + (c & 1) + 16 * h;
      o[2 * S + h] = operand_nibble_order(*(const uint32_t*)(src + 4 * g));
    }
  *(uint4*)(U + 2048 * j + 32 * l) = make_uint4(o[0], o[1], o[2], o[3]);
  *(uint4*)(U + 2048 * j + 32 * l + 16) = make_uint4(o[4], o[5], o[6], o[7]);
  const uint8_t* b = scales + row * (K / 32) + 8 * ss;
  *(uint32_t*)(U + 8192 + 16 * l + 4 * j) =
      (uint32_t)b[2 * q] | ((uint32_t)b[4 + 2 * q] << 8) | ((uint32_t)b[2 * q + 1] << 16) | ((uint32_t)b[5 + 2 * q] << 24);
}

int launch_prepack_dense(hipStream_t st, const uint8_t* codes, const uint8_t* scales, int32_t E, int32_t N, int32_t K,
                         uint8_t* kl) {
  const int64_t nfrag = (int64_t)E * (N / 16) * (K / 256);
  if (nfrag == 0) return MOESQ_OK;
  hipLaunchKernelGGL(prepack_dense_kernel, dim3((unsigned)((nfrag * 64 + 255) / 256)), dim3(256), 0, st, codes, scales,
                     N, K, nfrag, kl);
  return hipGetLastError() == hipSuccess ? MOESQ_OK : MOESQ_ERR_HIP;
}

// ------------------------------------------------------------------ tensor scale (Eq. 5) ---------
// amax of a [rows][K] tensor (leading dimension ld) accumulated as float bits in out[0], then
// replaced in place by gamma = 448 / (amax / 6).
__global__ __launch_bounds__(256) void amax_rows_kernel(const void* __restrict__ x, int x_bf16, int64_t rows,
                                                        int32_t K, int64_t ld, int vec, uint32_t* __restrict__ out) {
  __shared__ float wmax[4];
  float m = 0.0f;
  if (vec) {
    m = amax_groups<4>(x, x_bf16, (int32_t)(rows * (K / 8)), K / 8, ld, blockIdx.x * 256 + threadIdx.x,
                       gridDim.x * 256);
  } else {
    const int64_t n = rows * (int64_t)K;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
      const int64_t r = i / K, c = i % K;
      const float v = x_bf16 ? bf16_bits_to_f32(((const uint16_t*)x)[r * ld + c]) : ((const float*)x)[r * ld + c];
      m = __builtin_fmaxf(m, __builtin_fabsf(v));
    }
  }
  m = block_max256(m, wmax);
  if (threadIdx.x == 0 && m > 0.0f) atomicMax(out, __float_as_uint(m));  // one device atomic per block
}

// Eq. 5 from the amax bits in out[0], written to out[0 .. n) (one block; the copies are written before
// out[0] is replaced, after a barrier).
__global__ void finalize_scale_kernel(uint32_t* out, int32_t n) {
  const float g = global_scale_from_amax(__uint_as_float(out[0]));
  __syncthreads();
  for (int i = threadIdx.x + 1; i < n; i += blockDim.x) out[i] = __float_as_uint(g);
  __syncthreads();
  if (threadIdx.x == 0) out[0] = __float_as_uint(g);
}

int launch_global_scale(hipStream_t st, const void* x, bool x_bf16, int64_t rows, int32_t K, int64_t ld,
                        float* gamma_out, int32_t n_out) {
  uint32_t* o = (uint32_t*)gamma_out;
  hipLaunchKernelGGL(zero_words_kernel, dim3(1), dim3(64), 0, st, o, 1);
  const int64_t n = rows * (int64_t)K;
  if (n > 0) {
    // 8-value vector loads when the rows allow them (and the 8-group count fits 32 bits)
    const bool vec = K % 8 == 0 && ld % 8 == 0 && ((uintptr_t)x % 16) == 0 && n / 8 < ((int64_t)1 << 31);
    const int64_t per = vec ? n / 8 : n;
    int64_t blocks = (per + 1023) / 1024;  // about 4 items per thread
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(amax_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, (int)x_bf16, rows, K, ld,
                       (int)vec, o);
  }
  hipLaunchKernelGGL(finalize_scale_kernel, dim3(1), dim3(256), 0, st, o, n_out);
  return hipGetLastError() == hipSuccess ? MOESQ_OK : MOESQ_ERR_HIP;
}

}  // namespace moesq
