// C ABI of libmoesq.so: argument validation on the host, then kernel launches on the caller's
// stream. No allocation, no synchronization, no host read of device data.
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "launch.h"

using namespace moesq;

// Workspace of moesq_expert_mlp_noalloc: a file-scope device array, one copy per GPU, held until the
// process ends. In host code `scratch` names a host-side stand-in, not the device copy: its device
// address comes from hipGetSymbolAddress, once per device with that device current, and only that
// address is handed to kernels.
static __device__ __align__(256) uint8_t scratch[MOESQ_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (looked up on the first call on that device), or nullptr.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool weights_ok(const moesq_weights* W) {
  return W && W->E > 0 && W->N > 0 && W->K > 0 && W->kl && W->gscale;
}

constexpr size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Capacity routing workspace: the prefix routing's own workspace, then its offsets [E+1], sorted slots
// [n] and slot positions [n], each region 256-byte aligned.
static size_t route_capacity_ws(int64_t n, int32_t E) {
  return align256(route_workspace_bytes(n, E)) + align256((size_t)(E + 1) * 4) + 2 * align256((size_t)n * 4);
}

// MLP workspace: h_q [rows][I/2], h_s [rows][I/32], h_k [rows][I] f16, then (dumps) the fp32 gate_up
// outputs [rows][2I] and the fp32 h [rows][I], each region starting on a 256-byte boundary.
size_t mlp_ws_base(int64_t rows, int32_t I) {
  return align256((size_t)rows * (I / 2)) + align256((size_t)rows * (I / 32)) + align256((size_t)rows * I * 2);
}
size_t mlp_ws(int64_t rows, int32_t I, bool dump) {
  size_t b = mlp_ws_base(rows, I);
  if (dump) b += align256((size_t)rows * 2 * I * sizeof(float)) + (size_t)rows * I * sizeof(float);
  return b;
}
// Calibration workspace: amax_h [E] f32, then gamma_h [E] f32 at the next 256-byte boundary.
size_t mlp_calib_ws(int32_t E) { return align256((size_t)E * 4) + (size_t)E * 4; }

}  // namespace

extern "C" {

int32_t moesq_version(void) { return 100; }

const char* moesq_status_str(int32_t status) {
  switch (status) {
    case MOESQ_OK: return "ok";
    case MOESQ_ERR_INVALID_ARG: return "invalid argument";
    case MOESQ_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MOESQ_ERR_WORKSPACE: return "workspace missing or too small";
    case MOESQ_ERR_PATTERN: return "invalid paired-4:8 pattern";
    case MOESQ_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

size_t moesq_workspace_bytes(int32_t kind, int64_t T, int32_t k, int32_t E, int32_t K, int32_t N, int32_t I) {
  (void)K;
  (void)N;
  switch (kind) {
    case MOESQ_WS_ROUTE: return (T > 0 && k > 0 && E > 0) ? route_workspace_bytes(T * k, E) : 0;
    case MOESQ_WS_MLP: return T >= 0 && I > 0 ? mlp_ws(T, I, false) : 0;
    case MOESQ_WS_MLP_DUMP: return T >= 0 && I > 0 ? mlp_ws(T, I, true) : 0;
    case MOESQ_WS_COMPRESS: return E > 0 ? (size_t)E * sizeof(uint32_t) : 0;
    case MOESQ_WS_ROUTE_CAPACITY: return (T >= 0 && k > 0 && E > 0) ? route_capacity_ws(T * k, E) : 0;
    case MOESQ_WS_MLP_CALIBRATE: return E > 0 ? mlp_calib_ws(E) : 0;
    default: return 0;
  }
}

int moesq_route_permute(void* stream, const int32_t* topk_ids, int64_t T, int32_t k, int32_t E, int32_t* counts,
                        int32_t* offsets, int32_t* sorted_slot, int32_t* slot_pos, void* workspace,
                        size_t workspace_bytes, int32_t* dev_status) {
  if (T < 0 || k <= 0 || E <= 0 || k > E) return MOESQ_ERR_INVALID_ARG;
  if (!counts || !offsets) return MOESQ_ERR_INVALID_ARG;
  if (T > 0 && (!topk_ids || !sorted_slot || !slot_pos)) return MOESQ_ERR_INVALID_ARG;
  if (E > kMaxExpertsRoute) return MOESQ_ERR_UNSUPPORTED;
  if (T * (int64_t)k >= ((int64_t)1 << 31)) return MOESQ_ERR_UNSUPPORTED;
  const size_t need = route_workspace_bytes(T * k, E);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 4))) return MOESQ_ERR_WORKSPACE;
  return launch_route((hipStream_t)stream, topk_ids, T * k, E, counts, offsets, sorted_slot, slot_pos, workspace,
                      dev_status);
}

int moesq_route_capacity(void* stream, const int32_t* topk_ids, int64_t T, int32_t k, int32_t E, int32_t capacity,
                         int32_t* counts, int32_t* slot_pos, void* workspace, size_t workspace_bytes,
                         int32_t* dev_status) {
  if (T < 0 || k <= 0 || E <= 0 || k > E || capacity <= 0) return MOESQ_ERR_INVALID_ARG;
  if (!counts) return MOESQ_ERR_INVALID_ARG;
  if (T > 0 && (!topk_ids || !slot_pos)) return MOESQ_ERR_INVALID_ARG;
  if (E > kMaxExpertsRoute) return MOESQ_ERR_UNSUPPORTED;
  if (T * (int64_t)k >= ((int64_t)1 << 31) || (int64_t)E * capacity >= ((int64_t)1 << 31)) return MOESQ_ERR_UNSUPPORTED;
  const int64_t n = T * k;
  const size_t need = route_capacity_ws(n, E);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return MOESQ_ERR_WORKSPACE;
  uint8_t* w = (uint8_t*)workspace;
  void* rws = w;
  int32_t* offs = (int32_t*)(w + align256(route_workspace_bytes(n, E)));
  int32_t* sorted = (int32_t*)((uint8_t*)offs + align256((size_t)(E + 1) * 4));
  int32_t* pos = (int32_t*)((uint8_t*)sorted + align256((size_t)n * 4));
  const int rc = launch_route((hipStream_t)stream, topk_ids, n, E, counts, offs, sorted, pos,
                              route_workspace_bytes(n, E) ? rws : nullptr, dev_status);
  if (rc != MOESQ_OK) return rc;
  return launch_capacity_slots((hipStream_t)stream, topk_ids, n, E, capacity, offs, pos, slot_pos);
}

int moesq_quantize_act(void* stream, const void* x, int32_t x_dtype, int64_t T, int32_t K, int64_t ld_x,
                       const int32_t* slot_pos, int32_t k, int64_t rows, const float* gamma, const int32_t* offsets,
                       int32_t E, uint8_t* q, uint8_t* s, void* xk) {
  if (x_dtype != MOESQ_F32 && x_dtype != MOESQ_BF16) return MOESQ_ERR_INVALID_ARG;
  if (T < 0 || rows < 0 || K <= 0 || K % 32 != 0 || ld_x < K) return MOESQ_ERR_INVALID_ARG;
  if (!gamma) return MOESQ_ERR_INVALID_ARG;
  if (T > 0 && (!x || !q || !s)) return MOESQ_ERR_INVALID_ARG;
  if (slot_pos) {
    if (k <= 0) return MOESQ_ERR_INVALID_ARG;
    if (rows < T * (int64_t)k) return MOESQ_ERR_INVALID_ARG;
    if (k > 512) return MOESQ_ERR_UNSUPPORTED;
  } else if (rows != T) {
    return MOESQ_ERR_INVALID_ARG;
  }
  if (offsets && E <= 0) return MOESQ_ERR_INVALID_ARG;
  if (offsets && E > 4096) return MOESQ_ERR_UNSUPPORTED;
  if (!offsets && E > 0 && (rows % E != 0 || rows == 0)) return MOESQ_ERR_INVALID_ARG;  // capacity layout
  if (rows >= ((int64_t)1 << 31) || T >= ((int64_t)1 << 31)) return MOESQ_ERR_UNSUPPORTED;
  if (ld_x % 8 != 0 || !aligned(x, 16) || !aligned(q, 4) || !aligned(xk, 16)) return MOESQ_ERR_UNSUPPORTED;
  return launch_quantize((hipStream_t)stream, x, x_dtype == MOESQ_BF16, T, K, ld_x, slot_pos, k, gamma, offsets, E,
                         q, s, xk, (!offsets && E > 0) ? (int32_t)(rows / E) : 0);
}

static int route_quantize_checked(void* stream, const int32_t* topk_ids, int64_t T, int32_t k, int32_t E,
                                  const void* x, int32_t x_dtype, int32_t K, int64_t ld_x, const float* gamma,
                                  float* gamma_out, int32_t* counts, int32_t* offsets, int32_t* sorted_slot,
                                  int32_t* slot_pos, void* workspace, size_t workspace_bytes, uint8_t* q, uint8_t* s,
                                  void* xk, int32_t* dev_status) {
  // routing arguments, as moesq_route_permute
  if (T < 0 || k <= 0 || E <= 0 || k > E) return MOESQ_ERR_INVALID_ARG;
  if (!counts || !offsets || !(gamma || gamma_out)) return MOESQ_ERR_INVALID_ARG;
  if (T > 0 && (!topk_ids || !sorted_slot || !slot_pos || !x || !q || !s)) return MOESQ_ERR_INVALID_ARG;
  if (E > kMaxExpertsRoute) return MOESQ_ERR_UNSUPPORTED;
  if (T * (int64_t)k >= ((int64_t)1 << 31)) return MOESQ_ERR_UNSUPPORTED;
  // quantizer arguments, as moesq_quantize_act with slot_pos and offsets
  if (x_dtype != MOESQ_F32 && x_dtype != MOESQ_BF16) return MOESQ_ERR_INVALID_ARG;
  if (K <= 0 || K % 32 != 0 || ld_x < K) return MOESQ_ERR_INVALID_ARG;
  if (k > 512) return MOESQ_ERR_UNSUPPORTED;
  if (ld_x % 8 != 0 || !aligned(x, 16) || !aligned(q, 4) || !aligned(xk, 16) || !aligned(gamma_out, 4))
    return MOESQ_ERR_UNSUPPORTED;
  if (!route_quantize_fused(T, k, E)) {
    const size_t need = route_workspace_bytes(T * k, E);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 4))) return MOESQ_ERR_WORKSPACE;
  }
  return launch_route_quantize((hipStream_t)stream, topk_ids, T, k, E, x, x_dtype == MOESQ_BF16, K, ld_x, gamma,
                               counts, offsets, sorted_slot, slot_pos, workspace, dev_status, q, s, xk, gamma_out);
}

int moesq_route_quantize(void* stream, const int32_t* topk_ids, int64_t T, int32_t k, int32_t E, const void* x,
                         int32_t x_dtype, int32_t K, int64_t ld_x, const float* gamma, int32_t* counts,
                         int32_t* offsets, int32_t* sorted_slot, int32_t* slot_pos, void* workspace,
                         size_t workspace_bytes, uint8_t* q, uint8_t* s, void* xk, int32_t* dev_status) {
  if (!gamma) return MOESQ_ERR_INVALID_ARG;
  return route_quantize_checked(stream, topk_ids, T, k, E, x, x_dtype, K, ld_x, gamma, nullptr, counts, offsets,
                                sorted_slot, slot_pos, workspace, workspace_bytes, q, s, xk, dev_status);
}

int moesq_route_quantize_dyn(void* stream, const int32_t* topk_ids, int64_t T, int32_t k, int32_t E, const void* x,
                             int32_t x_dtype, int32_t K, int64_t ld_x, float* gamma_out, int32_t* counts,
                             int32_t* offsets, int32_t* sorted_slot, int32_t* slot_pos, void* workspace,
                             size_t workspace_bytes, uint8_t* q, uint8_t* s, void* xk, int32_t* dev_status) {
  if (!gamma_out) return MOESQ_ERR_INVALID_ARG;
  return route_quantize_checked(stream, topk_ids, T, k, E, x, x_dtype, K, ld_x, nullptr, gamma_out, counts, offsets,
                                sorted_slot, slot_pos, workspace, workspace_bytes, q, s, xk, dev_status);
}

static int gemm_common(const moesq_weights* W, const uint8_t* q, const uint8_t* s, const void* xk,
                       const float* gamma_a, const int32_t* offsets, int64_t rows, void* y) {
  if (!weights_ok(W) || rows < 0 || !gamma_a || !offsets) return MOESQ_ERR_INVALID_ARG;
  if (rows > 0 && (!q || !s || !y)) return MOESQ_ERR_INVALID_ARG;
  if (W->K % 32 != 0) return MOESQ_ERR_INVALID_ARG;
  if (W->K % 256 != 0 || W->N % 64 != 0 || W->E > kMaxExpertsGemm) return MOESQ_ERR_UNSUPPORTED;
  if (W->gscale_split != 0 && W->gscale_split != 1) return MOESQ_ERR_INVALID_ARG;
  if (W->gscale_split && W->N % 128 != 0) return MOESQ_ERR_UNSUPPORTED;
  if (!aligned(W->kl, 16) || !aligned(q, 16) || !aligned(s, 2) || !aligned(y, 16) || !aligned(xk, 16))
    return MOESQ_ERR_UNSUPPORTED;
  if (xk && rows * W->K * 2 >= ((int64_t)1 << 31)) return MOESQ_ERR_UNSUPPORTED;
  if (rows >= ((int64_t)1 << 31)) return MOESQ_ERR_UNSUPPORTED;
  // 32-bit buffer offsets: one expert's weights, and all activation rows
  if ((int64_t)W->N * W->K / 32 * 11 >= ((int64_t)1 << 31) || rows * (W->K / 2) >= ((int64_t)1 << 31))
    return MOESQ_ERR_UNSUPPORTED;
  return MOESQ_OK;
}

// MOESQ_F_CAPACITY: offsets holds counts[E] and the rows form E blocks of rows / E (the capacity).
int moesq_route_quantize_gemm(void* stream, const int32_t* topk_ids, int64_t T, int32_t k, int32_t E,
                              const void* x, int32_t x_dtype, int32_t K, int64_t ld_x, const float* gamma_a,
                              const moesq_weights* W, int32_t* counts, int32_t* offsets, int32_t* sorted_slot,
                              int32_t* slot_pos, void* workspace, size_t workspace_bytes, uint8_t* q, uint8_t* s,
                              void* xk, void* y, int32_t y_dtype, int32_t* dev_status) {
  if (y_dtype != MOESQ_F32 && y_dtype != MOESQ_BF16) return MOESQ_ERR_INVALID_ARG;
  if (!W || W->E != E || W->K != K) return MOESQ_ERR_INVALID_ARG;
  const int64_t rows = T * (int64_t)k;
  // the two calls' argument checks, all before anything is enqueued
  if (T < 0 || k <= 0 || E <= 0 || k > E) return MOESQ_ERR_INVALID_ARG;
  int rc = gemm_common(W, q, s, xk, gamma_a, offsets, rows, y);
  if (rc != MOESQ_OK) return rc;
  if (!counts) return MOESQ_ERR_INVALID_ARG;
  if (T > 0 && (!topk_ids || !sorted_slot || !slot_pos || !x)) return MOESQ_ERR_INVALID_ARG;
  if (E > kMaxExpertsRoute) return MOESQ_ERR_UNSUPPORTED;
  if (x_dtype != MOESQ_F32 && x_dtype != MOESQ_BF16) return MOESQ_ERR_INVALID_ARG;
  if (ld_x < K) return MOESQ_ERR_INVALID_ARG;
  if (k > 512) return MOESQ_ERR_UNSUPPORTED;
  if (ld_x % 8 != 0 || !aligned(x, 16) || !aligned(q, 4)) return MOESQ_ERR_UNSUPPORTED;
  hipStream_t st = (hipStream_t)stream;
  if (!dispatch_gemm_fused(T, k, E, K)) {
    if (!route_quantize_fused(T, k, E)) {
      const size_t need = route_workspace_bytes(rows, E);
      if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 4))) return MOESQ_ERR_WORKSPACE;
    }
    rc = launch_route_quantize(st, topk_ids, T, k, E, x, x_dtype == MOESQ_BF16, K, ld_x, gamma_a, counts, offsets,
                               sorted_slot, slot_pos, workspace, dev_status, q, s, xk);
    if (rc != MOESQ_OK) return rc;
  }
  GemmArgs a{};
  a.kl = W->kl; a.gscale = W->gscale;
  a.q = q; a.s = s; a.xk = xk; a.gamma_a = gamma_a; a.offsets = offsets; a.y = y;
  a.E = W->E; a.N = W->N; a.K = W->K; a.y_bf16 = y_dtype == MOESQ_BF16; a.gsplit = W->gscale_split;
  if (dispatch_gemm_fused(T, k, E, K))
    return launch_dispatch_gemm(st, a, topk_ids, T, k, x, x_dtype == MOESQ_BF16, ld_x, counts, offsets, sorted_slot,
                                slot_pos, dev_status, q, s, xk);
  return launch_gemm(st, a, rows);
}

static int capacity_of(uint32_t flags, int32_t E, int64_t rows, int32_t& cap) {
  cap = 0;
  if (!(flags & MOESQ_F_CAPACITY)) return MOESQ_OK;
  if (rows % E != 0) return MOESQ_ERR_INVALID_ARG;
  cap = (int32_t)(rows / E);
  return MOESQ_OK;
}

int moesq_grouped_gemm(void* stream, const moesq_weights* W, const uint8_t* q, const uint8_t* s, const void* xk,
                       const float* gamma_a, const int32_t* offsets, int64_t rows, void* y, int32_t y_dtype,
                       uint32_t flags) {
  if (y_dtype != MOESQ_F32 && y_dtype != MOESQ_BF16) return MOESQ_ERR_INVALID_ARG;
  const int rc = gemm_common(W, q, s, xk, gamma_a, offsets, rows, y);
  if (rc != MOESQ_OK) return rc;
  GemmArgs a{};
  a.kl = W->kl; a.gscale = W->gscale;
  a.q = q; a.s = s; a.xk = xk; a.gamma_a = gamma_a; a.offsets = offsets; a.y = y;
  a.E = W->E; a.N = W->N; a.K = W->K; a.y_bf16 = y_dtype == MOESQ_BF16; a.gsplit = W->gscale_split;
  if (capacity_of(flags, W->E, rows, a.cap) != MOESQ_OK) return MOESQ_ERR_INVALID_ARG;
  if (flags & MOESQ_F_FORCE_DECODE) return launch_gemm_variant((hipStream_t)stream, a, rows, 0);
  if (flags & MOESQ_F_FORCE_PREFILL) return launch_gemm_variant((hipStream_t)stream, a, rows, 1);
  return launch_gemm((hipStream_t)stream, a, rows);
}

int moesq_expert_mlp(void* stream, const moesq_weights* W13, const moesq_weights* W2, const uint8_t* q,
                     const uint8_t* s, const void* xk, const float* gamma_a, const float* gamma_h,
                     const int32_t* offsets, int64_t rows, void* y, int32_t y_dtype, void* workspace,
                     size_t workspace_bytes, uint32_t flags) {
  const bool calib = (flags & MOESQ_F_CALIBRATE) != 0;
  const bool dump = (flags & (MOESQ_F_DUMP_GATEUP | MOESQ_F_DUMP_H)) != 0;
  if (y_dtype != MOESQ_F32 && y_dtype != MOESQ_BF16) return MOESQ_ERR_INVALID_ARG;
  if (!weights_ok(W13) || !weights_ok(W2) || (!gamma_h && !calib)) return MOESQ_ERR_INVALID_ARG;
  if (calib && dump) return MOESQ_ERR_INVALID_ARG;
  const int32_t I = W13->N / 2;
  if (W13->N % 2 != 0 || W2->K != I || W2->E != W13->E) return MOESQ_ERR_INVALID_ARG;
  // y is neither read nor written in calibration: a host placeholder stands in for the common checks
  alignas(16) static const float no_output[4] = {0.f, 0.f, 0.f, 0.f};
  int rc = gemm_common(W13, q, s, xk, gamma_a, offsets, rows, calib ? (void*)no_output : y);
  if (rc != MOESQ_OK) return rc;
  if (I % 256 != 0 || W13->K % 256 != 0 || W2->N % 64 != 0) return MOESQ_ERR_UNSUPPORTED;
  if (W2->gscale_split != 0 && W2->gscale_split != 1) return MOESQ_ERR_INVALID_ARG;
  if (W2->gscale_split && W2->N % 128 != 0) return MOESQ_ERR_UNSUPPORTED;
  if (!aligned(W2->kl, 16)) return MOESQ_ERR_UNSUPPORTED;
  if ((int64_t)W2->N * W2->K / 32 * 11 >= ((int64_t)1 << 31) || rows * (I / 2) >= ((int64_t)1 << 31))
    return MOESQ_ERR_UNSUPPORTED;
  const size_t need = calib ? mlp_calib_ws(W13->E) : mlp_ws(rows, I, dump);
  if ((rows > 0 || calib) && (!workspace || workspace_bytes < need || !aligned(workspace, 256)))
    return MOESQ_ERR_WORKSPACE;
  if (rows * (int64_t)I * 2 >= ((int64_t)1 << 31)) return MOESQ_ERR_UNSUPPORTED;
  GemmArgs a{};
  a.kl = W13->kl; a.gscale = W13->gscale;
  a.q = q; a.s = s; a.xk = xk; a.gamma_a = gamma_a; a.offsets = offsets; a.y = nullptr;
  a.E = W13->E; a.N = W13->N; a.K = W13->K; a.y_bf16 = 0; a.gsplit = W13->gscale_split;
  if (capacity_of(flags, W13->E, rows, a.cap) != MOESQ_OK) return MOESQ_ERR_INVALID_ARG;
  // few tokens per expert: both GEMMs stream the weights; otherwise both are tiled
  int variant = rows <= (int64_t)16 * W13->E ? 0 : 1;
  if (flags & MOESQ_F_FORCE_DECODE) variant = 0;
  if (flags & MOESQ_F_FORCE_PREFILL) variant = 1;
  if (calib) {
    uint32_t* amax = (uint32_t*)workspace;
    float* gam = (float*)((uint8_t*)workspace + align256((size_t)W13->E * 4));
    return launch_calibrate_h((hipStream_t)stream, a, rows, variant, amax, gam);
  }
  if (rows == 0) return MOESQ_OK;
  uint8_t* hq = (uint8_t*)workspace;
  uint8_t* hs = hq + align256((size_t)rows * (I / 2));
  uint8_t* hk = hs + align256((size_t)rows * (I / 32));
  uint8_t* dumps = (uint8_t*)workspace + mlp_ws_base(rows, I);
  a.gamma_h = gamma_h; a.h_q = hq; a.h_s = hs;
  a.dump = (flags & MOESQ_F_DUMP_GATEUP) ? (float*)dumps : nullptr;
  a.hdump = (flags & MOESQ_F_DUMP_H) ? (float*)(dumps + align256((size_t)rows * 2 * I * sizeof(float))) : nullptr;
  // The weight-streaming down GEMM reads h from its f16 copy; the tiled one stages h from the NVFP4 codes
  // (at c4 the gate_up without the copy's 268 MB of stores is 4.5% faster and the down GEMM 3% slower, the
  // step 2.3% faster), so the tiled gate_up writes the copy only with the stage dumps, for their checks.
  const bool tiled = variant != 0;
  a.h_k = (!tiled || a.dump || a.hdump) ? hk : nullptr;
  rc = launch_gemm_variant((hipStream_t)stream, a, rows, variant);
  if (rc != MOESQ_OK) return rc;
  GemmArgs b{};
  b.kl = W2->kl; b.gscale = W2->gscale;
  b.q = hq; b.s = hs; b.xk = tiled ? nullptr : hk; b.gamma_a = gamma_h; b.offsets = offsets; b.y = y;
  b.E = W2->E; b.N = W2->N; b.K = W2->K; b.y_bf16 = y_dtype == MOESQ_BF16; b.gsplit = W2->gscale_split;
  b.cap = a.cap;
  return launch_gemm_variant((hipStream_t)stream, b, rows, variant);
}

int moesq_expert_mlp_noalloc(void* stream, const moesq_weights* W13, const moesq_weights* W2, const uint8_t* q,
                             const uint8_t* s, const void* xk, const float* gamma_a, const float* gamma_h,
                             const int32_t* offsets, int64_t rows, void* y, int32_t y_dtype, uint32_t flags) {
  if (!W13 || W13->N <= 0 || W13->N % 2 != 0 || rows < 0) return MOESQ_ERR_INVALID_ARG;
  // the dumps and the calibration write into the workspace, which the caller cannot see here
  if (flags & (MOESQ_F_DUMP_GATEUP | MOESQ_F_DUMP_H | MOESQ_F_CALIBRATE)) return MOESQ_ERR_INVALID_ARG;
  if (mlp_ws(rows, W13->N / 2, false) > (size_t)MOESQ_NOALLOC_SCRATCH_BYTES) return MOESQ_ERR_WORKSPACE;
  void* ws = scratch_on_current_device();
  if (!ws) return MOESQ_ERR_HIP;
  return moesq_expert_mlp(stream, W13, W2, q, s, xk, gamma_a, gamma_h, offsets, rows, y, y_dtype, ws,
                          MOESQ_NOALLOC_SCRATCH_BYTES, flags);
}

int moesq_unpermute_combine(void* stream, const void* y_sorted, int32_t y_dtype, const int32_t* slot_pos,
                            const float* topk_w, int64_t T, int32_t k, int32_t H, void* out, int32_t out_dtype) {
  if ((y_dtype != MOESQ_F32 && y_dtype != MOESQ_BF16) || (out_dtype != MOESQ_F32 && out_dtype != MOESQ_BF16))
    return MOESQ_ERR_INVALID_ARG;
  if (T < 0 || k <= 0 || H <= 0) return MOESQ_ERR_INVALID_ARG;
  if (T > 0 && (!y_sorted || !slot_pos || !topk_w || !out)) return MOESQ_ERR_INVALID_ARG;
  if (H % 8 != 0 || !aligned(y_sorted, 16) || !aligned(out, 16)) return MOESQ_ERR_UNSUPPORTED;
  return launch_combine((hipStream_t)stream, y_sorted, y_dtype == MOESQ_BF16, slot_pos, topk_w, T, k, H, out,
                        out_dtype == MOESQ_BF16);
}

int moesq_global_scale(void* stream, const void* x, int32_t x_dtype, int64_t rows, int32_t K, int64_t ld_x,
                       float* gamma_out) {
  if (x_dtype != MOESQ_F32 && x_dtype != MOESQ_BF16) return MOESQ_ERR_INVALID_ARG;
  if (rows < 0 || K <= 0 || ld_x < K || !gamma_out || (rows > 0 && !x)) return MOESQ_ERR_INVALID_ARG;
  if (!aligned(gamma_out, 4)) return MOESQ_ERR_UNSUPPORTED;
  return launch_global_scale((hipStream_t)stream, x, x_dtype == MOESQ_BF16, rows, K, ld_x, gamma_out);
}

int moesq_compress_weights(void* stream, const float* w, int32_t E, int32_t N, int32_t K, uint8_t* packed,
                           uint8_t* mask, uint8_t* scale, float* gscale, void* workspace, size_t workspace_bytes,
                           int32_t* dev_status) {
  if (E <= 0 || N <= 0 || K <= 0 || K % 32 != 0) return MOESQ_ERR_INVALID_ARG;
  if (!w || !packed || !mask || !scale || !gscale) return MOESQ_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < (size_t)E * sizeof(uint32_t) || !aligned(workspace, 4))
    return MOESQ_ERR_WORKSPACE;
  if (!aligned(w, 16) || !aligned(packed, 8) || !aligned(mask, 2)) return MOESQ_ERR_UNSUPPORTED;
  return launch_compress((hipStream_t)stream, w, E, N, K, packed, mask, scale, gscale, workspace, dev_status);
}

size_t moesq_kernel_layout_bytes(int32_t E, int32_t N, int32_t K) {
  if (E <= 0 || N <= 0 || K <= 0) return 0;
  return (size_t)E * (size_t)N * (size_t)K / 32 * 11;
}

int moesq_prepack_weights(void* stream, const moesq_weights* W, uint8_t* kl, size_t kl_bytes) {
  if (!W || W->E <= 0 || W->N <= 0 || W->K <= 0 || !W->packed || !W->mask || !W->scale || !kl)
    return MOESQ_ERR_INVALID_ARG;
  if (W->K % 32 != 0) return MOESQ_ERR_INVALID_ARG;
  if (W->K % 256 != 0 || W->N % 64 != 0) return MOESQ_ERR_UNSUPPORTED;
  if (kl_bytes < moesq_kernel_layout_bytes(W->E, W->N, W->K)) return MOESQ_ERR_WORKSPACE;
  if (!aligned(kl, 16) || !aligned(W->packed, 16) || !aligned(W->mask, 4) || !aligned(W->scale, 2))
    return MOESQ_ERR_UNSUPPORTED;
  return launch_prepack((hipStream_t)stream, W->packed, W->mask, W->scale, W->E, W->N, W->K, kl);
}

size_t moesq_dense_layout_bytes(int32_t E, int32_t N, int32_t K) {
  if (E <= 0 || N <= 0 || K <= 0) return 0;
  return (size_t)E * (size_t)N * (size_t)K / 16 * 9;
}

int moesq_prepack_dense_weights(void* stream, int32_t E, int32_t N, int32_t K, const uint8_t* codes,
                                const uint8_t* scales, uint8_t* kl, size_t kl_bytes) {
  if (E <= 0 || N <= 0 || K <= 0 || !codes || !scales || !kl) return MOESQ_ERR_INVALID_ARG;
  if (K % 32 != 0) return MOESQ_ERR_INVALID_ARG;
  if (K % 256 != 0 || N % 64 != 0) return MOESQ_ERR_UNSUPPORTED;
  if (kl_bytes < moesq_dense_layout_bytes(E, N, K)) return MOESQ_ERR_WORKSPACE;
  if (!aligned(kl, 16) || !aligned(codes, 4)) return MOESQ_ERR_UNSUPPORTED;
  return launch_prepack_dense((hipStream_t)stream, codes, scales, E, N, K, kl);
}

int moesq_dense_grouped_gemm(void* stream, const moesq_weights* W, const uint8_t* q, const uint8_t* s, const void* xk,
                             const float* gamma_a, const int32_t* offsets, int64_t rows, void* y, int32_t y_dtype,
                             uint32_t flags) {
  if (y_dtype != MOESQ_F32 && y_dtype != MOESQ_BF16) return MOESQ_ERR_INVALID_ARG;
  const int rc = gemm_common(W, q, s, xk, gamma_a, offsets, rows, y);
  if (rc != MOESQ_OK) return rc;
  if ((int64_t)W->N * W->K / 16 * 9 >= ((int64_t)1 << 31)) return MOESQ_ERR_UNSUPPORTED;
  if (W->gscale_split) return MOESQ_ERR_UNSUPPORTED;  // the dense control has one tensor scale per expert
  GemmArgs a{};
  a.kl = W->kl; a.gscale = W->gscale;
  a.q = q; a.s = s; a.xk = xk; a.gamma_a = gamma_a; a.offsets = offsets; a.y = y;
  a.E = W->E; a.N = W->N; a.K = W->K; a.y_bf16 = y_dtype == MOESQ_BF16;
  if (capacity_of(flags, W->E, rows, a.cap) != MOESQ_OK) return MOESQ_ERR_INVALID_ARG;
  int variant = rows <= (int64_t)16 * W->E ? 0 : 1;
  if (flags & MOESQ_F_FORCE_DECODE) variant = 0;
  if (flags & MOESQ_F_FORCE_PREFILL) variant = 1;
  return launch_dense_gemm((hipStream_t)stream, a, rows, variant);
}

int moesq_unpack_weights(void* stream, const moesq_weights* W, uint8_t* dense_nvfp4, int32_t* dev_status) {
  if (!W || W->E <= 0 || W->N <= 0 || W->K <= 0 || W->K % 32 != 0 || !W->packed || !W->mask || !dense_nvfp4)
    return MOESQ_ERR_INVALID_ARG;
  if (!aligned(dense_nvfp4, 4)) return MOESQ_ERR_UNSUPPORTED;
  return launch_unpack((hipStream_t)stream, W->packed, W->mask, W->E, W->N, W->K, dense_nvfp4, dev_status);
}

}  // extern "C"
