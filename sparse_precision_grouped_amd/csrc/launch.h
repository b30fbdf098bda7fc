// Host-side launchers of the kernels (one per translation unit) and shared limits.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moesq.h"

namespace moesq {

constexpr int64_t kRouteSingleMax = 2048;  // slots handled by the one-workgroup routing path
constexpr int32_t kMaxExpertsRoute = 512;
constexpr int32_t kFusedRouteMaxK = 32;    // top-k handled by the fused route + quantize kernel
constexpr int64_t kDynScaleMaxBytes = 256 * 1024;  // token bytes each fused workgroup scans for the dynamic scale
constexpr int32_t kMaxExpertsGemm = 1024;

constexpr int kFragBytes = 1408;  // 16 rows x 256 K of the kernel weight layout
constexpr int kGroupBytes = 4 * kFragBytes;  // 4 fragments (64 rows x 256 K): the layout unit

struct GemmArgs {
  const uint8_t* kl;      // kernel layout [E][N/16][K/256][1408 B]
  const float* gscale;    // [E]
  const uint8_t* q;       // [rows][K/2]
  const uint8_t* s;       // [rows][K/32]
  const void* xk;         // [rows][K] f16 activations in the kernel's group order, or nullptr
  const float* gamma_a;   // [E]
  const int32_t* offsets; // [E+1]
  void* y;                // [rows][N] (plain epilogue)
  int32_t E, N, K;
  int32_t y_bf16;
  int32_t gsplit;         // gscale holds (rows < N/2, rows >= N/2) pairs per expert
  int32_t cap;            // > 0: capacity layout, offsets holds counts[E] and expert e's rows start at e * cap
  // MLP gate_up epilogue (N = 2I): SwiGLU + requant into h_q [rows][I/2], h_s [rows][I/32]
  const float* gamma_h;   // [E] or nullptr for the plain epilogue
  uint8_t* h_q;
  uint8_t* h_s;
  void* h_k;              // [rows][I] f16 copy of the requantized h in the kernel's group order, or nullptr
  float* dump;            // [rows][N] fp32 gate_up outputs, or nullptr
  float* hdump;           // [rows][I] fp32 h = SiLU(g) * u (the values the requantization reads), or nullptr
  uint32_t* amax_h;       // calibration: [E] per-expert amax(h) as float bits (atomic max; zeroed by the caller);
                          // when set the epilogue writes no h codes, scales or copies
  int32_t lut_cap;        // tiled kernel (set by its launcher): LDS entries of the full-token-tile -> expert table
};

size_t route_workspace_bytes(int64_t n, int32_t E);
int launch_route(hipStream_t st, const int32_t* ids, int64_t n, int32_t E, int32_t* counts, int32_t* offsets,
                 int32_t* sorted_slot, int32_t* slot_pos, void* ws, int32_t* dev_status);

// cap > 0 (with offsets == nullptr): rows are in the capacity layout, row p belongs to expert p / cap.
int launch_quantize(hipStream_t st, const void* x, bool x_bf16, int64_t T, int32_t K, int64_t ld_x,
                    const int32_t* slot_pos, int32_t k, const float* gamma, const int32_t* offsets, int32_t E,
                    uint8_t* q, uint8_t* s, void* xk, int32_t cap = 0);
// Capacity-layout slot positions from the prefix routing: e * cap + rank, or -1 past the capacity.
int launch_capacity_slots(hipStream_t st, const int32_t* ids, int64_t n, int32_t E, int32_t cap,
                          const int32_t* offsets, const int32_t* slot_pos_prefix, int32_t* slot_pos);
// Routing + scatter quantization: one fused launch when route_quantize_fused(T, k, E), else the
// routing kernels followed by the quantizer (ws = the routing workspace). With gamma_out the
// activation tensor scale is computed on the device (Eq. 5 over all of x) and written to gamma_out[E]
// (gamma is then not read): inside the fused launch when route_quantize_dyn_fused, else by the amax
// pre-pass first.
bool route_quantize_fused(int64_t T, int32_t k, int32_t E);
bool route_quantize_dyn_fused(int64_t T, int32_t k, int32_t E, int32_t K, bool x_bf16);
int launch_route_quantize(hipStream_t st, const int32_t* ids, int64_t T, int32_t k, int32_t E, const void* x,
                          bool x_bf16, int32_t K, int64_t ld_x, const float* gamma, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_slot, int32_t* slot_pos, void* ws, int32_t* dev_status,
                          uint8_t* q, uint8_t* s, void* xk, float* gamma_out = nullptr);

int launch_prepack_dense(hipStream_t st, const uint8_t* codes, const uint8_t* scales, int32_t E, int32_t N, int32_t K,
                         uint8_t* kl);
int launch_dense_gemm(hipStream_t st, const GemmArgs& a, int64_t rows, int variant);

// Eq. 5 scale of a whole tensor, written to gamma_out[0 .. n_out).
int launch_global_scale(hipStream_t st, const void* x, bool x_bf16, int64_t rows, int32_t K, int64_t ld,
                        float* gamma_out, int32_t n_out = 1);

int launch_compress(hipStream_t st, const float* w, int32_t E, int32_t N, int32_t K, uint8_t* packed, uint8_t* mask,
                    uint8_t* scale, float* gscale, void* ws, int32_t* dev_status);
int launch_prepack(hipStream_t st, const uint8_t* packed, const uint8_t* mask, const uint8_t* scale, int32_t E,
                   int32_t N, int32_t K, uint8_t* kl);
int launch_unpack(hipStream_t st, const uint8_t* packed, const uint8_t* mask, int32_t E, int32_t N, int32_t K,
                  uint8_t* dense, int32_t* dev_status);

// Grouped GEMM: picks the decode (weight-streaming) or the prefill (tiled) kernel from rows / E.
int launch_gemm(hipStream_t st, const GemmArgs& a, int64_t rows);
// variant 0 = decode (weight streaming; with gamma_h the MLP gate_up epilogue), 1 = prefill (tiled).
int launch_gemm_variant(hipStream_t st, const GemmArgs& a, int64_t rows, int variant);
// Calibration of the intermediate tensor scales: zero amax_bits [E], run the MLP gate_up GEMM of `a`
// (a.amax_h = amax_bits) with the given variant, then gamma_h[e] = Eq. 5 of amax_bits[e].
int launch_calibrate_h(hipStream_t st, GemmArgs a, int64_t rows, int variant, uint32_t* amax_bits, float* gamma_h);

// Route + quantize + decode GEMM in one launch for small decode batches (dispatch_gemm_fused): the
// same outputs as launch_route_quantize followed by the default weight-streaming GEMM with xk.
bool dispatch_gemm_fused(int64_t T, int32_t k, int32_t E, int32_t K);
int launch_dispatch_gemm(hipStream_t st, const GemmArgs& a, const int32_t* ids, int64_t T, int32_t k, const void* x,
                         bool x_bf16, int64_t ld_x, int32_t* counts, int32_t* offsets, int32_t* sorted_slot,
                         int32_t* slot_pos, int32_t* dev_status, uint8_t* q, uint8_t* s, void* xk);

int launch_combine(hipStream_t st, const void* y, bool y_bf16, const int32_t* slot_pos, const float* w, int64_t T,
                   int32_t k, int32_t H, void* out, bool out_bf16);

}  // namespace moesq
