/*
 * moesq.h -- C ABI of the MI355X (gfx950) library for the Mixture-of-Experts expert path over
 * paired-4:8 sparse NVFP4 weights ("libmoesq.so").
 *
 * Source of the method: paper "Hardware-Native Joint Sparse-Quantization for Trillion-Scale
 * Mixture-of-Experts" (arxiv 2610.02241), Section 3.4 (Eq. 5, grouped sparse GEMM execution),
 * Appendix A (feasible set, storage cost), Appendix D.1 (operand layout, scheduling, serving
 * integration); model card "Kimi-K2.5-P48NVFP4-MoESQ" (compression details, sparse storage layout
 * "pair-bitmask v1").
 *
 * Conventions for every call
 *  - Pointers to tensors are DEVICE pointers unless a comment says "host". The caller allocates and
 *    owns every buffer (including workspace); the library never allocates, frees, or keeps a pointer
 *    after the call returns.
 *  - `stream` is a hipStream_t passed as void*. Every call only enqueues work on that stream: no
 *    host/device synchronization, no host read of device data, so calls can be captured in a HIP
 *    graph. Results are ready when the stream reaches them.
 *  - Return value: MOESQ_OK (0) or a negative status. Host-side argument validation happens before
 *    anything is enqueued; on error nothing is launched. Conditions that only the device can see
 *    (bad expert ids, invalid mask nibbles) are written to an optional device status word.
 *  - Tensors are row-major and densely packed unless a leading dimension is given.
 *  - FP4 codes: E2M1, sign in bit 3, magnitude index in bits 0..2 of the grid
 *    {0, 0.5, 1, 1.5, 2, 3, 4, 6}; two codes per byte, the lower K index in the low nibble.
 *    Block scales: UE4M3 codes (E4M3 with bias 7, largest value 448), one per 32 consecutive K.
 *    Tensor scales: fp32 gamma of Eq. 5; a dequantized value is e2m1 * e4m3 / gamma.
 *  - Thread safety: stateless; calls on different streams may run concurrently.
 */
#ifndef MOESQ_H
#define MOESQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------------------------------- */
#define MOESQ_OK 0
#define MOESQ_ERR_INVALID_ARG -1 /* null pointer, non-positive size, K % 32 != 0, k > E, ... */
#define MOESQ_ERR_UNSUPPORTED -2 /* valid but not handled by the kernels (e.g. K % 256 != 0)     */
#define MOESQ_ERR_WORKSPACE -3   /* workspace pointer missing or smaller than required           */
#define MOESQ_ERR_PATTERN -4     /* (device status) chunk with > 2 nonzero bytes, or mask nibble  */
                                 /* whose popcount is not 2                                       */
#define MOESQ_ERR_HIP -5         /* a kernel launch failed (hipGetLastError)                      */

/* ---- dtypes ------------------------------------------------------------------------------------ */
#define MOESQ_F32 0
#define MOESQ_BF16 1

/* ---- flags ------------------------------------------------------------------------------------ */
#define MOESQ_F_DUMP_GATEUP 1u   /* moesq_expert_mlp: also write the fp32 gate_up outputs (after alpha)
                                    to the workspace region described at moesq_expert_mlp */
#define MOESQ_F_FORCE_DECODE 2u  /* moesq_grouped_gemm: use the weight-streaming (decode) kernel */
#define MOESQ_F_FORCE_PREFILL 4u /* moesq_grouped_gemm: use the tiled (prefill) kernel; without either
                                    flag the kernel is chosen from rows / E (<= 16: decode) */
#define MOESQ_F_DUMP_H 16u       /* moesq_expert_mlp: also write the fp32 h = SiLU(g) * u that the gate_up
                                    epilogue requantizes, to the workspace region described at
                                    moesq_expert_mlp (for checking the requantization on identical inputs) */
#define MOESQ_F_CALIBRATE 32u    /* moesq_expert_mlp: calibrate the intermediate tensor scales instead of
                                    running the MLP (see moesq_expert_mlp) */
#define MOESQ_F_CAPACITY 8u      /* moesq_grouped_gemm, moesq_expert_mlp, moesq_dense_grouped_gemm: the
                                    activations and outputs are in the fixed-capacity layout of paper
                                    Appendix D.1 (expert e owns rows [e*C, (e+1)*C), C = rows / E, rows
                                    % E == 0) and `offsets` points to the token counts [E] instead: the
                                    first min(count, C) rows of each block are used, the others are
                                    padding, neither read nor written (moesq_route_capacity builds the
                                    layout's slot positions) */

/* ---- workspace query kinds --------------------------------------------------------------------- */
#define MOESQ_WS_ROUTE 1
#define MOESQ_WS_MLP 2
#define MOESQ_WS_MLP_DUMP 3
#define MOESQ_WS_COMPRESS 4
#define MOESQ_WS_ROUTE_CAPACITY 5
#define MOESQ_WS_MLP_CALIBRATE 6

/*
 * Compressed weights of one projection for E experts, pair-bitmask v1 layout (model card, "Sparse
 * storage layout"): per expert e a row-major [N][K] weight W_e (N = output features, K = contraction)
 * stored as
 *   packed [E][N][K/4]  the two kept dense-NVFP4 bytes of every 4-byte chunk, in K order
 *                       (one byte = one adjacent pair of E2M1 codes)
 *   mask   [E][N][K/16] 4 bits per chunk, bit i = byte i kept, exactly two bits set,
 *                       low nibble = lower-K chunk
 *   scale  [E][N][K/32] UE4M3 block-scale codes
 *   gscale [E]          fp32 tensor scale gamma_w,e of Eq. 5 (gscale_split = 0), or
 *          [E][2]       with gscale_split = 1: the scales of rows [0, N/2) and [N/2, N), for a gate_up
 *                       weight whose gate and up projections are separate linears with their own
 *                       Eq. 5 scale (the model card's checkpoint); needs N % 128 == 0. Compressing the
 *                       [2E][N/2][K] view of the same weights produces it: the byte layout of packed,
 *                       mask and scale is the same.
 *   kl                  the same weights in the kernel layout (moesq_prepack_weights), read by the
 *                       GEMM calls; moesq_kernel_layout_bytes(E, N, K) bytes, 16-byte aligned
 * The GEMM calls read only kl and gscale (packed/mask/scale may then be NULL); the storage calls
 * (prepack, unpack) read packed/mask/scale. The struct itself lives in host memory; its pointers
 * are device pointers read during the call.
 */
typedef struct {
  int32_t E, N, K;
  const uint8_t *packed;
  const uint8_t *mask;
  const uint8_t *scale;
  const float *gscale;
  const uint8_t *kl;
  int32_t gscale_split;  /* 0 or 1, see gscale */
} moesq_weights;

/*
 * Routing / dispatch planning (paper Appendix D.1: token counts stay on the device; the persistent
 * scheduler reads them there). Per-expert histogram of topk_ids, exclusive prefix scan, and a
 * stable scatter of the flat slots f = t*k + j into expert-sorted order.
 *   topk_ids    [T][k] int32 expert ids in [0, E)
 *   counts      [E]    tokens routed to each expert
 *   offsets     [E+1]  exclusive prefix sum of counts (offsets[E] = number of placed slots)
 *   sorted_slot [T*k]  permuted row p holds slot sorted_slot[p]; slots of one expert keep
 *                      ascending f (stable)
 *   slot_pos    [T*k]  inverse: slot f sits at permuted row slot_pos[f]; -1 for an invalid id
 * Ids outside [0, E) are dropped (not counted, slot_pos = -1) and, if dev_status is not NULL,
 * MOESQ_ERR_INVALID_ARG is written to *dev_status (which the caller zero-initializes).
 * Workspace: moesq_workspace_bytes(MOESQ_WS_ROUTE, T, k, E, 0, 0, 0) bytes (may be 0).
 * Limits: E <= 512, T*k < 2^31.
 */
int moesq_route_permute(void *stream, const int32_t *topk_ids, int64_t T, int32_t k, int32_t E,
                        int32_t *counts, int32_t *offsets, int32_t *sorted_slot, int32_t *slot_pos,
                        void *workspace, size_t workspace_bytes, int32_t *dev_status);

/*
 * Routing into the fixed-capacity layout (paper Appendix D.1: activations and outputs batched with a
 * fixed per-expert capacity C, so expert e's operands sit at a fixed stride and no pointer arrays are
 * needed): slot f = t*k + j routed to expert e with stable rank r among e's slots (ascending f) gets
 * slot_pos[f] = e*C + r when r < C, else -1 (over capacity: not placed; combine skips it).
 *   counts    [E] all slots routed to each expert (may exceed C; the GEMMs use min(count, C))
 *   slot_pos  [T*k]; -1 also for ids outside [0, E), reported in *dev_status as moesq_route_permute
 *   workspace moesq_workspace_bytes(MOESQ_WS_ROUTE_CAPACITY, T, k, E, 0, 0, 0) bytes, 256-byte aligned
 * Limits: E <= 512, T*k < 2^31, E*C < 2^31.
 */
int moesq_route_capacity(void *stream, const int32_t *topk_ids, int64_t T, int32_t k, int32_t E, int32_t capacity,
                         int32_t *counts, int32_t *slot_pos, void *workspace, size_t workspace_bytes,
                         int32_t *dev_status);

/*
 * Dynamic NVFP4 activation quantization (paper Section 3.4 and Appendix D.1: activations are
 * quantized at run time into 32-element blocks; Eq. 3 + Eq. 5 with the given tensor scale), fused
 * with token dispatch (a scatter: every token row of x is read once and its codes are written to each
 * permuted row the token is routed to).
 *   x           [T][ld_x] fp32 or bf16 (x_dtype), K <= ld_x, K % 32 == 0
 *   slot_pos    [T*k] or NULL: permuted row of the j-th routed copy of token t at slot_pos[t*k + j]
 *               (moesq_route_permute's output; negative = dropped). rows >= T*k, k <= 512; permuted
 *               rows no slot points to are not written. NULL: rows must equal T and row p is x row p.
 *   gamma       [G] fp32 tensor scales. With offsets != NULL, row p uses gamma[e] where
 *               offsets[e] <= p < offsets[e+1] (G = E, the per-expert input scale of the model
 *               card); with offsets == NULL and E > 0 the rows are in the fixed-capacity layout
 *               (MOESQ_F_CAPACITY; rows % E == 0) and row p uses gamma[p / (rows / E)]; with
 *               offsets == NULL and E == 0 every row uses gamma[0].
 *   q           [rows][K/2] E2M1 codes, s [rows][K/32] UE4M3 codes.
 *   xk          optional (NULL to skip), 16-byte aligned: [rows][K] f16, the same values dequantized
 *               (e2m1 * e4m3, exact in f16) with every 8-group of K stored in the order
 *               (0, 2, 4, 6, 1, 3, 5, 7) -- the GEMM's operand order, read by moesq_grouped_gemm /
 *               moesq_expert_mlp instead of decoding q and s once per weight-row block.
 * Per 32-block b of a row: amax = max |x|; code = E4M3(fp32(fp32(gamma*amax)/6)) rounded to
 * nearest even, saturating at 448; s = E4M3value/gamma; q = E2M1(x/s) (nearest, ties to the even
 * code, +0 for zero); q = 0 when s == 0. All in IEEE fp32 without fused multiply-add.
 */
int moesq_quantize_act(void *stream, const void *x, int32_t x_dtype, int64_t T, int32_t K, int64_t ld_x,
                       const int32_t *slot_pos, int32_t k, int64_t rows, const float *gamma,
                       const int32_t *offsets, int32_t E, uint8_t *q, uint8_t *s, void *xk);

/*
 * Dispatch in one call (paper Appendix D.1: routing metadata and the quantized activations are
 * produced on the device before the grouped GEMM): moesq_route_permute followed by
 * moesq_quantize_act(x, slot_pos, k, rows = T*k, gamma, offsets, E). Every output (counts, offsets,
 * sorted_slot, slot_pos, q, s, xk, *dev_status) is byte-identical to that pair of calls. For
 * decode-sized batches (T*k <= 2048, k <= 32) it is a single kernel launch in which each token's
 * workgroup ranks all T*k ids itself; otherwise it enqueues the two steps.
 *   topk_ids [T][k] int32 (device); E <= 512; gamma [E] per-expert tensor scales (device).
 *   x, x_dtype, K, ld_x, q [T*k][K/2], s [T*k][K/32], xk: as moesq_quantize_act.
 *   counts, offsets, sorted_slot, slot_pos, workspace, dev_status: as moesq_route_permute
 *   (workspace = moesq_workspace_bytes(MOESQ_WS_ROUTE, T, k, E, 0, 0, 0) bytes; unused, and may be
 *   NULL, on the single-launch path).
 * Errors: the union of the two calls' argument checks, returned before anything is enqueued.
 */
int moesq_route_quantize(void *stream, const int32_t *topk_ids, int64_t T, int32_t k, int32_t E,
                         const void *x, int32_t x_dtype, int32_t K, int64_t ld_x, const float *gamma,
                         int32_t *counts, int32_t *offsets, int32_t *sorted_slot, int32_t *slot_pos,
                         void *workspace, size_t workspace_bytes, uint8_t *q, uint8_t *s, void *xk,
                         int32_t *dev_status);

/*
 * Dispatch with a dynamic activation tensor scale (paper Section 3.4 / Eq. 5 applied to the step's own
 * tokens, the on-device counterpart of a calibrated per-expert constant): gamma = Eq. 5 over the
 * amax of all T x K values of x, computed on the device and written to gamma_out[0 .. E) (every
 * expert gets the same value; pass gamma_out as gamma_a to the grouped GEMM), then exactly
 * moesq_route_quantize(..., gamma = gamma_out, ...). Outputs are byte-identical to
 * moesq_global_scale(x) copied to E entries followed by moesq_route_quantize. On the single-launch
 * path of moesq_route_quantize, when the tokens take at most 256 KiB (T*K*sizeof(x)), each
 * workgroup also computes the amax itself, so the call stays one launch; otherwise an amax pre-pass
 * (three small launches) runs first.
 *   gamma_out [E] fp32 (device, 4-byte aligned); other arguments as moesq_route_quantize.
 * Errors: as moesq_route_quantize (gamma_out NULL: MOESQ_ERR_INVALID_ARG).
 */
int moesq_route_quantize_dyn(void *stream, const int32_t *topk_ids, int64_t T, int32_t k, int32_t E,
                             const void *x, int32_t x_dtype, int32_t K, int64_t ld_x, float *gamma_out,
                             int32_t *counts, int32_t *offsets, int32_t *sorted_slot, int32_t *slot_pos,
                             void *workspace, size_t workspace_bytes, uint8_t *q, uint8_t *s, void *xk,
                             int32_t *dev_status);

/*
 * Dispatch and grouped GEMM in one call (paper Appendix D.1: routing metadata and the quantized
 * activations are produced on the device and consumed by the grouped GEMM of Section 2 / 3.4):
 * moesq_route_quantize(topk_ids, T, k, E, x, ..., gamma = gamma_a, ...) followed by
 * moesq_grouped_gemm(W, q, s, xk, gamma_a, offsets, rows = T*k, y, y_dtype, flags = 0). Every output
 * (counts, offsets, sorted_slot, slot_pos, q, s, xk, y, *dev_status) is byte-identical to that pair of
 * calls. For the smallest decode batches (2 T*k <= E, K <= 2048) it is one kernel launch: each
 * weight-streaming workgroup ranks the ids of its expert and quantizes that expert's tokens itself, so
 * no dispatch kernel runs before the GEMM; otherwise it enqueues the two calls (pass xk for the faster
 * weight-streaming GEMM there).
 *   W->E == E, W->K == K; other arguments as in the two calls (workspace: as moesq_route_quantize).
 * Errors: the union of the two calls' argument checks, returned before anything is enqueued.
 */
int moesq_route_quantize_gemm(void *stream, const int32_t *topk_ids, int64_t T, int32_t k, int32_t E,
                              const void *x, int32_t x_dtype, int32_t K, int64_t ld_x, const float *gamma_a,
                              const moesq_weights *W, int32_t *counts, int32_t *offsets, int32_t *sorted_slot,
                              int32_t *slot_pos, void *workspace, size_t workspace_bytes, uint8_t *q, uint8_t *s,
                              void *xk, void *y, int32_t y_dtype, int32_t *dev_status);

/*
 * Grouped sparse GEMM (paper Section 2: Y_e = X_e W_e^T in one launch for variable per-expert token
 * counts; Section 3.4: sparse operand W on the left, Y_e^T = W_e X_e^T; block scales applied in the
 * product, alpha_e = 1/(gamma_w,e * gamma_a,e) applied to the fp32 accumulator).
 *   q, s        [rows][K/2], [rows][K/32] quantized activations in expert-sorted order
 *   xk          optional [rows][K] f16 copy from moesq_quantize_act (same rows); when given the tiled
 *               kernel stages it straight into LDS instead of decoding q and s
 *   gamma_a     [E] activation tensor scale of each expert
 *   offsets     [E+1] from moesq_route_permute (device)
 *   y           [rows][N] fp32 or bf16 (round to nearest even). Rows >= offsets[E] are not written.
 * Requires W->kl (MOESQ_ERR_INVALID_ARG if NULL), K % 256 == 0 and N % 64 == 0
 * (MOESQ_ERR_UNSUPPORTED otherwise); E <= 1024.
 */
int moesq_grouped_gemm(void *stream, const moesq_weights *W, const uint8_t *q, const uint8_t *s, const void *xk,
                       const float *gamma_a, const int32_t *offsets, int64_t rows, void *y, int32_t y_dtype,
                       uint32_t flags);

/*
 * Routed-expert MLP (paper Appendix D.1 serving integration: the two grouped GEMMs with SwiGLU and
 * requantization fused into the first GEMM's epilogue):
 *   gate_up:  W13 with N = 2I: rows [0, I) are the gate projection, rows [I, 2I) the up projection
 *   h = SiLU(alpha*g) * (alpha*u) in fp32, SiLU(v) = v / (1 + exp(-v))
 *   requant:  h quantized like moesq_quantize_act with gamma_h[e], 32-blocks along I
 *   down:     W2 with N = H, K = I, alpha = 1/(gamma_w2,e * gamma_h,e) -> y [rows][H]
 * xk is the optional f16 copy of (q, s) from moesq_quantize_act.
 * Workspace: moesq_workspace_bytes(MOESQ_WS_MLP, ..., rows, k=0, E, K=H, N=0, I) bytes; it holds, each
 *   region starting on a 256-byte boundary, h_q [rows][I/2], h_s [rows][I/32] and h_k [rows][I] (the
 *   f16 copy of the requantized h, which the weight-streaming down GEMM reads; the tiled down GEMM
 *   stages h from h_q/h_s, and the tiled kernels write h_k only with a dump flag). With MOESQ_F_DUMP_GATEUP and/or
 *   MOESQ_F_DUMP_H the size is moesq_workspace_bytes(MOESQ_WS_MLP_DUMP, ...) and two more regions
 *   follow: the fp32 gate_up outputs [rows][2I] (written with MOESQ_F_DUMP_GATEUP), then the fp32 h
 *   [rows][I] the requantization read (written with MOESQ_F_DUMP_H). Rows no expert owns are not
 *   written.
 * Calibration (MOESQ_F_CALIBRATE; model card: the input scale is stored per expert linear, Eq. 5 over
 *   the tensor's amax): only the gate_up GEMM and SwiGLU run; the call writes, at the start of the
 *   workspace, amax_h [E] (fp32, the largest |h| over each expert's rows, 0 for an expert without
 *   rows) and, at the next 256-byte boundary, gamma_h [E] = Eq. 5 of amax_h (1 where amax_h is 0).
 *   Workspace: moesq_workspace_bytes(MOESQ_WS_MLP_CALIBRATE, ..., E, ...) bytes. gamma_h is not read
 *   (may be NULL) and y is not written; the dump flags are invalid with it. The amax is a max, so the
 *   result does not depend on the kernel's order of work; it depends on the kernel family only
 *   through the fp32 accumulation order of h.
 * Kernels: with rows <= 16 E both GEMMs stream the weights (the gate_up epilogue computes SwiGLU and
 * the requantization per 32 intermediate columns), otherwise both are tiled; MOESQ_F_FORCE_DECODE /
 * MOESQ_F_FORCE_PREFILL pick one. Both produce the same results up to fp32 accumulation order.
 * Requires H % 256 == 0, I % 256 == 0.
 */
int moesq_expert_mlp(void *stream, const moesq_weights *W13, const moesq_weights *W2, const uint8_t *q,
                     const uint8_t *s, const void *xk, const float *gamma_a, const float *gamma_h,
                     const int32_t *offsets, int64_t rows, void *y, int32_t y_dtype, void *workspace,
                     size_t workspace_bytes, uint32_t flags);

/*
 * moesq_expert_mlp for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same call, arguments and results, without the
 * workspace argument. Its workspace is a static device array of MOESQ_NOALLOC_SCRATCH_BYTES inside the
 * library, one per GPU, held until the process ends; its device address is looked up on the first call
 * on each device (make that first call outside graph capture). The call itself allocates nothing.
 *   Limit: the call's workspace, moesq_workspace_bytes(MOESQ_WS_MLP, rows, 0, E, H, 0, I), must fit in
 *   MOESQ_NOALLOC_SCRATCH_BYTES, else MOESQ_ERR_WORKSPACE and nothing is launched (I = 2048: up to
 *   6472 rows; the decode-sized batches this is for take a few hundred).
 *   Every call on one GPU uses that GPU's one array: calls that may overlap on one GPU (different
 *   streams without ordering) race and must not be issued; calls ordered on one stream are safe. The
 *   array keeps the last call's contents; nothing in it needs to start at zero.
 * Errors: as moesq_expert_mlp; MOESQ_ERR_INVALID_ARG with MOESQ_F_DUMP_GATEUP, MOESQ_F_DUMP_H or
 * MOESQ_F_CALIBRATE (their results would stay in the array); MOESQ_ERR_HIP if the array's device
 * address cannot be obtained.
 */
#define MOESQ_NOALLOC_SCRATCH_BYTES (32u << 20)
int moesq_expert_mlp_noalloc(void *stream, const moesq_weights *W13, const moesq_weights *W2, const uint8_t *q,
                             const uint8_t *s, const void *xk, const float *gamma_a, const float *gamma_h,
                             const int32_t *offsets, int64_t rows, void *y, int32_t y_dtype, uint32_t flags);

/*
 * Router-weighted unpermute + combine (paper Appendix D.1, token combination):
 *   out[t][c] = sum over j = 0..k-1 (in that order, fp32) of topk_w[t][j] * y_sorted[slot_pos[t*k+j]][c]
 * Slots with slot_pos = -1 contribute nothing. out is fp32 or bf16 (round to nearest even).
 *   y_sorted [T*k][H] (y_dtype), slot_pos [T*k], topk_w [T][k] fp32, out [T][H]. Requires H % 8 == 0.
 */
int moesq_unpermute_combine(void *stream, const void *y_sorted, int32_t y_dtype, const int32_t *slot_pos,
                            const float *topk_w, int64_t T, int32_t k, int32_t H, void *out, int32_t out_dtype);

/* ---- setup and parity calls (not on the timed path) ----------------------------------------------
 *
 * Weight compression (setup; paper Section 3.4 last paragraph, Appendix A): per 8-group keep the
 * two adjacent pairs with the largest L2 norm (norms in fp64, ties to the lower pair), compute
 * gamma_w,e from the pruned expert tensor (Eq. 5), quantize 32-blocks along K like
 * moesq_quantize_act, and store the dense NVFP4 bytes as pair-bitmask v1 (a chunk with fewer than
 * two nonzero bytes marks its lowest-index zero bytes as kept).
 *   w [E][N][K] fp32; outputs as in moesq_weights (gscale is writable here).
 * Workspace: moesq_workspace_bytes(MOESQ_WS_COMPRESS, 0, 0, E, 0, 0, 0) bytes.
 * dev_status (optional, caller zero-initializes) receives MOESQ_ERR_PATTERN if a chunk has more
 * than two nonzero bytes (cannot happen after pruning; reported, not silently packed).
 */
int moesq_compress_weights(void *stream, const float *w, int32_t E, int32_t N, int32_t K, uint8_t *packed,
                           uint8_t *mask, uint8_t *scale, float *gscale, void *workspace,
                           size_t workspace_bytes, int32_t *dev_status);

/*
 * Tensor scale of Eq. 5 for a device tensor x [rows][ld_x] (fp32 or bf16, first K columns):
 * gamma_out[0] = 448 / (amax / 6) in fp32 (1 for an all-zero tensor). Calibration of the static
 * per-expert activation scale (model card: stored per expert linear), and the pre-pass of
 * moesq_route_quantize_dyn for batches past its single launch. gamma_out is used as scratch while the
 * call runs.
 */
int moesq_global_scale(void *stream, const void *x, int32_t x_dtype, int64_t rows, int32_t K, int64_t ld_x,
                       float *gamma_out);

/*
 * Load-time repack (model card: the sparse checkpoint is rebuilt into the kernel's own layout at
 * load time) of pair-bitmask v1 weights into the GEMM's fragment layout, same size (2.75 bits per
 * weight): per expert, per 64-row group, per 256-K super-step a 5632-byte unit holding four 16-row
 * fragments j = 0..3. Lane l = 16c + r (row r of a fragment, K [64c, +64) of the super-step) owns
 * bytes [1024 j + 16 l, +16) (its eight 8-groups of fragment j, the two kept bytes (b0, b1) of each
 * stored as (lo b0 | lo b1 << 4, hi b0 | hi b1 << 4)), [4096 + 16 l + 4 j, +4) (per group the code
 * i | j << 2 of its kept pairs i < j, one nibble each, groups in the order 0, 2, 4, 6, 1, 3, 5, 7)
 * and [5120 + 8 l + 2 j, +2) (its two scale codes). A wave reads the four fragments of a unit with
 * six loads.
 *   kl: moesq_kernel_layout_bytes(E, N, K) bytes, 16-byte aligned. Requires K % 256 == 0, N % 64 == 0.
 */
int moesq_prepack_weights(void *stream, const moesq_weights *W, uint8_t *kl, size_t kl_bytes);

/*
 * Dense NVFP4 control (paper Appendix D.2 compares the sparse kernel with a dense NVFP4 grouped GEMM):
 * the same kernels on unpruned weights, so that the two differ only in sparsity. Dense weights of
 * expert e: codes [E][N][K/2] (two E2M1 codes per byte, lower K in the low nibble), UE4M3 block
 * scales [E][N][K/32], tensor scale gscale [E] (Eq. 5); moesq_quantize_act with gamma = gscale[e]
 * produces codes and scales from fp32 rows.
 * moesq_prepack_dense_weights builds the dense kernel layout (moesq_dense_layout_bytes(E, N, K) =
 * E * N * K * 9 / 16 bytes, 4.5 bits per weight: per 64-row group and 256-K super-step a 9216-byte
 * unit; lane l of fragment j owns 32 code bytes at 2048 j + 32 l and 4 scale bytes at 8192 + 16 l + 4 j,
 * the scale bytes stored once per lane pair that reads them). Requires K % 256 == 0, N % 64 == 0.
 * moesq_dense_grouped_gemm: as moesq_grouped_gemm with W->kl = the dense layout and W->gscale
 * (W->packed, W->mask, W->scale are not read).
 */
size_t moesq_dense_layout_bytes(int32_t E, int32_t N, int32_t K);
int moesq_prepack_dense_weights(void *stream, int32_t E, int32_t N, int32_t K, const uint8_t *codes,
                                const uint8_t *scales, uint8_t *kl, size_t kl_bytes);
int moesq_dense_grouped_gemm(void *stream, const moesq_weights *W, const uint8_t *q, const uint8_t *s, const void *xk,
                             const float *gamma_a, const int32_t *offsets, int64_t rows, void *y, int32_t y_dtype,
                             uint32_t flags);

/* Bytes of the kernel layout of E experts of [N][K] weights: E * N * K * 11 / 32. */
size_t moesq_kernel_layout_bytes(int32_t E, int32_t N, int32_t K);

/*
 * Pair-bitmask v1 -> dense NVFP4 bytes [E][N][K/2] (the lossless round trip of the model card).
 * dev_status (optional) receives MOESQ_ERR_PATTERN for a mask nibble whose popcount is not 2.
 */
int moesq_unpack_weights(void *stream, const moesq_weights *W, uint8_t *dense_nvfp4, int32_t *dev_status);

/*
 * Workspace size in bytes for a call kind (MOESQ_WS_*). Arguments not used by a kind are ignored:
 *   ROUTE: T, k, E.   MLP / MLP_DUMP: T = rows, E, K = H, I.   MLP_CALIBRATE: E.   COMPRESS: E.
 */
size_t moesq_workspace_bytes(int32_t kind, int64_t T, int32_t k, int32_t E, int32_t K, int32_t N, int32_t I);

/* Human-readable text for a status code (static storage). */
const char *moesq_status_str(int32_t status);

/* Library version as major*10000 + minor*100 + patch. */
int32_t moesq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOESQ_H */
