// Routing / dispatch planning: per-expert histogram of the top-k ids, exclusive prefix scan,
// stable scatter of the flat slots into expert-sorted order (paper Appendix D.1: token counts
// stay on the device and drive the persistent GEMM schedule).
//
// Deterministic and atomics-free in its results: LDS atomics only count (order independent); the
// position of every slot is its expert's offset plus the number of earlier slots with the same
// expert, computed with wave ballots and per-wave prefix tables.
#include "common.h"
#include "launch.h"

namespace moesq {

constexpr int kRouteThreads = 256;   // multi-block path: 4 waves per block
constexpr int kRouteChunk = 1024;    // slots per block in the multi-block path
constexpr int kSmallThreads = 256;   // single-workgroup path: 4 waves

// Rank of this lane among the lanes of its wave holding the same key (lower lanes first), and the
// number of such lanes. Lanes with valid == false take no part. The set of lanes with the same key is
// the AND over the key's bits of the ballot of lanes that agree on that bit (keys < 2^bits).
MOESQ_DEV void wave_match_rank(int key, bool valid, int bits, int& rank, int& count) {
  const int lane = threadIdx.x & 63;
  uint64_t same = __ballot(valid);
  for (int b = 0; b < bits; b++) {
    const uint64_t ones = __ballot(valid && ((key >> b) & 1));
    same &= ((key >> b) & 1) ? ones : ~ones;
  }
  rank = __builtin_popcountll(same & ((1ull << lane) - 1ull));
  count = __builtin_popcountll(same);
}

MOESQ_DEV int key_bits(int E) { return 32 - __builtin_clz((unsigned)(E > 1 ? E - 1 : 1)); }

// Scatter one round of up to THREADS consecutive slots starting at `base_slot`, given the running
// per-expert positions pos_base[e] (LDS). Waves are ordered: wave w's slots come after waves
// 0..w-1 of the same round. wave_tab is LDS [THREADS/64][E].
template <int THREADS>
MOESQ_DEV void scatter_round(const int32_t* __restrict__ ids, int64_t n, int64_t base_slot, int32_t E,
                             int32_t* pos_base, int32_t* wave_tab, int32_t* __restrict__ sorted_slot,
                             int32_t* __restrict__ slot_pos, int32_t* dev_status, int e_pre = -2) {
  constexpr int WAVES = THREADS / 64;
  const int tid = threadIdx.x, w = tid >> 6;
  const int64_t f = base_slot + tid;
  int e = -1;
  if (f < n) e = e_pre != -2 ? e_pre : ids[f];
  const bool valid = (f < n) && e >= 0 && e < E;
  if (f < n && !valid) {
    slot_pos[f] = -1;
    if (dev_status) *dev_status = MOESQ_ERR_INVALID_ARG;
  }
  for (int i = tid; i < WAVES * E; i += THREADS) wave_tab[i] = 0;
  __syncthreads();
  int rank, count;
  wave_match_rank(e, valid, key_bits(E), rank, count);
  if (valid && rank == count - 1) wave_tab[w * E + e] = count;  // one writer per (wave, expert)
  __syncthreads();
  // exclusive prefix over waves per expert, then advance pos_base
  for (int x = tid; x < E; x += THREADS) {
    int run = pos_base[x];
#pragma unroll
    for (int v = 0; v < WAVES; v++) {
      const int c = wave_tab[v * E + x];
      wave_tab[v * E + x] = run;
      run += c;
    }
    pos_base[x] = run;
  }
  __syncthreads();
  if (valid) {
    const int p = wave_tab[w * E + e] + rank;
    sorted_slot[p] = (int32_t)f;
    slot_pos[f] = p;
  }
}


// Single-workgroup path (4 waves): histogram, scan and all scatter rounds in one launch.
__global__ __launch_bounds__(kSmallThreads) void route_single_kernel(const int32_t* __restrict__ ids, int64_t n,
                                                                     int32_t E, int32_t* __restrict__ counts,
                                                                     int32_t* __restrict__ offsets,
                                                                     int32_t* __restrict__ sorted_slot,
                                                                     int32_t* __restrict__ slot_pos,
                                                                     int32_t* dev_status) {
  extern __shared__ int32_t lds[];
  int32_t* hist = lds;                        // [E]
  int32_t* pos = hist + E;                    // [E+1]
  int32_t* wave_tab = pos + E + 1;            // [4 * E]
  __shared__ int32_t wsum[kSmallThreads / 64];
  constexpr int R = kRouteSingleMax / kSmallThreads;  // slots per thread, kept in registers
  const int tid = threadIdx.x;
  int ev[R];
#pragma unroll
  for (int r = 0; r < R; r++) {
    const int64_t f = tid + (int64_t)r * kSmallThreads;
    ev[r] = f < n ? ids[f] : -1;
  }
  for (int i = tid; i < E; i += kSmallThreads) hist[i] = 0;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; r++)
    if (ev[r] >= 0 && ev[r] < E) atomicAdd(&hist[ev[r]], 1);
  __syncthreads();
  block_exclusive_scan<kSmallThreads>(hist, E, pos, wsum);
  for (int i = tid; i <= E; i += kSmallThreads) {
    offsets[i] = pos[i];
    if (i < E) counts[i] = hist[i];
  }
#pragma unroll
  for (int r = 0; r < R; r++) {
    if ((int64_t)r * kSmallThreads >= n) break;
    scatter_round<kSmallThreads>(ids, n, (int64_t)r * kSmallThreads, E, pos, wave_tab, sorted_slot, slot_pos,
                                 dev_status, ev[r]);
    __syncthreads();
  }
}

// Multi-block path, step 1: per-chunk histograms, stored expert-major: hist[e][chunk].
__global__ __launch_bounds__(kRouteThreads) void route_hist_kernel(const int32_t* __restrict__ ids, int64_t n,
                                                                   int32_t E, int32_t nchunks,
                                                                   int32_t* __restrict__ hist_g) {
  extern __shared__ int32_t lds[];
  const int tid = threadIdx.x;
  for (int i = tid; i < E; i += kRouteThreads) lds[i] = 0;
  __syncthreads();
  const int64_t lo = (int64_t)blockIdx.x * kRouteChunk;
  const int64_t hi = min(n, lo + kRouteChunk);
  for (int64_t f = lo + tid; f < hi; f += kRouteThreads) {
    const int e = ids[f];
    if (e >= 0 && e < E) atomicAdd(&lds[e], 1);
  }
  __syncthreads();
  for (int i = tid; i < E; i += kRouteThreads) hist_g[(int64_t)i * nchunks + blockIdx.x] = lds[i];
}

// Step 2 (one wave per expert): exclusive prefix of the expert's chunk counts in place,
// hist[e][c] = sum of hist[e][c'] for c' < c, and its total -> tot[e], counts[e]. Lane l holds a
// contiguous run of chunks.
__global__ __launch_bounds__(kRouteThreads) void route_chunk_scan_kernel(int32_t* __restrict__ hist_g, int32_t nchunks,
                                                                        int32_t E, int32_t* __restrict__ tot,
                                                                        int32_t* __restrict__ counts) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * (kRouteThreads / 64) + (threadIdx.x >> 6);
  if (e >= E) return;
  int32_t* h = hist_g + (int64_t)e * nchunks;
  const int per = (nchunks + 63) / 64;
  const int c0 = min(nchunks, lane * per), c1 = min(nchunks, c0 + per);
  int sum = 0;
  for (int c = c0; c < c1; c++) sum += h[c];
  int incl = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  int run = incl - sum;
  for (int c = c0; c < c1; c++) {
    const int v = h[c];
    h[c] = run;
    run += v;
  }
  if (lane == 63) {
    tot[e] = incl;
    counts[e] = incl;
  }
}

// Step 3: stable scatter of each chunk. Every block scans the expert totals itself (offsets; block 0
// also stores them), adds the chunk's prefix, then scatters its slots.
__global__ __launch_bounds__(kRouteThreads) void route_scatter_kernel(const int32_t* __restrict__ ids, int64_t n,
                                                                      int32_t E, int32_t nchunks,
                                                                      const int32_t* __restrict__ base_g,
                                                                      const int32_t* __restrict__ tot_g,
                                                                      int32_t* __restrict__ offsets,
                                                                      int32_t* __restrict__ sorted_slot,
                                                                      int32_t* __restrict__ slot_pos,
                                                                      int32_t* dev_status) {
  extern __shared__ int32_t lds[];
  int32_t* tot = lds;                // [E]
  int32_t* pos = tot + E;            // [E+1]
  int32_t* wave_tab = pos + E + 1;   // [4 * E]
  __shared__ int32_t wsum[kRouteThreads / 64];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kRouteThreads) tot[e] = tot_g[e];
  __syncthreads();
  block_exclusive_scan<kRouteThreads>(tot, E, pos, wsum);
  if (blockIdx.x == 0)
    for (int e = tid; e <= E; e += kRouteThreads) offsets[e] = pos[e];
  for (int e = tid; e < E; e += kRouteThreads) pos[e] += base_g[(int64_t)e * nchunks + blockIdx.x];
  __syncthreads();
  const int64_t lo = (int64_t)blockIdx.x * kRouteChunk;
  const int64_t hi = min(n, lo + kRouteChunk);
  for (int64_t b = lo; b < hi; b += kRouteThreads) {
    scatter_round<kRouteThreads>(ids, hi, b, E, pos, wave_tab, sorted_slot, slot_pos, dev_status);
    __syncthreads();
  }
}

static size_t route_single_lds(int32_t E) { return sizeof(int32_t) * ((size_t)E + (E + 1) + 4 * (size_t)E); }

size_t route_workspace_bytes(int64_t n, int32_t E) {
  if (n <= kRouteSingleMax) return 0;
  const int64_t chunks = (n + kRouteChunk - 1) / kRouteChunk;
  return sizeof(int32_t) * ((size_t)chunks * (size_t)E + (size_t)E);
}

int launch_route(hipStream_t st, const int32_t* ids, int64_t n, int32_t E, int32_t* counts, int32_t* offsets,
                 int32_t* sorted_slot, int32_t* slot_pos, void* ws, int32_t* dev_status) {
  if (route_workspace_bytes(n, E) == 0) {
    hipLaunchKernelGGL(route_single_kernel, dim3(1), dim3(kSmallThreads), route_single_lds(E), st, ids, n, E,
                       counts, offsets, sorted_slot, slot_pos, dev_status);
    return hipGetLastError() == hipSuccess ? MOESQ_OK : MOESQ_ERR_HIP;
  }
  const int32_t chunks = (int32_t)((n + kRouteChunk - 1) / kRouteChunk);
  int32_t* hist = (int32_t*)ws;                     // [E][chunks]
  int32_t* tot = hist + (size_t)chunks * E;         // [E]
  hipLaunchKernelGGL(route_hist_kernel, dim3(chunks), dim3(kRouteThreads), sizeof(int32_t) * E, st, ids, n, E, chunks,
                     hist);
  hipLaunchKernelGGL(route_chunk_scan_kernel, dim3((E + 3) / 4), dim3(kRouteThreads), 0, st, hist, chunks, E, tot,
                     counts);
  hipLaunchKernelGGL(route_scatter_kernel, dim3(chunks), dim3(kRouteThreads),
                     sizeof(int32_t) * ((size_t)E + (E + 1) + 4 * (size_t)E), st, ids, n, E, chunks, hist, tot, offsets,
                     sorted_slot, slot_pos, dev_status);
  return hipGetLastError() == hipSuccess ? MOESQ_OK : MOESQ_ERR_HIP;
}

}  // namespace moesq
