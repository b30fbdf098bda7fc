// Seeded synthetic inputs drawn on the device: the same numbers as gen.cpp
// (bit-identical, same header), so large weight tensors need no host round trip.
#include <hip/hip_runtime.h>
#include "gen_math.h"

__global__ void gen_normal_kernel(uint64_t key, uint64_t start, int64_t n, double scale, float* out) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) out[i] = (float)(scale * gen_normal(key, start + (uint64_t)i));
}

__global__ void gen_student_t_kernel(uint64_t key, uint64_t start, int64_t n, int nu, double scale, float* out) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) out[i] = (float)(scale * gen_student_t(key, start + (uint64_t)i, nu));
}

static int grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (int)g;
}

extern "C" {

// Same contract as gen_fill_normal, writing a device buffer on the given stream.
int gen_gpu_fill_normal(void* stream, uint64_t seed, uint64_t strm, uint64_t start, int64_t n, double scale,
                        float* out) {
  if (n <= 0) return 0;
  if (out == nullptr) return -1;
  hipLaunchKernelGGL(gen_normal_kernel, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream,
                     gen_key(seed, strm), start, n, scale, out);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

int gen_gpu_fill_student_t(void* stream, uint64_t seed, uint64_t strm, uint64_t start, int64_t n, int32_t nu,
                           double scale, float* out) {
  if (n <= 0) return 0;
  if (out == nullptr || nu < 1) return -1;
  hipLaunchKernelGGL(gen_student_t_kernel, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream,
                     gen_key(seed, strm), start, n, (int)nu, scale, out);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
