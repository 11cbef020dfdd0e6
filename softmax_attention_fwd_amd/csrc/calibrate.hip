// Sustained matrix-core rate probe for gfx950: two waves per SIMD, each keeping four
// independent v_mfma_f32_32x32x16_bf16 accumulation chains in flight with operands that
// rotate over eight register pairs. Zero operands show the rate at the full clock; random
// bf16 operands show how far the clock falls under the switching load of real data.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include "tile_calibrate.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kWgPerCu = 2;

// A value in [-1, 1) from a 32-bit integer (an integer hash: xor-shift and multiply rounds).
__device__ inline float hash_unit(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return (float)(x >> 8) * (2.0f / 16777216.0f) - 1.0f;
}

__global__ __launch_bounds__(kThreads) void mfma_calibrate_kernel(float* out, int iterations,
                                                                  int random_operands) {
  const uint32_t t = blockIdx.x * kThreads + threadIdx.x;
  bf16x8 a[8], b[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t s = t * 131u + j * 17u + i;
      a[j][i] = (__bf16)(random_operands ? hash_unit(s) : 0.f);
      b[j][i] = (__bf16)(random_operands ? hash_unit(s ^ 0x9e3779b9U) : 0.f);
    }
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x16{};
  for (int it = 0; it < iterations; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(k + j) & 7], b[(k + 3 * j) & 7], acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[t] = s;
}

int cu_count(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return TILE_CAL_ELAUNCH;
  if (hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || *cus < 1)
    return TILE_CAL_ELAUNCH;
  return TILE_CAL_OK;
}

}  // namespace

extern "C" {

size_t tile_mfma_calibrate_out_floats(void) {
  int cus = 0;
  if (cu_count(&cus) != TILE_CAL_OK) return 0;
  return (size_t)cus * kWgPerCu * kThreads;
}

int tile_mfma_calibrate(float* out, size_t out_floats, int iterations, int random_operands,
                        double* flops, void* stream) {
  if (!out || !flops || iterations < 1 || iterations > (1 << 24) ||
      (random_operands != 0 && random_operands != 1))
    return TILE_CAL_EINVAL;
  int cus = 0;
  if (cu_count(&cus) != TILE_CAL_OK) return TILE_CAL_ELAUNCH;
  const size_t need = (size_t)cus * kWgPerCu * kThreads;
  if (out_floats < need) return TILE_CAL_EINVAL;
  const int blocks = cus * kWgPerCu;
  hipLaunchKernelGGL(mfma_calibrate_kernel, dim3(blocks), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), out, iterations, random_operands);
  if (hipGetLastError() != hipSuccess) return TILE_CAL_ELAUNCH;
  *flops = 2.0 * 32 * 32 * 16 * 32.0 * iterations * (double)blocks * (kThreads / 64);
  return TILE_CAL_OK;
}

}  // extern "C"
