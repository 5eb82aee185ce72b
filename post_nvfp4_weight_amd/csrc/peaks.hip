// Micro-benchmarks of the device's own peaks: the matrix cores' issue rate
// (bf16 and fp32 MFMA), the vector ALUs' fp32 FMA rate, and HBM streaming
// bandwidth.  The benchmark reports the quantizer's kernels against these
// beside the nominal figures.  Nothing here is part of the quantization path:
// this file builds a library of its own (libnvq_peaks.so) that only the
// benchmark loads.
//
// Every kernel runs 256-thread workgroups; the host passes the grid.  The
// arithmetic loops keep NACC independent accumulator chains per wave on
// register operands, and store one value per lane at the end so that nothing
// is dead.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int NACC = 4;

// NACC x iters v_mfma_f32_32x32x16_bf16 per wave (32768 flops each).
__global__ __launch_bounds__(256) void mfma_bf16_kernel(int iters, float* __restrict__ out) {
  const float t = (float)threadIdx.x;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(t * 0.001f + (float)e);
    b[e] = (__bf16)(1.0f - t * 0.002f * (float)e);
  }
  f32x16 acc[NACC];
#pragma unroll
  for (int j = 0; j < NACC; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;
#pragma unroll 4
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int j = 0; j < NACC; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < NACC; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// NACC x iters v_mfma_f32_32x32x2f32 per wave (4096 flops each).
__global__ __launch_bounds__(256) void mfma_f32_kernel(int iters, float* __restrict__ out) {
  const float a = (float)threadIdx.x * 0.001f, b = 1.0f - (float)threadIdx.x * 0.0005f;
  f32x16 acc[NACC];
#pragma unroll
  for (int j = 0; j < NACC; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;
#pragma unroll 4
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int j = 0; j < NACC; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[j], 0, 0, 0);
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < NACC; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// 16 x iters scalar fp32 FMAs per lane (2 flops each), 16 independent chains.
__global__ __launch_bounds__(256) void fma_f32_kernel(int iters, float m, float c, float* __restrict__ out) {
  float x[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) x[j] = (float)(threadIdx.x + j);
#pragma unroll 4
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = fmaf(x[j], m, c);
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += x[j];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// dst[i] = src[i] over n 16-byte vectors, grid-stride, U vectors per thread
// in flight (all U loads issued before the stores); n is a multiple of
// U * 256 * gridDim.x or the tail runs one vector at a time.
template <int U>
__global__ __launch_bounds__(256) void copy_kernel(const f32x4* __restrict__ src, f32x4* __restrict__ dst,
                                                   int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + (U - 1) * stride < n; i += U * stride) {
    f32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

}  // namespace

// kind 0: bf16 MFMA, 1: fp32 MFMA, 2: fp32 FMA (m = 0.999, c = 0.001).
// out holds grid * 256 floats.  Returns a hipError_t code.
extern "C" int nvq_peak_compute(int kind, int grid, int iters, float* out, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (grid <= 0 || iters <= 0 || !out) return (int)hipErrorInvalidValue;
  if (kind == 0)
    hipLaunchKernelGGL(mfma_bf16_kernel, dim3(grid), dim3(256), 0, s, iters, out);
  else if (kind == 1)
    hipLaunchKernelGGL(mfma_f32_kernel, dim3(grid), dim3(256), 0, s, iters, out);
  else if (kind == 2)
    hipLaunchKernelGGL(fma_f32_kernel, dim3(grid), dim3(256), 0, s, iters, 0.999f, 0.001f, out);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

// Copies bytes (a multiple of 16; both pointers 16-byte aligned) from src to
// dst with `grid` workgroups and `unroll` (1, 4 or 8) vectors per thread in
// flight.  Returns a hipError_t code.
extern "C" int nvq_peak_copy(const void* src, void* dst, int64_t bytes, int grid, int unroll, void* stream) {
  if (bytes <= 0 || bytes % 16 || grid <= 0 || (uintptr_t)src % 16 || (uintptr_t)dst % 16)
    return (int)hipErrorInvalidValue;
  hipStream_t s = (hipStream_t)stream;
  const f32x4* a = (const f32x4*)src;
  f32x4* b = (f32x4*)dst;
  if (unroll == 1)
    hipLaunchKernelGGL(copy_kernel<1>, dim3(grid), dim3(256), 0, s, a, b, bytes / 16);
  else if (unroll == 4)
    hipLaunchKernelGGL(copy_kernel<4>, dim3(grid), dim3(256), 0, s, a, b, bytes / 16);
  else if (unroll == 8)
    hipLaunchKernelGGL(copy_kernel<8>, dim3(grid), dim3(256), 0, s, a, b, bytes / 16);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}
