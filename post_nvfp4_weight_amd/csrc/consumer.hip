// NVFP4 weight-only GEMM, the consumer of the exported weights:
//   Y = X dequant(W)^T, X bf16 [T x k] activations, W NVFP4 [m x k].
//
// An element without the per-tensor scale, e2m1 * e4m3, has at most 6
// significant bits and is exact in bf16.  So the kernel expands codes and
// block scales to bf16 as it stages a weight tile into LDS, multiplies on the
// bf16 matrix cores (v_mfma_f32_32x32x16_bf16, exact products, fp32
// accumulation) and applies g once to the result: Y = g (X Q^T) with
// Q = e2m1 * e4m3.  Against X fl32(Q g)^T this differs by at most 2^-24 of
// each product.
//
// Tiles are 128 (tokens) x 128 (output channels), four waves of 64 x 64, k in
// steps of 64 (four NVFP4 blocks); both operands are kept [row][k] in LDS
// (k contiguous, rows padded to 72 elements) and double-buffered; the next
// step's loads are in flight while the current step is multiplied.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace nvq {

namespace {

constexpr int CT = 128, CK = 64, CLD = CK + 8;
constexpr int CBUF = 2 * CT * CLD;   // bf16 elements of one buffer: X tile, then Q tile

typedef float f32x2c __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2c __attribute__((ext_vector_type(2)));

// Two codes (low nibble first) under block scale value s -> packed bf16 pair of e2m1 * s.
__device__ __forceinline__ uint32_t dq_pair(uint32_t c2, float hs) {
  const uint32_t c0 = c2 & 0xF, c1 = (c2 >> 4) & 0xF;
  const float m0 = e2m1_twice_mag((int)(c0 & 7)) * hs, m1 = e2m1_twice_mag((int)(c1 & 7)) * hs;
  const uint32_t p = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2c{m0, m1}, bf16x2c));
  return p | ((c0 & 8) << 12) | ((c1 & 8) << 28);   // sign bits of the two bf16 halves
}

// OUT: 0 fp32 Y, 1 bf16 Y, 2 fp32 partial sums of k-split blockIdx.z (no g)
// at P + z * T * m.  ksplit: k per split (a multiple of CK).
template <int OUT>
__global__ __launch_bounds__(256) void nvfp4_gemm_kernel(const uint16_t* __restrict__ X, int64_t T, int64_t k,
                                                         int64_t ldx, const uint8_t* __restrict__ codes,
                                                         const uint8_t* __restrict__ scales,
                                                         const float* __restrict__ gptr, int64_t m,
                                                         void* __restrict__ Y, int64_t ldy, int64_t ksplit) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * CBUF];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int64_t t0 = (int64_t)blockIdx.y * CT, o0 = (int64_t)blockIdx.x * CT;
  const int64_t kb = k / 16;   // blocks per weight row

  // Per step: X 128 rows x 64 k = 4 x 16 B per thread; W 128 rows x 4 blocks
  // = 2 blocks (8 B of codes + 2 scale bytes) per thread.
  const int wrow = tid >> 1, wh = tid & 1;
  auto load = [&](int64_t k0, u32x4 (&xv)[4], u32x2 (&cv)[2], uint32_t (&sv)[2]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = q * 256 + tid, r = e >> 3, c8 = (e & 7) * 8;
      xv[q] = *(const u32x4*)(X + min(t0 + r, T - 1) * ldx + min(k0 + c8, k - 8));
    }
    const int64_t row = min(o0 + wrow, m - 1);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t blk = min(k0 / 16 + 2 * wh + b, kb - 1);
      cv[b] = *(const u32x2*)(codes + row * (k / 2) + blk * 8);
      sv[b] = scales[row * kb + blk];
    }
  };
  auto store = [&](uint16_t* buf, int64_t k0, const u32x4 (&xv)[4], const u32x2 (&cv)[2], const uint32_t (&sv)[2]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = q * 256 + tid, r = e >> 3, c8 = (e & 7) * 8;
      const bool ok = t0 + r < T && k0 + c8 < k;
      *(u32x4*)(buf + r * CLD + c8) = ok ? xv[q] : u32x4{0u, 0u, 0u, 0u};
    }
    uint16_t* qb = buf + CT * CLD;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const bool ok = o0 + wrow < m && k0 + 32 * wh + 16 * b < k;
      const float hs = 0.5f * e4m3_value((int)(sv[b] & 0x7F));
      u32x4 lo, hi;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        lo[j] = ok ? dq_pair((cv[b][0] >> (8 * j)) & 0xFF, hs) : 0u;
        hi[j] = ok ? dq_pair((cv[b][1] >> (8 * j)) & 0xFF, hs) : 0u;
      }
      *(u32x4*)(qb + wrow * CLD + 32 * wh + 16 * b) = lo;
      *(u32x4*)(qb + wrow * CLD + 32 * wh + 16 * b + 8) = hi;
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int64_t kbeg = (int64_t)blockIdx.z * ksplit, kend = min(k, kbeg + ksplit);
  const int64_t nsteps = (kend - kbeg + CK - 1) / CK;
  u32x4 xv[4];
  u32x2 cv[2];
  uint32_t sv[2];
  load(kbeg, xv, cv, sv);
  store(smem, kbeg, xv, cv, sv);
  __syncthreads();
  const int arow = wr * 64 + (lane & 31), brow = wc * 64 + (lane & 31), koff = 8 * (lane >> 5);
  for (int64_t st = 0; st < nsteps; ++st) {
    const int cur = (int)(st & 1);
    if (st + 1 < nsteps) load(kbeg + (st + 1) * CK, xv, cv, sv);
    const uint16_t* Xs = smem + cur * CBUF;
    const uint16_t* Qs = Xs + CT * CLD;
#pragma unroll
    for (int ks = 0; ks < CK; ks += 16) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        a[t] = *(const bf16x8*)(Xs + (arow + 32 * t) * CLD + ks + koff);
        b[t] = *(const bf16x8*)(Qs + (brow + 32 * t) * CLD + ks + koff);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (st + 1 < nsteps) store(smem + (cur ^ 1) * CBUF, kbeg + (st + 1) * CK, xv, cv, sv);
    __syncthreads();
  }

  // Accumulator layout: lane l, register r -> row 8 (r/4) + 4 (l/32) + r%4, column l%32.
  const float g = OUT == 2 ? 1.0f : *gptr;
  float* P = (float*)Y + (OUT == 2 ? (int64_t)blockIdx.z * T * m : 0);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = t0 + wr * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t col = o0 + wc * 64 + j * 32 + (lane & 31);
        if (row < T && col < m) {
          const float v = acc[i][j][r] * g;
          if (OUT == 1) ((__bf16*)Y)[row * ldy + col] = (__bf16)v;
          else if (OUT == 0) ((float*)Y)[row * ldy + col] = v;
          else P[row * m + col] = v;
        }
      }
}

// Y = g * (sum of the splits in split order).
template <bool OUT_BF16>
__global__ void nvfp4_gemm_reduce_kernel(const float* __restrict__ P, int nsplit, int64_t T, int64_t m,
                                         const float* __restrict__ gptr, void* __restrict__ Y, int64_t ldy) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= T * m) return;
  float s = 0.0f;
  for (int z = 0; z < nsplit; ++z) s += P[(int64_t)z * T * m + e];
  const float v = s * *gptr;
  const int64_t row = e / m, col = e % m;
  if (OUT_BF16) ((__bf16*)Y)[row * ldy + col] = (__bf16)v;
  else ((float*)Y)[row * ldy + col] = v;
}

int num_cus_consumer() {
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
  }
  return cus;
}

// k splits so that the launch has about two workgroups per CU (at most 16,
// and each split at least one k step).
int nvfp4_gemm_splits(int64_t T, int64_t k, int64_t m) {
  const int64_t tiles = ((m + CT - 1) / CT) * ((T + CT - 1) / CT);
  const int64_t steps = (k + CK - 1) / CK;
  int64_t sp = (2 * num_cus_consumer() + tiles - 1) / tiles;
  sp = std::min<int64_t>(std::min<int64_t>(sp, 16), steps);
  return (int)std::max<int64_t>(sp, 1);
}

}  // namespace

size_t nvfp4_gemm_workspace(int64_t T, int64_t k, int64_t m) {
  if (T <= 0 || m <= 0 || k <= 0) return 0;
  const int sp = nvfp4_gemm_splits(T, k, m);
  return sp > 1 ? (size_t)sp * T * m * sizeof(float) : 0;
}

hipError_t nvfp4_gemm_launch(const uint16_t* X, int64_t T, int64_t k, int64_t ldx, const uint8_t* codes,
                             const uint8_t* scales, const float* g, int64_t m, void* Y, int out_bf16, int64_t ldy,
                             float* ws, hipStream_t s) {
  if (T <= 0 || m <= 0) return hipSuccess;
  const int sp = nvfp4_gemm_splits(T, k, m);
  const int64_t steps = (k + CK - 1) / CK;
  const int64_t ksplit = ((steps + sp - 1) / sp) * CK;
  const int nz = (int)((k + ksplit - 1) / ksplit);
  dim3 grid((unsigned)((m + CT - 1) / CT), (unsigned)((T + CT - 1) / CT), (unsigned)nz);
  if (nz > 1) {
    hipLaunchKernelGGL(nvfp4_gemm_kernel<2>, grid, dim3(256), 0, s, X, T, k, ldx, codes, scales, g, m, (void*)ws,
                       ldy, ksplit);
    const dim3 rg((unsigned)((T * m + 255) / 256));
    if (out_bf16)
      hipLaunchKernelGGL(nvfp4_gemm_reduce_kernel<true>, rg, dim3(256), 0, s, ws, nz, T, m, g, Y, ldy);
    else
      hipLaunchKernelGGL(nvfp4_gemm_reduce_kernel<false>, rg, dim3(256), 0, s, ws, nz, T, m, g, Y, ldy);
  } else if (out_bf16) {
    hipLaunchKernelGGL(nvfp4_gemm_kernel<1>, grid, dim3(256), 0, s, X, T, k, ldx, codes, scales, g, m, Y, ldy, ksplit);
  } else {
    hipLaunchKernelGGL(nvfp4_gemm_kernel<0>, grid, dim3(256), 0, s, X, T, k, ldx, codes, scales, g, m, Y, ldy, ksplit);
  }
  return hipGetLastError();
}

}  // namespace nvq
