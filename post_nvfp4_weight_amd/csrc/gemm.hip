// fp32 GEMM on CDNA4 matrix cores (v_mfma_f32_32x32x2_f32).
//
// One 256-thread workgroup computes a 128x128 tile of C; its four waves hold
// 64x64 sub-tiles as 2x2 MFMA 32x32 accumulators.  K is consumed in chunks of
// 16 staged through LDS (A transposed so both operands are read as
// [k][row/col] with one float per lane per MFMA).  Used for the GPTQ trailing
// update, the Cholesky panel/trailing updates, the triangular inverse and the
// weighted error (row-dot epilogue).
#include "common.h"
#include "kernels.h"

namespace nvq {

namespace {

constexpr int BM = 128, BN = 128, BK = 16, PAD = 4;

template <bool TA, bool TB, bool LOWER, int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs p) {
  if (LOWER && blockIdx.x > blockIdx.y) return;
  __shared__ __attribute__((aligned(16))) float As[BK][BM + PAD];
  __shared__ __attribute__((aligned(16))) float Bs[BK][BN + PAD];
  __shared__ float red[BM][33];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
  const int64_t z = blockIdx.z;
  const float* A = p.A + z * p.sA;
  const float* B = p.B + z * p.sB;
  float* C = p.C + z * p.sC;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  for (int64_t k0 = 0; k0 < p.K; k0 += BK) {
    // ---- stage A tile (logical A'[i][kk], i in [m0, m0+128), kk in [k0, k0+16))
    if (!TA) {
      int i = tid >> 1, kk = (tid & 1) * 8;
      int64_t gi = m0 + i;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        int64_t gk = k0 + kk + 4 * h;
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (gi < p.M && gk < p.K) v = *(const f32x4*)(A + gi * p.lda + gk);
        As[kk + 4 * h + 0][i] = v[0];
        As[kk + 4 * h + 1][i] = v[1];
        As[kk + 4 * h + 2][i] = v[2];
        As[kk + 4 * h + 3][i] = v[3];
      }
    } else {
      int kk = tid >> 4, i = (tid & 15) * 8;
      int64_t gk = k0 + kk;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        int64_t gi = m0 + i + 4 * h;
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (gi < p.M && gk < p.K) v = *(const f32x4*)(A + gk * p.lda + gi);
        *(f32x4*)&As[kk][i + 4 * h] = v;
      }
    }
    // ---- stage B tile (logical B'[kk][j])
    if (!TB) {
      int kk = tid >> 4, j = (tid & 15) * 8;
      int64_t gk = k0 + kk;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        int64_t gj = n0 + j + 4 * h;
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (gj < p.N && gk < p.K) v = *(const f32x4*)(B + gk * p.ldb + gj);
        *(f32x4*)&Bs[kk][j + 4 * h] = v;
      }
    } else {
      int j = tid >> 1, kk = (tid & 1) * 8;
      int64_t gj = n0 + j;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        int64_t gk = k0 + kk + 4 * h;
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (gj < p.N && gk < p.K) v = *(const f32x4*)(B + gj * p.ldb + gk);
        Bs[kk + 4 * h + 0][j] = v[0];
        Bs[kk + 4 * h + 1][j] = v[1];
        Bs[kk + 4 * h + 2][j] = v[2];
        Bs[kk + 4 * h + 3][j] = v[3];
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; kk += 2) {
      float a[2], b[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        a[t] = As[kk + (lane >> 5)][wr * 64 + t * 32 + (lane & 31)];
        b[t] = Bs[kk + (lane >> 5)][wc * 64 + t * 32 + (lane & 31)];
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }

  // Accumulator layout of a 32x32 MFMA tile: lane l, register r holds
  // row 8*(r/4) + 4*(l/32) + r%4, column l%32.
  if (EPI == kEpiAxpby) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        int64_t gj = n0 + wc * 64 + j * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          int64_t gi = m0 + wr * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (gi < p.M && gj < p.N) {
            float v = p.alpha * acc[i][j][r];
            if (p.beta != 0.0f) v = fmaf(p.beta, C[gi * p.ldc + gj], v);
            C[gi * p.ldc + gj] = v;
          }
        }
      }
  } else {
    // Row-dot: P[row, tile] = sum over the tile's columns of alpha*acc*D.
    float part[2][16];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int64_t gi = m0 + wr * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        float s = 0.0f;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          int64_t gj = n0 + wc * 64 + j * 32 + (lane & 31);
          if (gi < p.M && gj < p.N) s = fmaf(p.alpha * acc[i][j][r], p.D[gi * p.ldd + gj], s);
        }
        part[i][r] = s;
      }
    // Each (row, wc) has 32 lanes of partials: write them and sum in a fixed order.
    for (int half = 0; half < 2; ++half) {
      if (wc == half) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            int row = wr * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            float prev = half ? red[row][lane & 31] : 0.0f;
            red[row][lane & 31] = prev + part[i][r];
          }
      }
      __syncthreads();
    }
    if (tid < BM) {
      float s = 0.0f;
      for (int c = 0; c < 32; ++c) s += red[tid][c];
      int64_t gi = m0 + tid;
      if (gi < p.M) p.P[gi * p.ldp + blockIdx.x] = s;
    }
  }
}

template <bool TA, bool TB, bool LOWER, int EPI>
hipError_t launch(const GemmArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((a.N + BN - 1) / BN), (unsigned)((a.M + BM - 1) / BM), (unsigned)a.batch);
  hipLaunchKernelGGL((gemm_f32_kernel<TA, TB, LOWER, EPI>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t gemm_f32(const GemmArgs& a, bool ta, bool tb, bool lower, GemmEpi epi, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0 || a.batch <= 0) return hipSuccess;
  if (epi == kEpiRowDot) {
    if (!ta && !tb && !lower) return launch<false, false, false, kEpiRowDot>(a, s);
    return hipErrorInvalidValue;
  }
  if (!ta && !tb) return lower ? launch<false, false, true, kEpiAxpby>(a, s) : launch<false, false, false, kEpiAxpby>(a, s);
  if (!ta && tb) return lower ? launch<false, true, true, kEpiAxpby>(a, s) : launch<false, true, false, kEpiAxpby>(a, s);
  if (ta && !tb) return lower ? launch<true, false, true, kEpiAxpby>(a, s) : launch<true, false, false, kEpiAxpby>(a, s);
  return launch<true, true, false, kEpiAxpby>(a, s);
}

}  // namespace nvq
