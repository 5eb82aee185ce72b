// Damped inverse factor for the GPTQ sweep: upper U with (H + lam I)^-1 = U^T U.
//
// With J the index reversal, A = J (H + lam I) J = L L^T (lower Cholesky), and
// R = J L J is upper with H + lam I = R R^T, so U = R^-1 = J L^-1 J.  The
// library therefore factors the reversed matrix with a right-looking blocked
// Cholesky (64-column panels: a one-workgroup panel factorization that also
// inverts the 64x64 diagonal block, a GEMM for the panel below it and a
// lower-triangular GEMM for the trailing update), inverts L by recursive
// doubling (at each level, for every pair of adjacent diagonal blocks,
// X21 = -L22^-1 L21 L11^-1 with two batched GEMMs) and finally writes
// U[i][j] = L^-1[k-1-i][k-1-j].  Everything is fp32.
#include "common.h"
#include "kernels.h"

namespace nvq {

namespace {

constexpr int NB = 64;

__global__ __launch_bounds__(256) void damping_kernel(const float* __restrict__ H, int64_t k, float damp_rel,
                                                      float* __restrict__ lam_ws, float* __restrict__ lam_out,
                                                      int32_t* __restrict__ info) {
  __shared__ float red[256];
  float s = 0.0f;
  for (int64_t i = threadIdx.x; i < k; i += 256) s += H[i * k + i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    float lam = damp_rel * (red[0] / (float)k);
    *lam_ws = lam;
    *lam_out = lam;
    *info = 0;
  }
}

// A[i][j] = H[k-1-i][k-1-j] + lam * (i == j), lower triangle (reads H's upper triangle).
__global__ void flip_damp_kernel(const float* __restrict__ H, int64_t k, const float* __restrict__ lam,
                                 float* __restrict__ A) {
  int64_t i = blockIdx.y, j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j > i || j >= k) return;
  float v = H[(k - 1 - i) * k + (k - 1 - j)];
  if (i == j) v += *lam;
  A[i * k + j] = v;
}

// Factor the 64x64 diagonal block at p in place (lower L), write its inverse
// into Linv's diagonal block and into Dinv [64 x 64].  One wave; lane l keeps
// column l of the block in registers.  Cholesky step j: lane j scales its
// column and publishes it in LDS, every lane l > j subtracts L[l][j] times it.
// The inverse is then solved column by column (lane c: L x = e_c) against an
// LDS copy of L, one row per step.  Sets *info (once) on a non-positive pivot:
// info = p + j + 1 is the order of the failing leading minor of A, i.e. of the
// failing trailing minor of H + lam I.
__global__ __launch_bounds__(64) void potf2_inv_kernel(float* __restrict__ A, int64_t k, int64_t p,
                                                       float* __restrict__ Linv, float* __restrict__ Dinv,
                                                       int32_t* __restrict__ info) {
  __shared__ __attribute__((aligned(16))) float colj[NB];
  __shared__ __attribute__((aligned(16))) float Ls[NB][NB + 4];
  const int lane = threadIdx.x;
  const int nb = (int)min((int64_t)NB, k - p);
  float c[NB];   // column `lane`: c[i] = A[i][lane] (lower part meaningful)
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    float v = 0.0f;
    if (i < nb && lane < nb && lane <= i) v = A[(p + i) * k + p + lane];
    else if (i == lane) v = 1.0f;   // pad beyond k with identity
    c[i] = v;
  }
  bool bad = false;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c[j]), j));
    if (!(d > 0.0f)) {
      if (!bad && j < nb && lane == 0 && *info == 0) *info = (int32_t)(p + j + 1);
      bad = true;
      d = 1.0f;
    }
    const float sd = sqrtf(d), rs = 1.0f / sd;
    if (lane == j) {
      c[j] = sd;
#pragma unroll
      for (int i = j + 1; i < NB; ++i) {
        c[i] *= rs;
        colj[i] = c[i];
      }
    }
    __syncthreads();
    if (lane > j) {
      const float cl = colj[lane];
#pragma unroll
      for (int i = j + 1; i < NB; ++i) c[i] = fmaf(-colj[i], cl, c[i]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) Ls[i][lane] = (lane <= i) ? c[i] : 0.0f;
  __syncthreads();
  // Column `lane` of L^-1 (x reuses c's registers).
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    __builtin_amdgcn_sched_barrier(0);
    float a0 = (i == lane) ? 1.0f : 0.0f, a1 = 0.0f;
#pragma unroll
    for (int l = 0; l + 1 < i; l += 2) {
      a0 = fmaf(-Ls[i][l], c[l], a0);
      a1 = fmaf(-Ls[i][l + 1], c[l + 1], a1);
    }
    if (i & 1) a0 = fmaf(-Ls[i][i - 1], c[i - 1], a0);
    c[i] = (a0 + a1) / Ls[i][i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const float xv = (lane <= i) ? c[i] : 0.0f;   // L^-1[i][lane]
    if (i < nb && lane < nb) {
      if (lane <= i) A[(p + i) * k + p + lane] = Ls[i][lane];
      Linv[(p + i) * k + p + lane] = xv;
    }
    Dinv[i * NB + lane] = xv;
  }
}

// U[i][j] = Linv[k-1-i][k-1-j] for j >= i, 0 below the diagonal.
__global__ void flip_out_kernel(const float* __restrict__ Linv, int64_t k, float* __restrict__ U) {
  int64_t i = blockIdx.y, j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= k) return;
  U[i * k + j] = (j >= i) ? Linv[(k - 1 - i) * k + (k - 1 - j)] : 0.0f;
}

__global__ void zero_kernel(float* p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

}  // namespace

size_t factor_workspace(int64_t k) {
  // A (k^2), Linv (k^2), T (k^2 / 2), Dinv (64^2), lam (64 floats)
  return ((size_t)k * k * 2 + (size_t)k * k / 2 + NB * NB + 64) * sizeof(float);
}

hipError_t factor_hinv_launch(const float* H, int64_t k, float damp_rel, float* U, float* lambda_out,
                              int32_t* info, void* ws, hipStream_t s) {
  float* A = (float*)ws;
  float* Linv = A + (size_t)k * k;
  float* T = Linv + (size_t)k * k;
  float* Dinv = T + (size_t)k * k / 2;
  float* lam = Dinv + NB * NB;

  hipLaunchKernelGGL(damping_kernel, dim3(1), dim3(256), 0, s, H, k, damp_rel, lam, lambda_out, info);
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)(((size_t)k * k + 255) / 256)), dim3(256), 0, s, Linv,
                     (int64_t)k * k);
  hipLaunchKernelGGL(flip_damp_kernel, dim3((unsigned)((k + 255) / 256), (unsigned)k), dim3(256), 0, s, H, k,
                     lam, A);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  for (int64_t p = 0; p < k; p += NB) {
    hipLaunchKernelGGL(potf2_inv_kernel, dim3(1), dim3(64), 0, s, A, k, p, Linv, Dinv, info);
    int64_t rest = k - p - NB;
    if (rest <= 0) break;
    // Panel below the block: A21 := A21 * Dinv^T (in place; one tile column).
    GemmArgs t{};
    t.A = A + (p + NB) * k + p; t.lda = k;
    t.B = Dinv; t.ldb = NB;
    t.C = A + (p + NB) * k + p; t.ldc = k;
    t.M = rest; t.N = NB; t.K = NB; t.batch = 1; t.alpha = 1.0f; t.beta = 0.0f;
    e = gemm_f32(t, false, true, false, kEpiAxpby, s);
    if (e != hipSuccess) return e;
    // Trailing update: A22 -= A21 A21^T (lower tiles).
    GemmArgs u{};
    u.A = A + (p + NB) * k + p; u.lda = k;
    u.B = A + (p + NB) * k + p; u.ldb = k;
    u.C = A + (p + NB) * k + p + NB; u.ldc = k;
    u.M = rest; u.N = rest; u.K = NB; u.batch = 1; u.alpha = -1.0f; u.beta = 1.0f;
    e = gemm_f32(u, false, true, true, kEpiAxpby, s);
    if (e != hipSuccess) return e;
  }

  // Triangular inverse by recursive doubling over diagonal blocks of size bs.
  for (int64_t bs = NB; bs < k; bs *= 2) {
    int64_t full = k / (2 * bs);  // pairs whose both halves are complete
    auto pair_step = [&](int64_t base, int64_t n1, int64_t n2, int batch) -> hipError_t {
      // T = L21 * L11^-1   (n2 x n1)
      GemmArgs a{};
      a.A = A + (base + bs) * k + base; a.lda = k;
      a.B = Linv + base * k + base; a.ldb = k;
      a.C = T; a.ldc = n1;
      a.M = n2; a.N = n1; a.K = n1; a.batch = batch;
      a.sA = 2 * bs * k + 2 * bs; a.sB = 2 * bs * k + 2 * bs; a.sC = n1 * n2;
      a.alpha = 1.0f; a.beta = 0.0f;
      hipError_t err = gemm_f32(a, false, false, false, kEpiAxpby, s);
      if (err != hipSuccess) return err;
      // X21 = -L22^-1 * T   (n2 x n1), written into Linv
      GemmArgs b{};
      b.A = Linv + (base + bs) * k + (base + bs); b.lda = k;
      b.B = T; b.ldb = n1;
      b.C = Linv + (base + bs) * k + base; b.ldc = k;
      b.M = n2; b.N = n1; b.K = n2; b.batch = batch;
      b.sA = 2 * bs * k + 2 * bs; b.sB = n1 * n2; b.sC = 2 * bs * k + 2 * bs;
      b.alpha = -1.0f; b.beta = 0.0f;
      return gemm_f32(b, false, false, false, kEpiAxpby, s);
    };
    if (full > 0) {
      e = pair_step(0, bs, bs, (int)full);
      if (e != hipSuccess) return e;
    }
    int64_t base = full * 2 * bs;
    if (base + bs < k) {
      e = pair_step(base, bs, k - base - bs, 1);
      if (e != hipSuccess) return e;
    }
  }
  hipLaunchKernelGGL(flip_out_kernel, dim3((unsigned)((k + 255) / 256), (unsigned)k), dim3(256), 0, s, Linv, k,
                     U);
  return hipGetLastError();
}

}  // namespace nvq
