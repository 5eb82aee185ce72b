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
// column l of the whole symmetric block in registers (c[i] = S[i][l]).  At
// step j the trailing block loses the rank-1 term S[:,j] S[j,:] / S[j][j]:
// lane l's multiplier S[l][j] / S[j][j] is its own c[j] (symmetry) and the
// broadcast S[i][j] comes from lane j by readlane, so a step needs no LDS and
// no barrier; columns are scaled by 1/sqrt(pivot) once at the end.  The
// inverse is then solved column by column (lane c: L x = e_c).  Sets *info
// (once) on a non-positive pivot: info = p + j + 1 is the order of the failing
// leading minor of A, i.e. of the failing trailing minor of H + lam I.
__global__ __launch_bounds__(64) void potf2_inv_kernel(float* __restrict__ A, int64_t k, int64_t p,
                                                       float* __restrict__ Linv, float* __restrict__ Dinv,
                                                       int32_t* __restrict__ info) {
  const int lane = threadIdx.x;
  const int nb = (int)min((int64_t)NB, k - p);
  float c[NB];   // column `lane` of the symmetric block (only the lower part of A is stored)
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int r = i > lane ? i : lane, q = i > lane ? lane : i;
    float v = 0.0f;
    if (r < nb) v = A[(p + r) * k + p + q];
    else if (i == lane) v = 1.0f;   // pad beyond k with identity
    c[i] = v;
  }
  bool bad = false;
  float piv = 1.0f;   // this lane's pivot S[lane][lane] at its step
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    __builtin_amdgcn_sched_barrier(0);   // keep each step's broadcasts within the step
    float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c[j]), j));
    if (!(d > 0.0f)) {
      if (!bad && j < nb && lane == 0 && *info == 0) *info = (int32_t)(p + j + 1);
      bad = true;
      d = 1.0f;
    }
    if (lane == j) piv = d;
    const float m = (lane > j) ? c[j] / d : 0.0f;
#pragma unroll
    for (int i = j + 1; i < NB; ++i) {
      const float sij = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c[i]), j));
      c[i] = fmaf(-sij, m, c[i]);
    }
  }
  // L[i][lane] = c[i] / sqrt(piv) below the diagonal, sqrt(piv) on it.
  const float sd = sqrtf(piv), rs = 1.0f / sd;
#pragma unroll
  for (int i = 0; i < NB; ++i) c[i] = (i > lane) ? c[i] * rs : (i == lane ? sd : 0.0f);
  // Rows of L to registers (lane = row) through LDS, then L^-1 by forward
  // elimination on [L | I]: after step j, row j of the unscaled inverse is
  // final and rows below subtract L[i][j] / L[j][j] times it; each row is
  // divided by its diagonal at the end.  Row j is broadcast by readlane.
  __shared__ float Ls[NB][NB + 1];
#pragma unroll
  for (int i = 0; i < NB; ++i) Ls[i][lane] = c[i];
  __syncthreads();
  float lrow[NB], x[NB];
#pragma unroll
  for (int q = 0; q < NB; ++q) {
    lrow[q] = Ls[lane][q];
    x[q] = (q == lane) ? 1.0f : 0.0f;
  }
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const float ljj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lrow[j]), j));
    const float f = (lane > j) ? lrow[j] / ljj : 0.0f;
#pragma unroll
    for (int q = 0; q <= j; ++q) {
      const float xj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x[q]), j));
      x[q] = fmaf(-f, xj, x[q]);
    }
  }
  const float rdiag = rs;   // 1 / L[lane][lane]
#pragma unroll
  for (int q = 0; q < NB; ++q) x[q] = (q <= lane) ? x[q] * rdiag : 0.0f;
  // Transpose the inverse back through LDS so that stores are row-coalesced.
  __syncthreads();
#pragma unroll
  for (int q = 0; q < NB; ++q) Ls[lane][q] = x[q];
  __syncthreads();
  // Row-major writes: lane = column.
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const float xv = Ls[i][lane];
    if (i < nb && lane < nb) {
      if (lane <= i) A[(p + i) * k + p + lane] = c[i];
      Linv[(p + i) * k + p + lane] = xv;
    }
    Dinv[i * NB + lane] = xv;
  }
}

// Panel solve below a factored diagonal block: A21 := A21 * Dinv^T, where
// Dinv = L11^-1 (64 x 64, lower).  Rows are independent: a workgroup takes 16
// rows; thread t computes 4 of the 16 x 64 outputs.
__global__ __launch_bounds__(256) void panel_solve_kernel(float* __restrict__ A, int64_t k, int64_t p,
                                                          int64_t rows, const float* __restrict__ Dinv) {
  __shared__ float D[NB][NB + 1];
  __shared__ float R[16][NB + 1];
  const int tid = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * 16;
  for (int e = tid; e < NB * NB; e += 256) D[e / NB][e % NB] = Dinv[e];
  for (int e = tid; e < 16 * NB; e += 256) {
    const int r = e / NB, c = e % NB;
    R[r][c] = (r0 + r < rows) ? A[(p + NB + r0 + r) * k + p + c] : 0.0f;
  }
  __syncthreads();
  const int r = tid >> 4, cb = tid & 15;
  float out[4] = {0.f, 0.f, 0.f, 0.f};
  for (int l = 0; l < NB; ++l) {
    const float a = R[r][l];
#pragma unroll
    for (int q = 0; q < 4; ++q) out[q] = fmaf(a, D[cb + 16 * q][l], out[q]);
  }
  if (r0 + r < rows) {
#pragma unroll
    for (int q = 0; q < 4; ++q) A[(p + NB + r0 + r) * k + p + cb + 16 * q] = out[q];
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
    // Panel below the block: A21 := A21 * Dinv^T.
    hipLaunchKernelGGL(panel_solve_kernel, dim3((unsigned)((rest + 15) / 16)), dim3(256), 0, s, A, k, p, rest, Dinv);
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
