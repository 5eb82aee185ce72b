// Damped inverse factor for the GPTQ sweep: upper U with (H + lam I)^-1 = U^T U.
//
// With J the index reversal, A = J (H + lam I) J = L L^T (lower Cholesky), and
// R = J L J is upper with H + lam I = R R^T, so U = R^-1 = J L^-1 J.  The
// library therefore factors the reversed matrix with a right-looking blocked
// Cholesky (64-column panels: one launch factors the diagonal block and
// solves the panel below it, one launch applies the lower-triangular
// trailing update), inverts the 64x64 diagonal blocks of L in one batched
// launch, completes L^-1 by recursive doubling (at each level, for every pair
// of adjacent diagonal blocks, X21 = -L22^-1 L21 L11^-1 with two batched
// GEMMs) and finally writes U[i][j] = L^-1[k-1-i][k-1-j].  Everything is
// fp32.
#include <utility>

#include "common.h"
#include "kernels.h"

namespace nvq {

namespace {

constexpr int NB = 64;
constexpr int SW = 8 * NB;   // super-panel width of the trailing updates

__global__ __launch_bounds__(256) void damping_kernel(const float* __restrict__ H, int64_t k, float damp_rel,
                                                      float* __restrict__ lam_ws, float* __restrict__ lam_out,
                                                      int32_t* __restrict__ info) {
  __shared__ float red[256];
  // Eight diagonal loads in flight at a time, added in the same order.
  float s = 0.0f;
  int64_t i = threadIdx.x;
  for (; i + 7 * 256 < k; i += 8 * 256) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = H[(i + u * 256) * k + (i + u * 256)];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; i < k; i += 256) s += H[i * k + i];
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
// Four columns j .. j+3 per thread, 16-byte loads and stores (k % 4 == 0):
// H's elements (k-1-i, k-4-j .. k-1-j) in reverse order.
__global__ void flip_damp_kernel(const float* __restrict__ H, int64_t k, const float* __restrict__ lam,
                                 float* __restrict__ A) {
  const int64_t i = blockIdx.y, j = 4 * ((int64_t)blockIdx.x * blockDim.x + threadIdx.x);
  if (j > i || j >= k) return;
  const f32x4 h = *(const f32x4*)(H + (k - 1 - i) * k + (k - 4 - j));
  f32x4 v = f32x4{h[3], h[2], h[1], h[0]};
  if (j + 3 <= i) {
    if (i < j + 4) v[i - j] += *lam;
    *(f32x4*)(A + i * k + j) = v;
  } else {
    // the vector holding the diagonal: its columns up to i only
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (j + u <= i) A[i * k + j + u] = j + u == i ? v[u] + *lam : v[u];
  }
}

// Lane n of each row of 16 lanes, broadcast to the row (DPP row_newbcast;
// every lane's source is valid, so no old value is needed and the move can
// fold into the instruction that uses it).
template <int N>
__device__ __forceinline__ float row_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x150 + N, 0xF, 0xF, false));
}

// Cholesky factor of a 16 x 16 SPD block S held as columns, and the inverse
// of the factor: lane l (of each row of 16 lanes, lf = l as a float) enters
// with c[i] = S[i][l] and x[i] = delta(i, l), and leaves with c[i] = the
// Schur-complemented column l, so that L[i][l] = c[i] * rsv[l] for i >= l,
// rsv[j] = 1 / L[j][j] (the same in every lane), and x = column l of L^-1.
// Column j comes to every lane by row broadcast; lanes l <= j, whose columns
// are final, have their multiplier scaled by 0 (no per-lane comparisons).
// The same broadcast column gives L[i][j] = bc[i] * rsv[j], with which step j
// finishes x[j] = x[j] / L[j][j] and removes its term from the later x[i]
// (forward substitution by columns: the updates of one step are independent).
// A non-positive pivot j is replaced by 1 and reported in bad (the first
// such j), so the arithmetic stays finite.
template <int J>
__device__ __forceinline__ void chol16_step(float (&c)[16], float (&x)[16], float lf, float (&rsv)[16], int& bad) {
  float bc[16];
#pragma unroll
  for (int i = J; i < 16; ++i) bc[i] = row_bcast<J>(c[i]);
  float d = bc[J];
  const bool ok = d > 0.0f;
  bad = (!ok && bad < 0) ? J : bad;
  d = ok ? d : 1.0f;
  rsv[J] = __builtin_amdgcn_rsqf(d);
  const float act = __builtin_amdgcn_fmed3f(lf - (float)J, 0.0f, 1.0f);   // 1 for l > J, else 0
  const float negm = -(c[J] * __builtin_amdgcn_rcpf(d)) * act;
#pragma unroll
  for (int i = J + 1; i < 16; ++i) c[i] = fmaf(bc[i], negm, c[i]);
  x[J] *= rsv[J];
  const float t = -(x[J] * rsv[J]);   // -x[J] / L[J][J]
#pragma unroll
  for (int i = J + 1; i < 16; ++i) x[i] = fmaf(bc[i], t, x[i]);
}
__device__ __forceinline__ void chol16(float (&c)[16], float (&x)[16], float lf, float (&rsv)[16], int& bad) {
  [&]<int... J>(std::integer_sequence<int, J...>) {
    (chol16_step<J>(c, x, lf, rsv, bad), ...);
  }(std::make_integer_sequence<int, 16>{});
}

// Panel p of the blocked Cholesky factorization (columns p .. p+nb-1 of the
// lower factor).  Every workgroup factors the nb x nb diagonal block itself
// (identical arithmetic, so identical results) and then solves its own 64
// rows of the panel below it: L21 = A21 L11^-T.  Inside the workgroup the
// block is factored in 16-column steps: one wave factors and inverts the
// 16 x 16 diagonal sub-block in registers; then the rows below it (the
// block's own rows and the panel rows) are multiplied by the inverse's
// transpose, and the step's contribution is subtracted from the columns to
// its right, both as 16 x 16 tiles on the matrix cores
// (v_mfma_f32_16x16x4f32, one tile per wave at a time).  Workgroup 0 stores
// L11 and, on a non-positive pivot, sets *info (once) to the order of the
// failing leading minor of the reversed matrix, i.e. of the failing trailing
// minor of H + lam I.
//
// 16x16x4 operand layout: lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16]; accumulator register r of lane l is D[4 (l / 16) + r][l % 16].
constexpr int SP = NB + 4;   // LDS row stride: the tiles' operand and accumulator accesses are conflict free
__global__ __launch_bounds__(256) void panel_kernel(float* __restrict__ A, int64_t k, int64_t p,
                                                    int32_t* __restrict__ info) {
  // Rows 0..63: the diagonal block (lower part; -> L11); rows 64..127: this
  // workgroup's panel rows (-> L21 rows).
  __shared__ __attribute__((aligned(16))) float V[2 * NB][SP];
  __shared__ float Li[16][17];   // inverse of the current 16 x 16 diagonal sub-block
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  const int nb = (int)min((int64_t)NB, k - p);
  const int64_t r0 = (int64_t)blockIdx.x * NB;
  const int rows = (int)max((int64_t)0, min((int64_t)NB, k - p - nb - r0));
  // All loads first (16-byte, clamped to valid rows), then the LDS writes.
  f32x4 ld[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int e = tid + 256 * (q & 3), i = e >> 4, j4 = (e & 15) * 4;
    const int64_t row = q < 4 ? p + min(i, nb - 1) : p + nb + r0 + min(i, max(rows - 1, 0));
    // nb is a multiple of 16: a 4-column group lies wholly inside or past it.
    ld[q] = (q < 4 || rows > 0) ? *(const f32x4*)(A + row * k + p + min(j4, nb - 4)) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int e = tid + 256 * (q & 3), i = e >> 4, j4 = (e & 15) * 4;
    f32x4 v;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j4 + u;
      if (q < 4) v[u] = (i < nb && j < nb) ? (j <= i ? ld[q][u] : 0.0f) : (i == j ? 1.0f : 0.0f);
      else v[u] = (i < rows && j < nb) ? ld[q][u] : 0.0f;
    }
    *(f32x4*)&V[q < 4 ? i : NB + i][j4] = v;
  }
  __syncthreads();
  int first_bad = 0;
  // Wave 0 factors and inverts sub-block o (16 x 16 at rows/columns o).
  auto factor_sub = [&](int o) {
    // The lane index is made opaque here, so that the compiler forms what
    // depends on it where it is used.
    int lo = l16;
    asm volatile("" : "+v"(lo));
    const float lf = (float)lo;
    float c[16], rsv[16], x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      c[i] = V[o + max(i, lo)][o + min(i, lo)];
      const float dl = lf - (float)i;
      x[i] = fmaxf(fmaf(-dl, dl, 1.0f), 0.0f);   // delta(i, l)
    }
    int bad = -1;
    chol16(c, x, lf, rsv, bad);
    if (bad >= 0 && first_bad == 0 && o + bad < nb) first_bad = (int)(p + o + bad + 1);
    // Lane l's scale 1 / L[l][l], through LDS (column 16 of Li is spare).
    if (lane == 0) {
#pragma unroll
      for (int j = 0; j < 16; ++j) Li[j][16] = rsv[j];
    }
    const float rsl = Li[lo][16];
    // L into V (entries above the diagonal get values that nothing reads).
    if (lane < 16) {
#pragma unroll
      for (int i = 0; i < 16; ++i) V[o + i][o + lane] = c[i] * rsl;
    }
    if (lane < 16) {
#pragma unroll
      for (int i = 0; i < 16; ++i) Li[i][lane] = x[i];
    }
  };
  if (wave == 0) factor_sub(0);
  __syncthreads();
  for (int b = 0; b < NB / 16; ++b) {
    const int o = 16 * b;
    // Rows below the sub-block (o+16 .. 127): columns o..o+15 := V Li^T.
    const int nrt = (2 * NB - o - 16) / 16;
    for (int t = wave; t < nrt; t += 4) {
      const int t0 = o + 16 + 16 * t;
      float av[4], bv[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        av[kk] = V[t0 + l16][o + 4 * kk + lq];
        bv[kk] = Li[l16][4 * kk + lq];
      }
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[kk], bv[kk], acc, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) V[t0 + 4 * lq + r][o + l16] = acc[r];
    }
    __syncthreads();
    // Columns right of the step (o+16 .. 63), every row below:
    // V[r][j] -= V[r][o:o+16] . V[j][o:o+16].  Tiles wholly above the
    // diagonal of the block are never read and are skipped.  Wave 0 updates
    // the next diagonal sub-block (tile 0) and goes on to factor it while
    // waves 1-3 update the other tiles.
    const int nct = (NB - o - 16) / 16;
    auto c_tile = [&](int t) {
      const int ti = t / nct, tj = t % nct;
      const int t0 = o + 16 + 16 * ti, j0 = o + 16 + 16 * tj;
      if (t0 < j0) return;
      float av[4], bv[4];
      f32x4 acc;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = V[t0 + 4 * lq + r][j0 + l16];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        av[kk] = -V[t0 + l16][o + 4 * kk + lq];
        bv[kk] = V[j0 + l16][o + 4 * kk + lq];
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[kk], bv[kk], acc, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) V[t0 + 4 * lq + r][j0 + l16] = acc[r];
    };
    if (nct > 0) {
      if (wave == 0) {
        c_tile(0);
        factor_sub(o + 16);
      } else {
        for (int t = wave; t < nrt * nct; t += 3) c_tile(t);
      }
    }
    __syncthreads();
  }
  // 16-byte stores; the diagonal block's upper triangle is written as zeros.
  if (blockIdx.x == 0 && tid == 0 && first_bad != 0 && *info == 0) *info = first_bad;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int e = tid + 256 * (q & 3), i = e >> 4, j4 = (e & 15) * 4;
    if ((q < 4 ? (blockIdx.x != 0 || i >= nb) : i >= rows) || j4 >= nb) continue;
    f32x4 v = *(const f32x4*)&V[q < 4 ? i : NB + i][j4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (q < 4 && j4 + u > i) v[u] = 0.0f;
    *(f32x4*)(A + (q < 4 ? p + i : p + nb + r0 + i) * k + p + j4) = v;
  }
}

// Trailing update by the kw panel columns starting at column p: C -= P P^T
// on the lower triangle, where P is those columns' L21 (rest x kw, at
// A + (p+kw) k + p) and C the block right of and below them (rest x rest, at
// A + (p+kw)(k+1)).  With lim < 0 every lower tile is updated; otherwise only
// the tiles in the first lim 64-column blocks of C (grid lim x tiles; the
// workgroups of tiles above the diagonal exit).  One workgroup per 64 x 64
// tile; each wave holds a 32 x 32 quadrant in MFMA accumulators initialized
// from C, and multiplies -P_i by P_j^T (v_mfma_f32_32x32x2f32) in chunks of
// 64 columns, in column order, so that C is read and written once for all kw
// columns and every element sees the same sums in the same order as kw / 64
// separate updates.
constexpr int UP = NB + 2;   // LDS row stride: a lane's (row, k) reads hit 64 distinct banks
__global__ __launch_bounds__(256) void chol_update_kernel(float* __restrict__ A, int64_t k, int64_t p,
                                                          int64_t rest, int kw, int lim) {
  __shared__ float Pi[NB][UP], Pj[NB][UP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t = blockIdx.x;
  int64_t ti, tj;
  if (lim < 0) {
    // Tile t -> (ti, tj), tj <= ti, row-major over the lower triangle of tiles.
    ti = (int64_t)((sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
    while (ti * (ti + 1) / 2 > t) --ti;
    while ((ti + 1) * (ti + 2) / 2 <= t) ++ti;
    tj = t - ti * (ti + 1) / 2;
  } else {
    const int64_t nt = (rest + NB - 1) / NB;
    tj = t / nt;
    ti = t % nt;
    if (ti < tj) return;
  }
  const float* P = A + (p + kw) * k + p;
  float* C = A + (p + kw) * k + p + kw;
  const int wr = wave >> 1, wc = wave & 1;
  const int64_t col = tj * NB + wc * 32 + (lane & 31);
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t row = ti * NB + wr * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    acc[r] = (row < rest && col < rest && col <= row) ? C[row * k + col] : 0.0f;
  }
  for (int kc = 0; kc < kw; kc += NB) {
    // All panel loads in flight together (clamped rows), then the LDS writes.
    f32x4 vi[4], vj[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = q * 256 + tid, r = e / (NB / 4), c4 = (e % (NB / 4)) * 4;
      vi[q] = *(const f32x4*)(P + min(ti * NB + r, rest - 1) * k + kc + c4);
      vj[q] = *(const f32x4*)(P + min(tj * NB + r, rest - 1) * k + kc + c4);
    }
    if (kc > 0) __syncthreads();   // every wave is done with the previous chunk
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = q * 256 + tid, r = e / (NB / 4), c4 = (e % (NB / 4)) * 4;
      const bool oki = ti * NB + r < rest, okj = tj * NB + r < rest;
#pragma unroll
      for (int u = 0; u < 4; ++u) { Pi[r][c4 + u] = oki ? -vi[q][u] : 0.0f; Pj[r][c4 + u] = okj ? vj[q][u] : 0.0f; }
    }
    __syncthreads();
    const float* pa = &Pi[wr * 32 + (lane & 31)][lane >> 5];
    const float* pb = &Pj[wc * 32 + (lane & 31)][lane >> 5];
    // Operands of the next 16 k-values are read while the current 8 MFMAs run.
    float a8[2][8], b8[2][8];
#pragma unroll
    for (int u = 0; u < 8; ++u) { a8[0][u] = pa[2 * u]; b8[0][u] = pb[2 * u]; }
#pragma unroll
    for (int h = 0; h < NB / 16; ++h) {
      if (h + 1 < NB / 16) {
#pragma unroll
        for (int u = 0; u < 8; ++u) { a8[(h + 1) & 1][u] = pa[16 * (h + 1) + 2 * u]; b8[(h + 1) & 1][u] = pb[16 * (h + 1) + 2 * u]; }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < 8; ++u) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a8[h & 1][u], b8[h & 1][u], acc, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t row = ti * NB + wr * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    if (row < rest && col < rest && col <= row) C[row * k + col] = acc[r];
  }
}

// Inverses of the diagonal 64-blocks of L (one wave each) into Linv: lane c
// solves L x = e_c by forward substitution (column c of the inverse), with
// the block in LDS so that row i of L reaches every lane as broadcast reads
// (the same address in every lane), four values at a time.
__global__ __launch_bounds__(64) void diag_inv_kernel(const float* __restrict__ A, int64_t k,
                                                      float* __restrict__ Linv) {
  __shared__ __attribute__((aligned(16))) float Ls[NB][NB];
  const int lane = threadIdx.x;
  const int64_t p = (int64_t)blockIdx.x * NB;
  const int nb = (int)min((int64_t)NB, k - p);
  // L's lower part; the identity outside nb.
#pragma unroll 8
  for (int i = 0; i < NB; ++i) {
    float v = (i == lane) ? 1.0f : 0.0f;
    if (i < nb && lane < nb && lane <= i) v = A[(p + i) * k + p + lane];
    Ls[i][lane] = v;
  }
  __syncthreads();
  float x[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    float acc = (i == lane) ? 1.0f : 0.0f;
#pragma unroll
    for (int m = 0; m < i; ++m) acc = fmaf(-Ls[i][m], x[m], acc);
    x[i] = acc * (1.0f / Ls[i][i]);
    // Row by row: x[i] is formed here (not sunk to its stores, which would
    // keep every value read alive), and later rows' reads stay below.
    asm volatile("" : "+v"(x[i]) :: "memory");
  }
#pragma unroll
  for (int i = 0; i < NB; ++i)
    if (i < nb && lane < nb) Linv[(p + i) * k + p + lane] = x[i];
}

// U[i][j] = Linv[k-1-i][k-1-j] for j >= i, 0 below the diagonal.
// Four columns j .. j+3 per thread, 16-byte loads and stores (k % 4 == 0).
__global__ void flip_out_kernel(const float* __restrict__ Linv, int64_t k, float* __restrict__ U) {
  const int64_t i = blockIdx.y, j = 4 * ((int64_t)blockIdx.x * blockDim.x + threadIdx.x);
  if (j >= k) return;
  f32x4 v = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (j + 3 >= i) {
    const f32x4 l = *(const f32x4*)(Linv + (k - 1 - i) * k + (k - 4 - j));
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = j + u >= i ? l[3 - u] : 0.0f;
  }
  *(f32x4*)(U + i * k + j) = v;
}

// p[0 .. 4 n4) = 0 in 16-byte stores (p 16-byte aligned).
__global__ void zero_kernel(float* p, int64_t n4) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n4) ((f32x4*)p)[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
}

}  // namespace

size_t factor_workspace(int64_t k) {
  // A (k^2), Linv (k^2), T (k^2 / 2), lam (64 floats)
  return ((size_t)k * k * 2 + (size_t)k * k / 2 + 64) * sizeof(float);
}

hipError_t factor_hinv_launch(const float* H, int64_t k, float damp_rel, float* U, float* lambda_out,
                              int32_t* info, void* ws, hipStream_t s) {
  float* A = (float*)ws;
  float* Linv = A + (size_t)k * k;
  float* T = Linv + (size_t)k * k;
  float* lam = T + (size_t)k * k / 2;

  hipLaunchKernelGGL(damping_kernel, dim3(1), dim3(256), 0, s, H, k, damp_rel, lam, lambda_out, info);
  // k % 16 == 0, so k * k is a multiple of 4 (and Linv, k * k floats into the workspace, is 16-byte aligned).
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)(((size_t)k * k / 4 + 255) / 256)), dim3(256), 0, s, Linv,
                     (int64_t)k * k / 4);
  hipLaunchKernelGGL(flip_damp_kernel, dim3((unsigned)((k / 4 + 255) / 256), (unsigned)k), dim3(256), 0, s, H, k,
                     lam, A);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  // Panels are grouped in super-panels of SW columns.  After each panel only
  // the rest of its super-panel is updated (the columns the next panels
  // factor); the columns right of the super-panel take all of its panels in
  // one update after its last panel, so they are read and written once per
  // SW columns instead of once per panel.
  for (int64_t p = 0; p < k; p += NB) {
    const int64_t rest = k - p - NB;
    const unsigned groups = rest > 0 ? (unsigned)((rest + NB - 1) / NB) : 1u;
    hipLaunchKernelGGL(panel_kernel, dim3(groups), dim3(256), 0, s, A, k, p, info);
    if (rest <= 0) break;
    const int64_t s0 = p / SW * SW, send = min(s0 + SW, k);
    if (p + NB < send) {
      const int64_t tiles = (rest + NB - 1) / NB, lim = (send - p - NB + NB - 1) / NB;
      hipLaunchKernelGGL(chol_update_kernel, dim3((unsigned)(lim * tiles)), dim3(256), 0, s, A, k, p, rest, NB,
                         (int)lim);
    } else if (send < k) {
      const int64_t rest2 = k - send, tiles = (rest2 + NB - 1) / NB;
      hipLaunchKernelGGL(chol_update_kernel, dim3((unsigned)(tiles * (tiles + 1) / 2)), dim3(256), 0, s, A, k, s0,
                         rest2, (int)(send - s0), -1);
    }
  }
  hipLaunchKernelGGL(diag_inv_kernel, dim3((unsigned)((k + NB - 1) / NB)), dim3(64), 0, s, A, k, Linv);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

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
      a.alpha = 1.0f; a.beta = 0.0f; a.kmode = kGemmKLowerB;   // L11^-1 is lower triangular
      hipError_t err = gemm_f32(a, false, false, false, kEpiAxpby, s);
      if (err != hipSuccess) return err;
      // X21 = -L22^-1 * T   (n2 x n1), written into Linv
      GemmArgs b{};
      b.A = Linv + (base + bs) * k + (base + bs); b.lda = k;
      b.B = T; b.ldb = n1;
      b.C = Linv + (base + bs) * k + base; b.ldc = k;
      b.M = n2; b.N = n1; b.K = n2; b.batch = batch;
      b.sA = 2 * bs * k + 2 * bs; b.sB = n1 * n2; b.sC = 2 * bs * k + 2 * bs;
      b.alpha = -1.0f; b.beta = 0.0f; b.kmode = kGemmKLowerA;  // L22^-1 is lower triangular
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
  hipLaunchKernelGGL(flip_out_kernel, dim3((unsigned)((k / 4 + 255) / 256), (unsigned)k), dim3(256), 0, s, Linv, k,
                     U);
  return hipGetLastError();
}

}  // namespace nvq
