// Damped inverse factor for the GPTQ sweep: upper U with (H + lam I)^-1 = U^T U.
//
// With J the index reversal, A = J (H + lam I) J = L L^T (lower Cholesky), and
// R = J L J is upper with H + lam I = R R^T, so U = R^-1 = J L^-1 J.  The
// library therefore factors the reversed matrix with a right-looking blocked
// Cholesky (64-column panels: one launch per panel factors the diagonal block,
// solves the panel below it and applies the previous panel's trailing update,
// with one lower-triangular update per 512 columns), inverts the 64x64 diagonal blocks of L in one batched
// launch, completes L^-1 by recursive doubling (at each level, for every pair
// of adjacent diagonal blocks, X21 = -L22^-1 L21 L11^-1 with two batched
// GEMMs) and finally writes U[i][j] = L^-1[k-1-i][k-1-j].  Everything is
// fp32.
#include <mutex>
#include <utility>

#include "common.h"
#include "kernels.h"

namespace nvq {

namespace {

constexpr int NB = 64;
constexpr int SW = 8 * NB;   // super-panel width of the trailing updates

// Matrix b = blockIdx.x of a batch: H + b * stride_h, lam_ws[b], lam_out[b], info[b].
__global__ __launch_bounds__(256) void damping_kernel(const float* __restrict__ H, int64_t k, int64_t stride_h,
                                                      float damp_rel, float* __restrict__ lam_ws,
                                                      float* __restrict__ lam_out, int32_t* __restrict__ info) {
  __shared__ float red[256];
  const int64_t b = blockIdx.x;
  H += b * stride_h;
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
    lam_ws[b] = lam;
    lam_out[b] = lam;
    info[b] = __builtin_isfinite(lam) ? 0 : -1;
  }
}

// A[i][j] = H[k-1-i][k-1-j] + lam * (i == j), lower triangle (reads H's upper triangle).
// Four columns j .. j+3 per thread, 16-byte loads and stores (k % 4 == 0):
// H's elements (k-1-i, k-4-j .. k-1-j) in reverse order.  A non-finite value
// in the upper triangle of H sets *info = -1 (every writer writes the same).
// Matrix b = blockIdx.z: H + b * stride_h -> A + b * k^2 (lam[b], info[b]).
__global__ void flip_damp_kernel(const float* __restrict__ H, int64_t k, int64_t stride_h,
                                 const float* __restrict__ lam, float* __restrict__ A, int32_t* __restrict__ info) {
  const int64_t i = blockIdx.y, j = 4 * ((int64_t)blockIdx.x * blockDim.x + threadIdx.x);
  const int64_t b = blockIdx.z;
  if (j > i || j >= k) return;
  H += b * stride_h;
  A += b * k * k;
  lam += b;
  info += b;
  const f32x4 h = *(const f32x4*)(H + (k - 1 - i) * k + (k - 4 - j));
  f32x4 v = f32x4{h[3], h[2], h[1], h[0]};
  bool bad = false;
#pragma unroll
  for (int u = 0; u < 4; ++u) bad |= j + u <= i && !__builtin_isfinite(v[u]);
  if (bad) *info = -1;
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

// Trailing update of one 64 x 64 tile (ti, tj) of C by the kw columns of L
// starting at column pp: C -= P_i P_j^T on the tile's lower part, where P is
// those columns' rows below them (rest x kw, at A + (pp+kw) k + pp) and C the
// block right of and below them (rest x rest, at A + (pp+kw)(k+1)).  Each of
// the four waves holds a 32 x 32 quadrant in MFMA accumulators initialized
// from C, and multiplies -P_i by P_j^T (v_mfma_f32_32x32x2f32) in chunks of
// 64 columns.  Pi and Pj are the workgroup's LDS operand tiles.
constexpr int UP = NB + 2;   // LDS row stride: a lane's (row, k) reads hit 64 distinct banks
__device__ __forceinline__ void update_tile(float* __restrict__ A, int64_t k, int64_t pp, int64_t rest, int kw,
                                            int64_t ti, int64_t tj, float (*__restrict__ Pi)[UP],
                                            float (*__restrict__ Pj)[UP]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* P = A + (pp + kw) * k + pp;
  float* C = A + (pp + kw) * k + pp + kw;
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

// Panel p of the blocked Cholesky factorization (columns p .. p+nb-1 of the
// lower factor).  The first `groups` workgroups form the panel: every one
// factors the nb x nb diagonal block itself (identical arithmetic, so
// identical results) and then solves its own 64 rows of the panel below it:
// L21 = A21 L11^-T.  With PRE, the previous panel (columns p-64 .. p-1)
// has not yet been subtracted from this panel's columns: each of these
// workgroups first applies it to the rows it holds (the diagonal block and
// its own rows: A -= P P_d^T, with P those rows of the previous panel and P_d
// the diagonal block's rows of it).  The other workgroups of the launch apply
// the previous panel to the rest of its super-panel, the 64 x 64 tiles of
// column blocks 1 .. lim-1 right of p (grid (lim-1) x tiles; those above the
// diagonal exit): columns that this launch's panel workgroups do not read.
// Inside a panel workgroup the block is factored in 16-column steps: one wave
// factors and inverts the 16 x 16 diagonal sub-block in registers; then the
// rows below it (the block's own rows and the panel rows) are multiplied by
// the inverse's transpose, and the step's contribution is subtracted from the
// columns to its right, both as 16 x 16 tiles on the matrix cores
// (v_mfma_f32_16x16x4f32, one tile per wave at a time).  Workgroup 0 stores
// L11 into Ld (the same block of the inverse's buffer, which diag_inv_kernel
// later inverts in place): A's diagonal block is read by every panel
// workgroup of the launch, so no workgroup may write it.  On a non-positive
// pivot workgroup 0 also sets *info (once) to the order of the failing
// leading minor of the reversed matrix, i.e. of the failing trailing minor of
// H + lam I.
//
// 16x16x4 operand layout: lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16]; accumulator register r of lane l is D[4 (l / 16) + r][l % 16].
constexpr int SP = NB + 4;   // LDS row stride: the tiles' operand and accumulator accesses are conflict free
template <bool PRE>
__global__ __launch_bounds__(256, 2) void panel_kernel(float* __restrict__ A, float* __restrict__ Ld, int64_t k,
                                                       int64_t p, int32_t* __restrict__ info, int groups) {
  // Rows 0..63: the diagonal block (lower part; -> L11); rows 64..127: this
  // workgroup's panel rows (-> L21 rows).  Ps: the same rows of the previous
  // panel (pre-update), or an extra workgroup's operand tiles.  Matrix
  // b = blockIdx.y of a batch (A, Ld: k^2 floats per matrix; info[b]).
  __shared__ __attribute__((aligned(16))) float V[2 * NB][SP];
  __shared__ __attribute__((aligned(16))) float Ps[PRE ? 2 * NB : 1][SP];
  {
    const int64_t b = blockIdx.y;
    A += b * k * k;
    Ld += b * k * k;
    info += b;
  }
  if (PRE && (int)blockIdx.x >= groups) {
    const int64_t rest = k - p, nt = (rest + NB - 1) / NB, t = (int64_t)blockIdx.x - groups;
    const int64_t tj = 1 + t / nt, ti = t % nt;
    if (ti < tj) return;
    static_assert(2 * NB * UP <= 2 * NB * SP, "operand tiles fit in Ps");
    update_tile(A, k, p - NB, rest, NB, ti, tj, (float (*)[UP]) & Ps[0][0], (float (*)[UP])(&Ps[0][0] + NB * UP));
    return;
  }
  // Inverse of the current 16 x 16 diagonal sub-block (rows of 20: 16-byte
  // aligned; column 16 carries the pivots' scales).
  __shared__ __attribute__((aligned(16))) float Li[16][20];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  const int nb = (int)min((int64_t)NB, k - p);
  const int64_t r0 = (int64_t)blockIdx.x * NB;
  const int rows = (int)max((int64_t)0, min((int64_t)NB, k - p - nb - r0));
  // All loads first (16-byte, clamped to valid rows), then the LDS writes.
  f32x4 ld[8], lp[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int e = tid + 256 * (q & 3), i = e >> 4, j4 = (e & 15) * 4;
    const int64_t row = q < 4 ? p + min(i, nb - 1) : p + nb + r0 + min(i, max(rows - 1, 0));
    // nb is a multiple of 16: a 4-column group lies wholly inside or past it.
    ld[q] = (q < 4 || rows > 0) ? *(const f32x4*)(A + row * k + p + min(j4, nb - 4)) : f32x4{0.f, 0.f, 0.f, 0.f};
    // The previous panel is whole (64 columns) whenever PRE is set.
    if (PRE) lp[q] = (q < 4 || rows > 0) ? *(const f32x4*)(A + row * k + p - NB + j4) : f32x4{0.f, 0.f, 0.f, 0.f};
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
    if (PRE) {
      const bool ok = q < 4 ? i < nb : i < rows;
      *(f32x4*)&Ps[q < 4 ? i : NB + i][j4] = ok ? lp[q] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  __syncthreads();
  // With PRE: V -= Ps Ps[0:64]^T on the diagonal block's lower 16 x 16 tiles
  // (10) and the panel rows' tiles (16), 64 k-values each; a tile's upper part
  // on the diagonal gets values that nothing reads.  Rows and columns past nb
  // or rows hold zeros in Ps, so the identity and zero padding stay.  Wave 0
  // takes tile 0 (the first diagonal sub-block) and factors it at once, while
  // waves 1-3 update the other 25 tiles, two at a time.
  auto pre_tiles = [&]<int NT>(int t0, int t1) {   // NT (1 or 2) tiles: t0 and t1
    int ti[NT], tj[NT];
#pragma unroll
    for (int h = 0; h < NT; ++h) {
      const int t = h ? t1 : t0;
      if (t < 10) {
        ti[h] = t < 1 ? 0 : (t < 3 ? 1 : (t < 6 ? 2 : 3));
        tj[h] = t - ti[h] * (ti[h] + 1) / 2;
      } else {
        ti[h] = 4 + (t - 10) / 4;
        tj[h] = (t - 10) % 4;
      }
    }
    // Lane (l16, lq) supplies k = 16 lq .. 16 lq + 15 (step 4j + u: k = 16 lq
    // + 4j + u), so that its operands are four 16-byte reads per tile side.
    // The accumulators hold -V, so that no operand needs negating.
    f32x4 acc[NT], a4[NT][4], b4[NT][4];
#pragma unroll
    for (int h = 0; h < NT; ++h) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a4[h][j] = *(const f32x4*)&Ps[16 * ti[h] + l16][16 * lq + 4 * j];
        b4[h][j] = *(const f32x4*)&Ps[16 * tj[h] + l16][16 * lq + 4 * j];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[h][r] = -V[16 * ti[h] + 4 * lq + r][16 * tj[h] + l16];
    }
#pragma unroll
    for (int kk = 0; kk < NB / 4; ++kk)
#pragma unroll
      for (int h = 0; h < NT; ++h)
        acc[h] = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[h][kk >> 2][kk & 3], b4[h][kk >> 2][kk & 3], acc[h], 0, 0, 0);
#pragma unroll
    for (int h = 0; h < NT; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) V[16 * ti[h] + 4 * lq + r][16 * tj[h] + l16] = -acc[h][r];
  };
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
  if (wave == 0) {
    if constexpr (PRE) pre_tiles.template operator()<1>(0, 0);
    factor_sub(0);
  } else if constexpr (PRE) {
    // Wave w takes tiles w, w+3, ... (pairs w+6i, w+6i+3; wave 1's last tile, 25, alone).
    for (int t = wave; t + 3 < 26; t += 6) pre_tiles.template operator()<2>(t, t + 3);
    if (wave == 1) pre_tiles.template operator()<1>(25, 25);
  }
  __syncthreads();
  for (int b = 0; b < NB / 16; ++b) {
    const int o = 16 * b;
    // Rows below the sub-block (o+16 .. 127): columns o..o+15 := V Li^T.
    const int nrt = (2 * NB - o - 16) / 16;
    for (int t = wave; t < nrt; t += 4) {
      const int t0 = o + 16 + 16 * t;
      // Lane (l16, lq) supplies k = 4 lq + kk: one 16-byte read per operand.
      const f32x4 av = *(const f32x4*)&V[t0 + l16][o + 4 * lq];
      const f32x4 bv = *(const f32x4*)&Li[l16][4 * lq];
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
      // Lane (l16, lq) supplies k = o + 4 lq + kk; the accumulator holds -V.
      const f32x4 av = *(const f32x4*)&V[t0 + l16][o + 4 * lq];
      const f32x4 bv = *(const f32x4*)&V[j0 + l16][o + 4 * lq];
      f32x4 acc;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = -V[t0 + 4 * lq + r][j0 + l16];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[kk], bv[kk], acc, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) V[t0 + 4 * lq + r][j0 + l16] = -acc[r];
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
    *(f32x4*)((q < 4 ? Ld + (p + i) * k : A + (p + nb + r0 + i) * k) + p + j4) = v;
  }
}

// Inverses of the diagonal 64-blocks of L (one wave each), in place in Linv,
// where the panel launches stored them: lane c solves L x = e_c by forward
// substitution (column c of the inverse), with the block in LDS so that row i
// of L reaches every lane as broadcast reads (the same address in every
// lane), four values at a time.  The block is read whole before it is
// overwritten, and only by its own workgroup.  An even block also zeroes the
// 64 x 64 block right of it: the inverse's products read the upper triangle
// of each 128-aligned diagonal block (as zeros), and nothing else writes that
// part of Linv (the panels write their diagonal blocks' upper triangles as
// zeros).
__global__ __launch_bounds__(64) void diag_inv_kernel(float* __restrict__ Linv, int64_t k) {
  Linv += (int64_t)blockIdx.y * k * k;   // matrix of a batch
  __shared__ __attribute__((aligned(16))) float Ls[NB][NB];
  const int lane = threadIdx.x;
  const int64_t p = (int64_t)blockIdx.x * NB;
  const int nb = (int)min((int64_t)NB, k - p);
  // L's lower part; the identity outside nb.
#pragma unroll 8
  for (int i = 0; i < NB; ++i) {
    float v = (i == lane) ? 1.0f : 0.0f;
    if (i < nb && lane < nb && lane <= i) v = Linv[(p + i) * k + p + lane];
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
  if ((blockIdx.x & 1) == 0 && p + NB + lane < k) {
    for (int i = 0; i < nb; ++i) Linv[(p + i) * k + p + NB + lane] = 0.0f;
  }
}

// U[i][j] = Linv[k-1-i][k-1-j] for j >= i, 0 below the diagonal.
// Four columns j .. j+3 per thread, 16-byte loads and stores (k % 4 == 0).
// Matrix b = blockIdx.z: Linv + b * k^2 -> U + b * stride_u.
__global__ void flip_out_kernel(const float* __restrict__ Linv, int64_t k, float* __restrict__ U, int64_t stride_u) {
  const int64_t i = blockIdx.y, j = 4 * ((int64_t)blockIdx.x * blockDim.x + threadIdx.x);
  if (j >= k) return;
  Linv += (int64_t)blockIdx.z * k * k;
  U += (int64_t)blockIdx.z * stride_u;
  f32x4 v = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (j + 3 >= i) {
    const f32x4 l = *(const f32x4*)(Linv + (k - 1 - i) * k + (k - 4 - j));
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = j + u >= i ? l[3 - u] : 0.0f;
  }
  *(f32x4*)(U + i * k + j) = v;
}

// The Cholesky factor itself, for the sweep's form without the inverse:
// L = chol(J H_d J) is stored by the panel launches with its diagonal 64-blocks
// in Ld and the rest of its lower part in A; R = J L J is upper triangular
// with H_d = R R^T (R = U^-1).  V[i][j] = -R[i][j] / R[j][j] above the
// diagonal, V[i][i] = R[i][i], 0 below.  Four columns j .. j+3 per thread
// (they lie in one 64-block of L: k % 4 == 0), 16-byte loads and stores.
// Matrix b = blockIdx.z: A + b * k^2, Ld + b * k^2 -> V + b * stride_v.
// dv[c] = L[c][c] (from the diagonal blocks in Ld) for each matrix z of the
// pass (dv + z * stride_d), so that chol_out_kernel reads the pivots as
// contiguous vectors instead of one strided element per output.
__global__ void diag_vec_kernel(const float* __restrict__ Ld, int64_t k, float* __restrict__ dv, int64_t stride_d) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= k) return;
  dv[(int64_t)blockIdx.y * stride_d + c] = Ld[(int64_t)blockIdx.y * k * k + c * k + c];
}

__global__ void chol_out_kernel(const float* __restrict__ A, const float* __restrict__ Ld, int64_t k,
                                float* __restrict__ V, int64_t stride_v, const float* __restrict__ dv,
                                int64_t stride_d) {
  const int64_t i = blockIdx.y, j = 4 * ((int64_t)blockIdx.x * blockDim.x + threadIdx.x);
  if (j >= k) return;
  A += (int64_t)blockIdx.z * k * k;
  Ld += (int64_t)blockIdx.z * k * k;
  V += (int64_t)blockIdx.z * stride_v;
  dv += (int64_t)blockIdx.z * stride_d;
  f32x4 v = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (j + 3 >= i) {
    const int64_t r = k - 1 - i, c0 = k - 4 - j;   // L[r][c0 + 3 - u] = R[i][j + u]
    const float* src = r / NB == c0 / NB ? Ld : A;
    const f32x4 l = *(const f32x4*)(src + r * k + c0);
    const f32x4 dd = *(const f32x4*)(dv + c0);   // dd[3 - u] = L[d][d], d = k - 1 - (j + u)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t jj = j + u;
      if (jj == i) {
        v[u] = l[3 - u];
      } else if (jj > i) {
        v[u] = -l[3 - u] / dd[3 - u];
      }
    }
  }
  *(f32x4*)(V + i * k + j) = v;
}

}  // namespace

size_t factor_workspace(int64_t k) {
  // per matrix: A (k^2), Linv (k^2), T (k^2 / 2), lam (64 floats)
  return ((size_t)k * k * 2 + (size_t)k * k / 2 + 64) * sizeof(float);
}

int64_t factor_max_chunk(int64_t k) {
  // grid.z of the batched GEMMs: (pairs of 64-blocks, at most k / 128) x matrices <= 65535
  const int64_t pairs = k / 128 > 0 ? k / 128 : 1;
  return 65535 / pairs > 0 ? 65535 / pairs : 1;
}

// A second stream per device for the trailing updates that run beside the
// panel chain (default priority, non-blocking, created on first use).
static hipError_t helper_stream(hipStream_t* out) {
  static std::mutex mu;
  static hipStream_t hs[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!hs[dev]) {
    e = hipStreamCreateWithFlags(&hs[dev], hipStreamNonBlocking);
    if (e != hipSuccess) return e;
  }
  *out = hs[dev];
  return hipSuccess;
}

// nb matrices of one pass: the workspace holds `chunk` per-matrix buffers in
// four regions (A: chunk x k^2, Linv: chunk x k^2, T: chunk x k^2 / 2, lam),
// so a matrix's buffers sit at the same offsets whatever nb is.
static hipError_t factor_pass(const float* H, int64_t k, int64_t nb, int64_t stride_h, float damp_rel, float* U,
                              int64_t stride_u, float* lambda_out, int32_t* info, float* ws, int64_t chunk,
                              bool chol, hipStream_t s) {
  const size_t kk = (size_t)k * k;
  float* A = ws;
  float* Linv = A + chunk * kk;
  float* T = Linv + chunk * kk;
  float* lam = T + chunk * kk / 2;
  const unsigned nbu = (unsigned)nb;

  hipLaunchKernelGGL(damping_kernel, dim3(nbu), dim3(256), 0, s, H, k, stride_h, damp_rel, lam, lambda_out, info);
  hipLaunchKernelGGL(flip_damp_kernel, dim3((unsigned)((k / 4 + 255) / 256), (unsigned)k, nbu), dim3(256), 0, s, H,
                     k, stride_h, lam, A, info);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  // Panels are grouped in super-panels of SW columns.  Each panel's update of
  // the rest of its super-panel (the columns the next panels factor) runs in
  // the next panel's launch: its panel workgroups apply it to the columns they
  // factor, extra workgroups to the columns right of them.  The columns right
  // of the super-panel take all of its panels in one update after its last
  // panel, so they are read and written once per SW columns instead of once
  // per panel.  Above 8 super-panels that update is split: the next
  // super-panel's columns on the main stream (the next panels need them), the
  // columns right of those on a second stream, where it runs beside the next
  // super-panel's panels (which use a fraction of the device).  The next split
  // update waits for it, and so does everything after the last panel.  (At k
  // = 14336 a factor took 17.2 instead of 18.4 ms; at k = 4096 1.69 instead of
  // 1.60, where the narrow first part underfills the device.)  Every launch
  // covers the nb matrices of the pass (grid.y).
  hipStream_t s2 = nullptr;
  hipEvent_t ev_panels = nullptr, ev_rest = nullptr;
  bool rest_pending = false;
  auto release = [&]() {
    if (ev_panels) (void)hipEventDestroy(ev_panels);
    if (ev_rest) (void)hipEventDestroy(ev_rest);
  };
  if (k > 8 * SW) {
    e = helper_stream(&s2);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ev_panels, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ev_rest, hipEventDisableTiming);
    if (e != hipSuccess) {
      release();
      return e;
    }
  }
  for (int64_t p = 0; p < k; p += NB) {
    const int64_t rest = k - p - NB;
    const int64_t groups = rest > 0 ? (rest + NB - 1) / NB : 1;
    const int64_t s0 = p / SW * SW, send = min(s0 + SW, k);
    const bool pre = p > s0;
    int64_t extra = 0;
    if (pre) {
      const int64_t nt = (k - p + NB - 1) / NB, lim = (send - p + NB - 1) / NB;
      extra = (lim - 1) * nt;
    }
    if (pre)
      hipLaunchKernelGGL(panel_kernel<true>, dim3((unsigned)(groups + extra), nbu), dim3(256), 0, s, A, Linv, k, p,
                         info, (int)groups);
    else
      hipLaunchKernelGGL(panel_kernel<false>, dim3((unsigned)groups, nbu), dim3(256), 0, s, A, Linv, k, p, info,
                         (int)groups);
    if (rest <= 0) break;
    if (p + NB == send && send < k) {
      // C -= P P^T over the super-panel's columns: P = its rows below it
      // (rest2 x SW), C the trailing matrix (lower tiles).  First the next
      // super-panel's na columns (rest2 x na), then the square right of them.
      const int64_t rest2 = k - send, na = min((int64_t)SW, rest2);
      auto update = [&](int64_t r0, int64_t c0, int64_t M, int64_t N, hipStream_t st) {
        GemmArgs g{};
        g.A = A + r0 * k + s0; g.lda = k;
        g.B = A + c0 * k + s0; g.ldb = k;
        g.C = A + r0 * k + c0; g.ldc = k;
        g.M = M; g.N = N; g.K = send - s0;
        g.batch = (int)nb; g.sA = (int64_t)kk; g.sB = (int64_t)kk; g.sC = (int64_t)kk;
        g.alpha = -1.0f; g.beta = 1.0f; g.kmode = kGemmKFull;
        return gemm_f32(g, false, true, true, kEpiAxpby, st);
      };
      if (rest_pending) e = hipStreamWaitEvent(s, ev_rest, 0);
      if (e == hipSuccess && rest2 > na && s2) {
        e = hipEventRecord(ev_panels, s);
        if (e == hipSuccess) e = hipStreamWaitEvent(s2, ev_panels, 0);
        if (e == hipSuccess) e = update(send + na, send + na, rest2 - na, rest2 - na, s2);
        if (e == hipSuccess) e = hipEventRecord(ev_rest, s2);
        rest_pending = true;
        if (e == hipSuccess) e = update(send, send, rest2, na, s);
      } else if (e == hipSuccess) {
        e = update(send, send, rest2, rest2, s);
      }
      if (e != hipSuccess) {
        release();
        return e;
      }
    }
  }
  if (rest_pending) e = hipStreamWaitEvent(s, ev_rest, 0);
  release();
  if (e != hipSuccess) return e;
  if (chol) {   // the factor itself (scaled as the sweep takes it), no inverse; T holds the pivots
    hipLaunchKernelGGL(diag_vec_kernel, dim3((unsigned)((k + 255) / 256), nbu), dim3(256), 0, s, Linv, k, T,
                       (int64_t)(kk / 2));
    hipLaunchKernelGGL(chol_out_kernel, dim3((unsigned)((k / 4 + 255) / 256), (unsigned)k, nbu), dim3(256), 0, s, A,
                       Linv, k, U, stride_u, T, (int64_t)(kk / 2));
    return hipGetLastError();
  }
  hipLaunchKernelGGL(diag_inv_kernel, dim3((unsigned)((k + NB - 1) / NB), nbu), dim3(64), 0, s, Linv, k);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  // Triangular inverse by recursive doubling over diagonal blocks of size bs;
  // the GEMMs of a level run over (pairs of one matrix) x (nb matrices).  At
  // the levels whose tiles of one matrix do not fill the device, every
  // tile's triangular k range is split in two halves (the second half's
  // product into T2, added afterwards): the long tiles of those levels hold
  // twice the average work, so the halves even the launch out.  The choice
  // counts one matrix's tiles, so a matrix gets the same bits in any batch.
  for (int64_t bs = NB; bs < k; bs *= 2) {
    int64_t full = k / (2 * bs);  // pairs whose both halves are complete
    auto pair_step = [&](int64_t base, int64_t n1, int64_t n2, int pairs) -> hipError_t {
      const int64_t tiles = (int64_t)pairs * ((n1 + 127) / 128) * ((n2 + 127) / 128);
      const bool split = bs >= 1024 && tiles <= 256;
      float* T2 = T + (int64_t)kk / 4;   // pairs * n1 * n2 <= k bs / 2 <= k^2 / 4 floats per matrix
      // T = L21 * L11^-1   (n2 x n1)
      GemmArgs a{};
      a.A = A + (base + bs) * k + base; a.lda = k;
      a.B = Linv + base * k + base; a.ldb = k;
      a.C = T; a.ldc = n1;
      a.M = n2; a.N = n1; a.K = n1; a.batch = pairs * (int)nb; a.bi = pairs;
      a.sA = 2 * bs * k + 2 * bs; a.sB = 2 * bs * k + 2 * bs; a.sC = n1 * n2;
      a.sA2 = (int64_t)kk; a.sB2 = (int64_t)kk; a.sC2 = (int64_t)kk / 2;
      a.alpha = 1.0f; a.beta = 0.0f; a.kmode = kGemmKLowerB;   // L11^-1 is lower triangular
      if (split) { a.ksplit = 2; a.C2 = T2; a.ldc2 = n1; a.s2C = n1 * n2; a.s2C2 = (int64_t)kk / 2; }
      hipError_t err = gemm_f32(a, false, false, false, kEpiAxpby, s);
      if (err == hipSuccess && split)
        err = add_into(T, n1, T2, n1, (int64_t)pairs * n2, n1, s, nb, (int64_t)kk / 2, (int64_t)kk / 2);
      if (err != hipSuccess) return err;
      // X21 = -L22^-1 * T   (n2 x n1), written into Linv
      GemmArgs b{};
      b.A = Linv + (base + bs) * k + (base + bs); b.lda = k;
      b.B = T; b.ldb = n1;
      b.C = Linv + (base + bs) * k + base; b.ldc = k;
      b.M = n2; b.N = n1; b.K = n2; b.batch = pairs * (int)nb; b.bi = pairs;
      b.sA = 2 * bs * k + 2 * bs; b.sB = n1 * n2; b.sC = 2 * bs * k + 2 * bs;
      b.sA2 = (int64_t)kk; b.sB2 = (int64_t)kk / 2; b.sC2 = (int64_t)kk;
      b.alpha = -1.0f; b.beta = 0.0f; b.kmode = kGemmKLowerA;  // L22^-1 is lower triangular
      // With the split, the second half goes to T2 as [pair][n2][n1] (T itself
      // stays intact: it is this product's B operand), then into X21.
      if (split) { b.ksplit = 2; b.C2 = T2; b.ldc2 = n1; b.s2C = n1 * n2; b.s2C2 = (int64_t)kk / 2; }
      err = gemm_f32(b, false, false, false, kEpiAxpby, s);
      if (err != hipSuccess || !split) return err;
      if (nb == 1)   // the pairs as one batch
        return add_into(Linv + (base + bs) * k + base, k, T2, n1, n2, n1, s, pairs, 2 * bs * k + 2 * bs, n1 * n2);
      for (int q = 0; err == hipSuccess && q < pairs; ++q)
        err = add_into(Linv + (base + bs + q * 2 * bs) * k + base + q * 2 * bs, k, T2 + q * n1 * n2, n1, n2, n1, s, nb,
                       (int64_t)kk, (int64_t)kk / 2);
      return err;
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
  hipLaunchKernelGGL(flip_out_kernel, dim3((unsigned)((k / 4 + 255) / 256), (unsigned)k, nbu), dim3(256), 0, s,
                     Linv, k, U, stride_u);
  return hipGetLastError();
}

hipError_t factor_hinv_launch(const float* H, int64_t k, int64_t batch, int64_t stride_h, float damp_rel, float* U,
                              int64_t stride_u, float* lambda_out, int32_t* info, void* ws, int64_t chunk,
                              hipStream_t s, bool chol) {
  if (chunk < 1) chunk = 1;
  chunk = min(chunk, factor_max_chunk(k));
  for (int64_t b0 = 0; b0 < batch; b0 += chunk) {
    const int64_t nb = min(chunk, batch - b0);
    hipError_t e = factor_pass(H + b0 * stride_h, k, nb, stride_h, damp_rel, U + b0 * stride_u, stride_u,
                               lambda_out + b0, info + b0, (float*)ws, chunk, chol, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace nvq
