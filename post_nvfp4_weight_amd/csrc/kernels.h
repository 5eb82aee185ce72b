// Internal launchers (host side) of the gfx950 kernels.  Every launcher
// enqueues on `s` and returns the hipGetLastError() of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nvq {

// ---- fp32 MFMA GEMM: C = (alpha * op(A)) op(B) + beta * C --------------------
// (alpha scales the A operand before the product: exact when alpha = +-1.)
enum GemmEpi { kEpiAxpby = 0, kEpiRowDot = 1 };

struct GemmArgs {
  const float* A; const float* B; float* C;
  const float* D;       // row-dot epilogue: the matrix multiplied into op(A)op(B)
  float* P;             // row-dot epilogue: partial sums [M x ldp]
  int64_t M, N, K;
  int64_t lda, ldb, ldc, ldd, ldp;
  int64_t sA, sB, sC;   // batch strides (elements)
  int batch;            // grid.z: batch items (inner x outer when bi > 1)
  // Two-level batch (e.g. pairs of blocks within each of several matrices):
  // with bi > 0, item z is inner z % bi and outer z / bi, and the outer
  // strides sA2.. are added per outer index (bi = 0: one level).  sD, sP (and sD2, sP2) move the
  // row-dot epilogue's D and P the same way.
  int bi;
  int64_t sA2, sB2, sC2;
  int64_t sD, sP, sD2, sP2;
  float alpha, beta;
  int kmode;            // GemmK: which part of the k range each output tile needs
  int64_t noff;         // column of C (and of B) 0 within the whole matrix, for kmode's triangle
  // ksplit 2 (split-bf16 kernel, beta = 0): every tile's k range is cut in two
  // halves of whole 32-chunks, the first half's product written to C, the
  // second's to C2 (row stride ldc2, batch strides s2C, s2C2 like sC, sC2);
  // the caller adds C2 into C.  This evens out tiles whose triangular k
  // ranges differ in length.
  int ksplit;
  float* C2;
  int64_t ldc2, s2C, s2C2;
};
// kmode: kGemmKFull; kGemmKLowerA (A lower triangular: row tile i needs
// k < its last row); kGemmKLowerB (B lower triangular: column tile j needs
// k >= its first column); kGemmKSymUpperB (B symmetric, used as its upper
// triangle with the off-diagonal entries doubled: column tile j needs
// k < its last column; for x^T B x = x^T B' x with B' = 2 triu(B, 1) + diag(B)).
enum GemmK { kGemmKFull = 0, kGemmKLowerA = 1, kGemmKLowerB = 2, kGemmKSymUpperB = 3 };
// trans_a: A is stored [K x M]; trans_b: B is stored [N x K].  lower: skip
// 128x128 tiles that lie entirely above the diagonal (square C only).
// Requires M, N, K, leading dimensions and offsets to be multiples of 4 and
// 16-byte aligned matrix starts.
hipError_t gemm_f32(const GemmArgs& a, bool trans_a, bool trans_b, bool lower, GemmEpi epi,
                    hipStream_t s);
constexpr int kGemmTile = 128;
// C[i][j] += C2[i][j] for i < M, j < N (row strides ldc, ldc2); nb matrices at C + e sC, C2 + e sC2.
hipError_t add_into(float* C, int64_t ldc, const float* C2, int64_t ldc2, int64_t M, int64_t N, hipStream_t s,
                    int64_t nb = 1, int64_t sC = 0, int64_t sC2 = 0);
// C -= A B with A [M x K] and C [M x N] fp64, B [K x N] fp32 (all row-major).
// nb matrices: item e at A + e * sA, B + e * sB, C + e * sC.
hipError_t rank_update_f64(const double* A, int64_t lda, const float* B, int64_t ldb, double* C, int64_t ldc,
                           int64_t M, int64_t N, int64_t K, hipStream_t s, int64_t nb = 1, int64_t sA = 0,
                           int64_t sB = 0, int64_t sC = 0);

// ---- Hessian -------------------------------------------------------------
size_t syrk_bf16_workspace(int64_t n, int64_t k);
hipError_t syrk_bf16(const uint16_t* X, int64_t n, int64_t k, int64_t ldx, float* H, void* ws,
                     hipStream_t s);
hipError_t symmetrize_from_upper(float* H, int64_t k, hipStream_t s);
// Grouped Hessians of small experts at k = 4096 (see syrk_k4_grouped_kernel):
// expert j of a group has cnt[j] gathered bf16 rows (ld k) from row beg[j] and
// adds into H + hexp[j] * k * k (upper triangle, then mirrored into the lower
// one).  syrk_bf16_grouped fills nx and xe itself.
constexpr int K4G_EXP = 128, K4G_PER_XCD = 32;
struct K4Grouped {
  int32_t beg[K4G_EXP], cnt[K4G_EXP], hexp[K4G_EXP];
  uint8_t nx[8], xe[8][K4G_PER_XCD];
};
bool syrk_k4_grouped_applies(int64_t k);
hipError_t syrk_bf16_grouped(const uint16_t* rows, int64_t k, K4Grouped& g, int nexp, float* H, hipStream_t s);
// out[t] = row clamp(idx[t], 0, nsrc-1) of X (rows of k elements of esize bytes, ld ldx).
hipError_t gather_rows(const void* X, int esize, int64_t ldx, const int32_t* idx, int64_t nsrc, int64_t n,
                       int64_t k, void* out, hipStream_t s);

// ---- factor ----------------------------------------------------------------
// Workspace of one matrix; a workspace of c such sizes factors c matrices per pass.
size_t factor_workspace(int64_t k);
// The largest number of matrices one pass takes (a grid-size limit).
int64_t factor_max_chunk(int64_t k);
// batch matrices H + b * stride_h -> U + b * stride_u, lambda_out[b], info[b],
// `chunk` matrices per pass (ws holds chunk per-matrix workspaces).  With
// chol, the output is V (the Cholesky factor R of H_d = R R^T with its
// strictly upper part scaled to -R_ij / R_jj and R_ii on the diagonal)
// instead of U = R^-1: no triangular inverse is formed.
hipError_t factor_hinv_launch(const float* H, int64_t k, int64_t batch, int64_t stride_h, float damp_rel, float* U,
                              int64_t stride_u, float* lambda_out, int32_t* info, void* ws, int64_t chunk,
                              hipStream_t s, bool chol = false);

// ---- codec / sweep -----------------------------------------------------------
// Batched launches (nb matrices, grid.y = matrix e) take per-matrix strides:
// W in elements of its dtype; g, codes, scales, row_err and row_loss advance
// by 1, m*k/2, m*k/16, m and m per matrix.
struct SweepStrides {
  int64_t wp = 0;     // working weights (elements of the working type)
  int64_t u = 0;      // U (floats)
  int64_t invd = 0;   // 1 / U_jj (floats)
  int64_t e = 0;      // error slab (elements of the working type)
  int64_t mb = 0;     // Cholesky-factor form: the diagonal blocks' M - I (floats)
};
hipError_t global_scale_launch(const void* W, int bf16, int64_t m, int64_t k, int64_t ldw,
                               float* g, float* partial, int nparts, hipStream_t s);
int global_scale_parts(int64_t m, int64_t k);
hipError_t dequant_launch(const uint8_t* codes, const uint8_t* scales, const float* g,
                          int64_t m, int64_t k, void* out, int out_bf16, hipStream_t s);
hipError_t rtn_launch(const void* W, int bf16, int64_t m, int64_t k, int64_t ldw,
                      const float* g, int n_cand, uint8_t* codes, uint8_t* scales,
                      float* row_loss, hipStream_t s, int64_t nb = 1, int64_t stride_w = 0);
hipError_t load_working_copy(const void* W, int bf16, int64_t m, int64_t k, int64_t ldw,
                             float* Wp, hipStream_t s, int64_t nb = 1, int64_t stride_w = 0, int64_t stride_wp = 0);
// invd[j] = 1 / U_jj, or U_jj itself with copy (the Cholesky-factor form).
hipError_t inv_diag_launch(const float* U, int64_t k, float* invd, hipStream_t s, int64_t nb = 1,
                           int64_t stride_u = 0, int64_t stride_invd = 0, bool copy = false);
// indep: choose each block's scale by the block-independent squared rounding
// error instead of the replay score (the committed block is still replayed).
// pre (a multiple of 128, with sweep_applies_inblock(n_cand)): the batch's
// columns have not yet received the errors of the pre columns before it in
// its 512-column block, which the error slab holds just before Eslab; the
// launch applies them to its rows first.  Otherwise pre must be 0.
// W0 (non-null): the Cholesky-factor form.  U then holds V (-R_ij / R_jj
// above the diagonal of the factor R of H_d = R R^T, R_jj on it), invd
// holds R_jj, W0 the input weights in the working layout (as Wp before any
// update) and Mb the blocks' M - I (chol_block_m_launch, stride bs.mb); a
// committed column propagates w0_j - q_j and scores ((w'_j - q_j) R_jj)^2.
hipError_t sweep_batch_launch(float* Wp, const float* U, const float* invd, const float* g,
                              int64_t m, int64_t k, int i1, int ncols, int n_cand, bool indep,
                              uint8_t* codes, uint8_t* scales, float* Eslab, int64_t lde, float* row_loss,
                              hipStream_t s, int64_t nb = 1, const SweepStrides& bs = SweepStrides(), int pre = 0,
                              const float* W0 = nullptr, const float* Mb = nullptr);
bool sweep_applies_inblock(int n_cand);
// The same sweep with fp64 working weights and errors (U read as fp32).
hipError_t sweep_batch_launch_f64(double* Wp, const float* U, const float* g, int64_t m, int64_t k, int i1,
                                  int ncols, int n_cand, bool indep, uint8_t* codes, uint8_t* scales, double* Eslab,
                                  int64_t lde, float* row_loss, hipStream_t s, int64_t nb = 1,
                                  const SweepStrides& bs = SweepStrides(), const double* W0 = nullptr,
                                  const float* Mb = nullptr);
// Cholesky-factor form: for each diagonal 16x16 block of V, Mb[16 j + i] (j
// the block's column, i < j) = (M - I)_ij with M = (I - N)^-1 and N the
// block's strictly upper part (0 for i >= j); k * 16 floats per matrix.
hipError_t chol_block_m_launch(const float* V, int64_t k, float* Mb, hipStream_t s, int64_t nb = 1,
                               int64_t stride_v = 0, int64_t stride_m = 0);
hipError_t load_working_copy_f64(const void* W, int bf16, int64_t m, int64_t k, int64_t ldw, double* Wp,
                                 hipStream_t s, int64_t nb = 1, int64_t stride_w = 0, int64_t stride_wp = 0);
// Columns of the two-level lazy update: each 128-column batch updates the
// rest of its 512-column block; each finished block updates every later
// column with its whole error slab (m x 512).
constexpr int kSuperBatch = 512;
hipError_t delta_w_launch(const void* W, int bf16, int64_t m, int64_t k, int64_t ldw,
                          const uint8_t* codes, const uint8_t* scales, const float* g,
                          float* dW, hipStream_t s, int64_t c0 = 0, int64_t c1 = -1, int64_t nb = 1,
                          int64_t stride_w = 0, int64_t stride_dw = 0);
hipError_t row_sum_launch(const float* P, int64_t m, int64_t nparts, float* out, hipStream_t s, int64_t nb = 1,
                          int64_t stride_p = 0);
hipError_t fill_f32(float* p, int64_t n, float v, hipStream_t s);
// *status = 0 if every A[r][c] (r < rows, c < cols; bf16 or fp32, row stride
// ld) is finite, else 1 + the lowest row holding a non-finite value.
hipError_t nonfinite_scan_launch(const void* A, int bf16, int64_t rows, int64_t cols, int64_t ld, int32_t* status,
                                 hipStream_t s);
// Rejects the rows of W holding a non-finite value (all rows if g is not a
// finite positive number): codes 0, scales 0x7F, row_err and row_loss NaN.
hipError_t reject_nonfinite_rows_launch(const void* W, int bf16, int64_t m, int64_t k, int64_t ldw, const float* g,
                                        uint8_t* codes, uint8_t* scales, float* row_err, float* row_loss,
                                        hipStream_t s, int64_t nb = 1, int64_t stride_w = 0);


// NVFP4 weight-only GEMM: Y [T x m] = g (X Q^T), X bf16 [T x k] (row stride ldx),
// Q = e2m1 * e4m3 from codes [m x k/2] and scales [m x k/16]; Y fp32 or bf16 (row stride ldy).
// Small token counts split k over workspace partials (nvfp4_gemm_workspace bytes, 0 if unsplit).
size_t nvfp4_gemm_workspace(int64_t T, int64_t k, int64_t m);
// The no-allocation variant: its split partial sums use a fixed device array
// of kNoAllocScratchBytes per device; noalloc_scratch gives this device's
// address of it (looked up once per device).
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
hipError_t noalloc_scratch(float** out);
hipError_t nvfp4_gemm_launch(const uint16_t* X, int64_t T, int64_t k, int64_t ldx, const uint8_t* codes,
                             const uint8_t* scales, const float* g, int64_t m, void* Y, int out_bf16, int64_t ldy,
                             float* ws, hipStream_t s);

}  // namespace nvq
