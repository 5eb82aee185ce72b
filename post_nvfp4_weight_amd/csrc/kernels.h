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
  int batch;
  float alpha, beta;
  int kmode;            // GemmK: which part of the k range each output tile needs
  int64_t noff;         // column of C (and of B) 0 within the whole matrix, for kmode's triangle
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
// C -= A B with A [M x K] and C [M x N] fp64, B [K x N] fp32 (all row-major).
hipError_t rank_update_f64(const double* A, int64_t lda, const float* B, int64_t ldb, double* C, int64_t ldc,
                           int64_t M, int64_t N, int64_t K, hipStream_t s);

// ---- Hessian -------------------------------------------------------------
size_t syrk_bf16_workspace(int64_t n, int64_t k);
hipError_t syrk_bf16(const uint16_t* X, int64_t n, int64_t k, int64_t ldx, float* H, void* ws,
                     hipStream_t s);
hipError_t symmetrize_from_upper(float* H, int64_t k, hipStream_t s);
// out[t] = row clamp(idx[t], 0, nsrc-1) of X (rows of k elements of esize bytes, ld ldx).
hipError_t gather_rows(const void* X, int esize, int64_t ldx, const int32_t* idx, int64_t nsrc, int64_t n,
                       int64_t k, void* out, hipStream_t s);

// ---- factor ----------------------------------------------------------------
size_t factor_workspace(int64_t k);
hipError_t factor_hinv_launch(const float* H, int64_t k, float damp_rel, float* U,
                              float* lambda_out, int32_t* info, void* ws, hipStream_t s);

// ---- codec / sweep -----------------------------------------------------------
hipError_t global_scale_launch(const void* W, int bf16, int64_t m, int64_t k, int64_t ldw,
                               float* g, float* partial, int nparts, hipStream_t s);
int global_scale_parts(int64_t m, int64_t k);
hipError_t dequant_launch(const uint8_t* codes, const uint8_t* scales, const float* g,
                          int64_t m, int64_t k, void* out, int out_bf16, hipStream_t s);
hipError_t rtn_launch(const void* W, int bf16, int64_t m, int64_t k, int64_t ldw,
                      const float* g, int n_cand, uint8_t* codes, uint8_t* scales,
                      float* row_loss, hipStream_t s);
hipError_t load_working_copy(const void* W, int bf16, int64_t m, int64_t k, int64_t ldw,
                             float* Wp, hipStream_t s);
hipError_t inv_diag_launch(const float* U, int64_t k, float* invd, hipStream_t s);
// indep: choose each block's scale by the block-independent squared rounding
// error instead of the replay score (the committed block is still replayed).
hipError_t sweep_batch_launch(float* Wp, const float* U, const float* invd, const float* g,
                              int64_t m, int64_t k, int i1, int ncols, int n_cand, bool indep,
                              uint8_t* codes, uint8_t* scales, float* Eslab, int64_t lde, float* row_loss,
                              hipStream_t s);
// The same sweep with fp64 working weights and errors (U read as fp32).
hipError_t sweep_batch_launch_f64(double* Wp, const float* U, const float* g, int64_t m, int64_t k, int i1,
                                  int ncols, int n_cand, bool indep, uint8_t* codes, uint8_t* scales, double* Eslab,
                                  int64_t lde, float* row_loss, hipStream_t s);
hipError_t load_working_copy_f64(const void* W, int bf16, int64_t m, int64_t k, int64_t ldw, double* Wp,
                                 hipStream_t s);
// Columns of the two-level lazy update: each 128-column batch updates the
// rest of its 512-column block; each finished block updates every later
// column with its whole error slab (m x 512).
constexpr int kSuperBatch = 512;
hipError_t delta_w_launch(const void* W, int bf16, int64_t m, int64_t k, int64_t ldw,
                          const uint8_t* codes, const uint8_t* scales, const float* g,
                          float* dW, hipStream_t s, int64_t c0 = 0, int64_t c1 = -1);
hipError_t row_sum_launch(const float* P, int64_t m, int64_t nparts, float* out, hipStream_t s);
hipError_t fill_f32(float* p, int64_t n, float v, hipStream_t s);

// NVFP4 weight-only GEMM: Y [T x m] = g (X Q^T), X bf16 [T x k] (row stride ldx),
// Q = e2m1 * e4m3 from codes [m x k/2] and scales [m x k/16]; Y fp32 or bf16 (row stride ldy).
// Small token counts split k over workspace partials (nvfp4_gemm_workspace bytes, 0 if unsplit).
size_t nvfp4_gemm_workspace(int64_t T, int64_t k, int64_t m);
hipError_t nvfp4_gemm_launch(const uint16_t* X, int64_t T, int64_t k, int64_t ldx, const uint8_t* codes,
                             const uint8_t* scales, const float* g, int64_t m, void* Y, int out_bf16, int64_t ldy,
                             float* ws, hipStream_t s);

}  // namespace nvq
