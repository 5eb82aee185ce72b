/*
 * nvq.h -- C ABI of the NVFP4 GPTQ / Schur Replay weight quantizer for AMD
 * Instinct MI355X (gfx950).
 *
 * Method: "Replay the Curvature: Accurate and Scalable NVFP4 Quantization for
 * Large Language Model Inference" (arXiv 2609.36654), Abstract.  Given a
 * linear layer's weights W [m x k] (m output rows, k input columns) and
 * calibration activations X [n x k], the library returns NVFP4 weights --
 * E2M1 element codes with one E4M3 scale per 16 consecutive weights of a row
 * -- chosen by a GPTQ column sweep in which each block's scale is selected by
 * Schur Replay, plus the layer's weighted reconstruction error.
 *
 * Conventions shared by every call:
 *   - Matrices are row-major; leading dimensions (ld*) count elements.
 *   - Pointers named as device pointers must be device memory of the current
 *     HIP device; "stream" is a hipStream_t passed as void* (NULL = default
 *     stream).  Every compute call is asynchronous on that stream: it only
 *     enqueues kernels, never allocates, frees or synchronizes, and keeps no
 *     pointer after returning.  Buffers must stay valid until the stream has
 *     run the work.
 *   - Callers own every buffer, including workspaces sized by the matching
 *     *_workspace_size query.  Workspaces must be 256-byte aligned.
 *   - Return value: NVQ_OK (0) on success, a negative NVQ_ERR_* code when the
 *     arguments are rejected on the host (nothing is enqueued then), or
 *     NVQ_ERR_HIP when the HIP runtime reports a launch error.  The reason of
 *     the last failure on the calling thread is given by nvq_last_error().
 *   - Calls on different streams may run concurrently when their output and
 *     workspace buffers do not overlap.
 *   - A call may run part of its work on an internal stream of the library
 *     (one per device, default priority; factor_hinv and factor_chol above
 *     k = 4096): that
 *     work starts after the work enqueued on "stream" before the call, and
 *     the work enqueued on "stream" after the call waits for it (HIP events),
 *     so the call is ordered on "stream" as if it ran there alone, also under
 *     stream capture.
 */
#ifndef NVQ_H
#define NVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------- */
#define NVQ_OK                 0
#define NVQ_ERR_NULL          -1  /* a required pointer is NULL                 */
#define NVQ_ERR_SHAPE         -2  /* a size or leading dimension is invalid     */
#define NVQ_ERR_DTYPE         -3  /* unsupported dtype code                     */
#define NVQ_ERR_NCAND         -4  /* candidate count outside [1, 16]            */
#define NVQ_ERR_WORKSPACE     -5  /* workspace too small or misaligned          */
#define NVQ_ERR_VALUE         -6  /* a scalar argument is out of range          */
#define NVQ_ERR_HIP           -7  /* the HIP runtime reported an error          */
#define NVQ_ERR_ALIGN         -8  /* a pointer is not aligned as required       */

/* ---- element types of W, X and dequantized outputs ------------------------ */
#define NVQ_DTYPE_F32  0
#define NVQ_DTYPE_BF16 1

/* ---- flags of gptq_nvfp4_quantize ------------------------------------------ */
/* Round to nearest without GPTQ updates: U is not read; each block's scale is
 * the candidate with the least plain squared error (the absmax scale when
 * n_cand = 1). */
#define NVQ_FLAG_RTN    1u
/* Do not compute the weighted error (row_err is not written; H may be NULL). */
#define NVQ_FLAG_NO_ERR 2u
/* fp64 working precision for the sweep: working weights, errors, scores and
 * the lazy updates are fp64 (U and H are read as fp32 inputs; the weighted
 * error is computed as without the flag).  Needs a larger workspace
 * (gptq_nvfp4_workspace_size with the same flags).  Ignored with RTN.
 * When to set it.  GPTQ's column coupling carries every flipped near-tie
 * decision along its row, so the working precision decides how many
 * decisions differ from the exact computation.  Measured against an fp64
 * computation:
 *   - layers fed by zero-mean activations (attention projections, MLP gate
 *     and up projections) stay well inside 0.1% in fp32 (about 2e-5 of
 *     codes and scales over a whole 4096 x 4096 layer): leave the flag off;
 *   - layers fed by activations with a large common mean or heavy tails
 *     (MLP down projections over gated activations; sparse non-negative
 *     inputs), whose Hessians span about 8 orders of magnitude, move 0.1% to
 *     0.7% of the decisions in fp32: set the flag (the lazy updates then run
 *     on the fp64 matrix cores, whose dense peak is half the fp32 one).
 * The library cannot inspect H's range without synchronizing, so the caller
 * chooses per layer. */
#define NVQ_FLAG_FP64   4u
/* Block-independent scale selection, the baseline that Schur Replay corrects
 * ("Replay the Curvature", Abstract: scoring blocks independently can
 * misestimate their final error): each candidate is scored by the plain
 * squared rounding error sum_j (w'_j - q_j)^2 of the block's weights at the
 * block start, every element rounded on its own with no in-block updates; the
 * least score wins (ties: the smaller scale) and that candidate's block is
 * committed with its replayed GPTQ updates as usual.  For the scale-selection
 * ablation; ignored with RTN. */
#define NVQ_FLAG_INDEP  8u
/* Reject non-finite input instead of quantizing it: a NaN or infinity in W,
 * or a g that is not a finite positive number, has no NVFP4 encoding
 * ("Replay the Curvature", Abstract: E2M1 codes under an E4M3 scale).  Every row of W that holds a non-finite value among its
 * first k columns -- every row, if *g is not finite and positive -- is
 * written as: codes 0, all of its scale bytes 0x7F (the E4M3FN NaN code, so
 * that nvfp4_dequantize gives NaN for the row), row_err and row_loss NaN.
 * Other rows are unaffected (rows are independent throughout the sweep).
 * The check reads W once more on the device and never synchronizes: the
 * caller finds the rejected rows by reading row_err (or the scales) back.
 * Without the flag a non-finite weight still gives deterministic outputs
 * (NaN scores lose every arg-min), but they mean nothing. */
#define NVQ_FLAG_CHECK_FINITE 16u
/* The U argument is the V that factor_chol writes (the Cholesky factor R of
 * H + lambda I = R R^T, scaled) instead of the U that factor_hinv writes
 * (U = R^-1).  The sweep is the same GPTQ computation ("Replay the
 * Curvature", Abstract: quantizing one column updates those that follow)
 * taken in the factor's own form: a committed column j propagates its raw
 * error w_j - q_j (against its input value) through V_jl = -R_jl / R_ll, the
 * later columns receive w'_l = w_l + sum_{j<l} (w_j - q_j) R_jl / R_ll,
 * and the score term of column j is ((w'_j - q_j) R_jj)^2.  With exact
 * arithmetic these are the updates and scores of the inverse form, term by
 * term (e_j U_jl = (w_j - q_j) R_jl / R_ll summed over j); in fp32 they
 * differ by rounding.  The candidate window, decisions, codes, scales,
 * row_loss and row_err are defined as without the flag.  Needs a larger
 * workspace (gptq_nvfp4_workspace_size with the same flags: one more copy of
 * W in the working precision).  Ignored with RTN. */
#define NVQ_FLAG_CHOL_FACTOR 32u

/*
 * hessian_accumulate -- second-order state of the layer ("Replay the
 * Curvature", Abstract: the second-order state of GPTQ), H += X^T X.
 *
 *   X      device, [n x ldx] row-major, element type x_dtype (NVQ_DTYPE_BF16
 *          or NVQ_DTYPE_F32); only the first k columns are used.  Rows must
 *          start 16-byte aligned: X itself 16-byte aligned and ldx % 8 == 0
 *          for bf16, ldx % 4 == 0 for fp32.
 *   n      number of tokens (rows of X), n >= 0; n = 0 leaves H unchanged.
 *   k      number of input channels, k > 0, k % 16 == 0.
 *   H      device, fp32 [k x k] row-major.  On entry only the upper triangle
 *          (j >= i) is read; on return H holds the full symmetric matrix
 *          (old upper triangle + X^T X, mirrored into the lower triangle).
 *          Products of bf16 inputs are exact in fp32; sums are fp32 in a
 *          fixed order, so results are bitwise reproducible.
 *   ws     device workspace of hessian_workspace_size(n, k, x_dtype) bytes.
 * Streaming: calling it on consecutive token chunks accumulates into H, so
 * calibration data can arrive in pieces (the caller tracks the token count).
 */
size_t hessian_workspace_size(int64_t n, int64_t k, int x_dtype);
int hessian_accumulate(const void* X, int x_dtype, int64_t n, int64_t k, int64_t ldx,
                       float* H, void* ws, size_t ws_bytes, void* stream);

/*
 * hessian_accumulate_host -- the same H += X^T X with X resident in host
 * memory ("Replay the Curvature", Abstract: calibration activations are
 * tiered across device, host and disk, and only the active layer is kept on
 * the device).  X is streamed to the device in chunks of `chunk` tokens
 * through two device buffers: chunk i+1 is copied (on copy_stream) while
 * chunk i is accumulated (on stream), ordered by events.  The result equals
 * calling hessian_accumulate on the chunks in order.
 *
 *   X_host   host [n x ldx], element type x_dtype: pinned (hipHostMalloc) or
 *            pageable (e.g. a memory-mapped file).  Without staging it must
 *            stay valid until copy_stream's work is done; pageable memory is
 *            then copied synchronously by the runtime.
 *   n, k     tokens and channels; n >= 0, k > 0, k % 16 == 0; ldx >= k.
 *   H        device fp32 [k x k], accumulated in place.
 *   chunk    tokens per chunk, > 0.
 *   ws       device workspace of hessian_host_workspace_size(chunk, k, x_dtype)
 *            bytes (two chunk buffers and the Hessian workspace), 256-aligned.
 *   staging  NULL, or pinned host memory of hessian_host_staging_size(chunk,
 *            k, x_dtype) bytes: pageable chunks are then copied into it by
 *            host threads and sent asynchronously; the call returns once the
 *            staging buffers have been read (the accumulation itself is still
 *            asynchronous on stream).
 *   stream, copy_stream  compute and copy streams (default priority); a NULL
 *            copy_stream means stream (no overlap).
 * The device memory used is H plus two chunks plus the Hessian workspace,
 * whatever n is.
 */
size_t hessian_host_workspace_size(int64_t chunk, int64_t k, int x_dtype);
size_t hessian_host_staging_size(int64_t chunk, int64_t k, int x_dtype);
int hessian_accumulate_host(const void* X_host, int x_dtype, int64_t n, int64_t k, int64_t ldx, float* H,
                            int64_t chunk, void* ws, size_t ws_bytes, void* staging, size_t staging_bytes,
                            void* stream, void* copy_stream);

/*
 * hessian_accumulate_grouped -- one Hessian per group of token rows, for a
 * mixture-of-experts layer in which every expert is a linear layer of its own
 * that sees only the tokens routed to it ("Replay the Curvature", Abstract:
 * the second-order state of each layer's GPTQ solve; its MoE evaluation model
 * routes each token to a few experts).  For every group e:
 *   H[e] += X[tok_idx[j]]^T X[tok_idx[j]] summed over j in [grp_off[e], grp_off[e+1]).
 *
 *   X        device [n x ldx], element type x_dtype, as for hessian_accumulate
 *            (16-byte aligned; ldx % 8 == 0 for bf16, % 4 for fp32).
 *   n        number of token rows of X.
 *   tok_idx  device int32 [grp_off[G]]: the token row of every assignment,
 *            grouped by expert.  Values outside [0, n) are clamped into it
 *            (no out-of-bounds read); the caller guarantees they lie inside.
 *   grp_off  HOST int64 [G + 1]: grp_off[0] = 0, non-decreasing; group e owns
 *            entries grp_off[e] .. grp_off[e+1]-1 of tok_idx (empty groups are
 *            skipped).  Read during the call only.
 *   G        number of groups, G > 0.
 *   H        device fp32 [G][k][k]; each H[e] as in hessian_accumulate (upper
 *            triangle read, full symmetric matrix written).
 *   ws       device workspace of hessian_grouped_workspace_size(grp_off, G, k,
 *            x_dtype) bytes: a gathered-row buffer (the largest group's rows,
 *            and for bf16 X with k = 4096 at least the smaller groups' rows up
 *            to 2 GiB) plus the Hessian workspace for the largest group.
 * Groups of at least 16384 rows, and every group unless X is bf16 and k is
 * 4096, are gathered and accumulated one at a time, in order, on the stream.
 * With bf16 X and k = 4096 the smaller groups are gathered one after another
 * into the row buffer and accumulated together, up to 128 groups per launch
 * (each H[e] entry then sums its group's rows in one fixed order, so results
 * are bitwise reproducible; they may differ in rounding from a
 * hessian_accumulate call on the same rows, within the same fp32 bound).
 */
size_t hessian_grouped_workspace_size(const int64_t* grp_off, int64_t G, int64_t k, int x_dtype);
int hessian_accumulate_grouped(const void* X, int x_dtype, int64_t n, int64_t k, int64_t ldx, const int32_t* tok_idx,
                               const int64_t* grp_off, int64_t G, float* H, void* ws, size_t ws_bytes, void* stream);

/*
 * factor_hinv -- damped inverse factor used by the GPTQ sweep ("Replay the
 * Curvature", Abstract: GPTQ, in which quantizing one column updates those
 * that follow).
 *
 *   lambda = damp_rel * mean(diag H); U is the upper-triangular matrix with
 *   positive diagonal such that (H + lambda I)^-1 = U^T U.
 *
 *   H          device fp32 [k x k], symmetric (only the upper triangle is read).
 *   k          k > 0, k % 16 == 0.
 *   damp_rel   relative damping, >= 0 and finite (0.01 is the usual value).
 *   U          device fp32 [k x k] output; entries below the diagonal are set
 *              to 0.  U must not overlap H.
 *   lambda_out device, 1 float: lambda.
 *   info       device, 1 int32: 0 on success; j > 0 if the trailing principal
 *              submatrix of H + lambda I of order j is not positive definite;
 *              -1 if the upper triangle of H or lambda holds a NaN or an
 *              infinity (U then holds no meaningful values).
 *   ws         device workspace of factor_hinv_workspace_size(k) bytes.
 * Computed in fp32: a blocked Cholesky factorization of the index-reversed
 * damped matrix followed by a blocked triangular inverse.
 */
size_t factor_hinv_workspace_size(int64_t k);
int factor_hinv(const float* H, int64_t k, float damp_rel, float* U, float* lambda_out,
                int32_t* info, void* ws, size_t ws_bytes, void* stream);

/*
 * factor_chol -- the damped Cholesky factor in the form the sweep takes with
 * NVQ_FLAG_CHOL_FACTOR, without the triangular inverse that factor_hinv
 * forms ("Replay the Curvature", Abstract: GPTQ, in which quantizing one
 * column updates those that follow).
 *
 *   lambda = damp_rel * mean(diag H) as in factor_hinv; R is the
 *   upper-triangular matrix with positive diagonal such that
 *   H + lambda I = R R^T (so R = U^-1 for factor_hinv's U).
 *   V          device fp32 [k x k] output: V[i][j] = -R[i][j] / R[j][j] for
 *              j > i, V[i][i] = R[i][i], 0 below the diagonal.  V must not
 *              overlap H.
 *   H, k, damp_rel, lambda_out, info: as for factor_hinv (info > 0 names the
 *              order of the trailing principal submatrix that is not positive
 *              definite; V then holds no meaningful values).
 *   ws         device workspace of factor_chol_workspace_size(k) bytes.
 * Computed in fp32 by the same blocked Cholesky factorization of the
 * index-reversed damped matrix as factor_hinv (R = J L J for L = chol(J (H +
 * lambda I) J), J the index reversal); the same internal stream above k =
 * 4096.
 */
size_t factor_chol_workspace_size(int64_t k);
int factor_chol(const float* H, int64_t k, float damp_rel, float* V, float* lambda_out, int32_t* info, void* ws,
                size_t ws_bytes, void* stream);

/*
 * factor_hinv_batched -- factor_hinv of `batch` matrices (one per expert of a
 * mixture-of-experts layer): H + e*stride_h -> U + e*stride_u,
 * lambda_out[e], info[e].  Strides count floats, are >= k*k and multiples of
 * 4; the U and H ranges must not overlap.
 *   ws  at least factor_hinv_workspace_size(k) bytes; a workspace of
 *       c * factor_hinv_workspace_size(k) bytes lets one pass factor c
 *       matrices together: every launch of the blocked factorization (panel,
 *       trailing update, inverse) covers all matrices of the pass, so the
 *       serial chain of panels is walked once per pass instead of once per
 *       matrix.  Results do not depend on c.
 * batch = 0 is a no-op; nothing is enqueued when an argument is rejected.
 */
int factor_hinv_batched(const float* H, int64_t k, int64_t batch, int64_t stride_h, float damp_rel, float* U,
                        int64_t stride_u, float* lambda_out, int32_t* info, void* ws, size_t ws_bytes,
                        void* stream);

/*
 * factor_chol_batched -- factor_chol of `batch` matrices (one per expert of a
 * mixture-of-experts layer; "Replay the Curvature", Abstract: GPTQ, in which
 * quantizing one column updates those that follow): H + e*stride_h ->
 * V + e*stride_v, lambda_out[e], info[e], each as factor_chol gives it.
 * Strides count floats, are >= k*k and multiples of 4; the V and H ranges
 * must not overlap.
 *   ws  at least factor_chol_workspace_size(k) bytes; c times that lets one
 *       pass factor c matrices together (every launch covers all matrices of
 *       the pass).  Results do not depend on c: each matrix gets the bits
 *       factor_chol gives it alone.
 * batch = 0 is a no-op; nothing is enqueued when an argument is rejected.
 */
int factor_chol_batched(const float* H, int64_t k, int64_t batch, int64_t stride_h, float damp_rel, float* V,
                        int64_t stride_v, float* lambda_out, int32_t* info, void* ws, size_t ws_bytes,
                        void* stream);

/*
 * nvfp4_global_scale -- per-tensor fp32 scale applied on top of the E4M3 block
 * scales: g = fl32(max|W| / 2688) (2688 = 6 * 448, the largest E2M1 magnitude
 * times the largest finite E4M3 value), or g = 1 when W is all zero.
 *
 *   W      device [m x ldw], element type w_dtype; m, k > 0, ldw >= k.
 *   g_out  device, 1 float.
 *   ws     device workspace of nvfp4_global_scale_workspace_size(m, k) bytes.
 */
size_t nvfp4_global_scale_workspace_size(int64_t m, int64_t k);
int nvfp4_global_scale(const void* W, int w_dtype, int64_t m, int64_t k, int64_t ldw,
                       float* g_out, void* ws, size_t ws_bytes, void* stream);

/*
 * gptq_nvfp4_quantize -- NVFP4 quantization of W by a GPTQ column sweep with
 * Schur Replay block-scale selection ("Replay the Curvature", Abstract: each
 * 16-weight block's E4M3 scale is chosen by reproducing the GPTQ updates it
 * causes inside the block and scoring the block error left after compensation
 * from the still-unquantized columns).
 *
 * For each row and each 16-column block (natural column order):
 *   a  = max |w'| over the block's current (updated) weights;
 *   the candidates are the n_cand consecutive E4M3 codes centred on the code
 *   nearest to a / (6 g), [c0 - n_cand/2, c0 + ceil(n_cand/2) - 1], shifted to
 *   lie in [1, 126]; an all-zero block gets scale code 0 and +0 elements;
 *   each candidate c is replayed: column by column, q_j = nearest E2M1 value
 *   of w'_j under scale dec(c) * g (ties to even, clipped at 6),
 *   e_j = (w'_j - q_j) / U_jj, later columns l of the block get
 *   w'_l -= e_j U_jl; its score is sum_j e_j^2;
 *   the least score wins (ties: the smaller scale); its codes are stored and
 *   its errors update every later column of the row: w'_l -= sum_j e_j U_jl.
 * Later columns receive the updates lazily: the errors of each 128-column
 * batch update the rest of its 512-column block at once, and the columns past
 * a finished 512-column block receive that block's errors together (fp32
 * MFMA GEMMs; the same sums as eager updates in another order); all working
 * values are fp32 (fp64 with NVQ_FLAG_FP64).
 *
 *   W        device [m x ldw], element type w_dtype (bf16 or fp32); not
 *            modified.  m > 0, k > 0, k % 16 == 0, ldw >= k, ldw % 4 == 0.
 *   U        device fp32 [k x k] from factor_hinv, or from factor_chol with
 *            NVQ_FLAG_CHOL_FACTOR (read unless NVQ_FLAG_RTN).
 *   H        device fp32 [k x k] symmetric (the undamped Hessian), read only
 *            for the weighted error; may be NULL with NVQ_FLAG_NO_ERR.
 *   g        device, 1 float: the per-tensor scale (e.g. nvfp4_global_scale).
 *   n_cand   candidates per block, 1 <= n_cand <= 16.
 *   codes    device uint8 [m x k/2] output: two E2M1 codes per byte, the even
 *            column in the low nibble; code = sign << 3 | magnitude index
 *            (magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6); zero is always +0.
 *   scales   device uint8 [m x k/16] output: E4M3 (FN) block-scale codes.
 *   row_err  device fp32 [m] output: E_r = dW_r H dW_r^T with
 *            dW = W - dequantized W (not written with NVQ_FLAG_NO_ERR).
 *   row_loss device fp32 [m] output or NULL: sum of the committed e_j^2 of
 *            the row (the damped loss that the sweep minimizes); 0 for RTN.
 *   ws       device workspace of gptq_nvfp4_workspace_size(m, k, flags) bytes.
 */
size_t gptq_nvfp4_workspace_size(int64_t m, int64_t k, unsigned flags);
int gptq_nvfp4_quantize(const void* W, int w_dtype, int64_t m, int64_t k, int64_t ldw,
                        const float* U, const float* H, const float* g, int n_cand,
                        unsigned flags, uint8_t* codes, uint8_t* scales, float* row_err,
                        float* row_loss, void* ws, size_t ws_bytes, void* stream);

/*
 * gptq_nvfp4_quantize_batched -- gptq_nvfp4_quantize of `batch` weight
 * matrices of equal shape (the experts of a mixture-of-experts layer), one
 * after the other on the stream.  Element e reads W + e*stride_w (elements of
 * w_dtype), U + e*stride_u, H + e*stride_h (floats; U and H are not read when
 * the flags say so) and g[e], and writes codes + e*m*(k/2),
 * scales + e*m*(k/16), row_err + e*m and row_loss + e*m.  Strides: stride_w
 * >= m*ldw; stride_u and stride_h >= k*k and multiples of 4.
 *   ws  at least gptq_nvfp4_workspace_size(m, k, flags) bytes; a workspace
 *       of c times that size quantizes c matrices per pass, every launch
 *       (sweep batches, lazy updates, weighted error) covering all of them.
 *       Results do not depend on c.
 * batch = 0 is a no-op; arguments are checked as for gptq_nvfp4_quantize.
 */
int gptq_nvfp4_quantize_batched(const void* W, int w_dtype, int64_t batch, int64_t m, int64_t k, int64_t ldw,
                                int64_t stride_w, const float* U, int64_t stride_u, const float* H,
                                int64_t stride_h, const float* g, int n_cand, unsigned flags, uint8_t* codes,
                                uint8_t* scales, float* row_err, float* row_loss, void* ws, size_t ws_bytes,
                                void* stream);

/*
 * nvfp4_dequantize -- NVFP4 weights back to real values ("Replay the
 * Curvature", Abstract: E2M1 elements sharing an E4M3 block scale):
 * out = fl32(e2m1(code) * e4m3(scale) * g), one rounding of the exact product;
 * for bf16 output that fp32 value is rounded to nearest-even bf16.
 *
 *   codes   device uint8 [m x k/2], layout as produced by gptq_nvfp4_quantize.
 *   scales  device uint8 [m x k/16].
 *   g       device, 1 float.
 *   out     device [m x k] of out_dtype (NVQ_DTYPE_F32 or NVQ_DTYPE_BF16).
 *   m >= 0, k > 0, k % 16 == 0.
 */
int nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* g, int64_t m,
                     int64_t k, void* out, int out_dtype, void* stream);

/*
 * nvfp4_gemm -- a consumer of the exported weights ("Replay the Curvature",
 * Abstract: the quantized layer is exported in NVFP4 for use): the
 * weight-only product Y = X dequant(W)^T with bf16 activations.
 * Computed as Y = g (X Q^T) with Q = e2m1 * e4m3 exact in bf16, on the bf16
 * matrix cores with fp32 accumulation (within 2^-24 per product of
 * X fl32(Q g)^T).
 *
 *   X       device bf16 [T x ldx]; T >= 0, k > 0, k % 16 == 0, ldx >= k,
 *           ldx % 8 == 0; 16-byte aligned.
 *   codes, scales, g   the layer as written by gptq_nvfp4_quantize: codes
 *           [m x k/2] (8-byte aligned), scales [m x k/16], g 1 float (device).
 *   Y       device [T x ldy] of y_dtype (fp32 or bf16, RNE), ldy >= m.
 *   ws      device workspace of nvfp4_gemm_workspace_size(T, k, m) bytes
 *           (256-aligned; may be NULL when that is 0): for few tokens k is
 *           split over workgroups and the fp32 partial sums are added in
 *           split order, so results do not depend on timing.  (With at most
 *           32 tokens, k % 128 == 0 and codes 16-byte aligned, one workgroup
 *           sums all of k for 16 output channels and the workspace is not
 *           touched.)
 */
size_t nvfp4_gemm_workspace_size(int64_t T, int64_t k, int64_t m);
int nvfp4_gemm(const void* X, int x_dtype, int64_t T, int64_t k, int64_t ldx, const uint8_t* codes,
               const uint8_t* scales, const float* g, int64_t m, void* Y, int y_dtype, int64_t ldy, void* ws,
               size_t ws_bytes, void* stream);

/*
 * nvfp4_gemm_noalloc -- nvfp4_gemm for callers that cannot allocate memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation, kernels and results, bit for bit, with
 * no workspace argument.  Its k-split partial sums use a fixed array of
 * 32 MiB (33554432 bytes) of device memory inside the library, one per device
 * that runs the call, held until the process ends (its address is looked up
 * on the first call on each device).
 *
 *   Arguments as for nvfp4_gemm, without ws.  Shapes whose
 *   nvfp4_gemm_workspace_size(T, k, m) exceeds 33554432 bytes are rejected
 *   with NVQ_ERR_WORKSPACE (nothing is enqueued).  The call allocates and
 *   frees nothing.
 *   Every call on one device shares that device's array, which keeps the last
 *   call's contents: calls that overlap on one device (concurrent streams,
 *   host threads) race and must be serialized by the caller.  Nothing in the
 *   array needs to start at zero: each call writes every partial sum it reads.
 */
int nvfp4_gemm_noalloc(const void* X, int x_dtype, int64_t T, int64_t k, int64_t ldx, const uint8_t* codes,
                       const uint8_t* scales, const float* g, int64_t m, void* Y, int y_dtype, int64_t ldy,
                       void* stream);

/*
 * nvq_check_finite -- device-side scan for NaN and infinity, for the inputs
 * the quantizer cannot represent (W) or that would poison the second-order
 * state (X, before hessian_accumulate; "Replay the Curvature", Abstract:
 * the calibration activations and weights of the layer solve).
 *
 *   A       device [rows x ld], element type dtype (bf16 or fp32); only the
 *           first cols values of each row are read.
 *   rows    0 <= rows < 2^31 - 1; cols > 0; ld >= cols.
 *   status  device, 1 int32 output: 0 if every value is finite, otherwise
 *           1 + the lowest row index holding a NaN or infinity.  The value
 *           does not depend on timing.  Written asynchronously; the library
 *           does not read it back.
 * A NaN in X makes H non-finite, which factor_hinv reports as info = -1.
 */
int nvq_check_finite(const void* A, int dtype, int64_t rows, int64_t cols, int64_t ld, int32_t* status,
                     void* stream);

/* Text of a status code; never NULL. */
const char* nvq_status_string(int status);
/* Reason of the most recent failing call on this thread ("" if none). */
const char* nvq_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* NVQ_H */
