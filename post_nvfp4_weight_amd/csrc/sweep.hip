// GPTQ column sweep with Schur Replay block-scale selection, and the NVFP4
// streaming kernels (global scale, round-to-nearest encode, dequantization).
//
// Sweep mapping.  Output rows are independent; inside a row the 16-column
// blocks are processed in order.  One lane per (row, candidate): a row's G
// candidate lanes (G = next power of two >= n_cand) replay the block in
// registers, each with its own scale, reduce their scores with DPP lane
// permutations (ties to the lower candidate), and the winner publishes its
// codes, scale and errors.  A workgroup owns ROWS rows of one 128-column lazy
// batch: the rows' batch slab, the transposed 128x128 diagonal block of U, its
// eight 16x16 diagonal blocks and 1/U_jj live in LDS (the in-block factor
// entries are read as wave-wide broadcasts), and after each block the row's G
// lanes update the later columns of the batch.  Columns beyond the batch are
// updated by fp32 MFMA products with the error slab: with G >= 8 the batch's
// own rows first take the errors of the earlier batches of their 512-column
// block inside the sweep launch (one 16 x 128 product per workgroup), else a
// GEMM after each batch updates the rest of the block.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace nvq {

namespace {

template <int BF16>
__device__ __forceinline__ float load_w(const void* W, int64_t idx) {
  if (BF16) return bf16_bits_to_f32(((const uint16_t*)W)[idx]);
  return ((const float*)W)[idx];
}

// ---- global scale --------------------------------------------------------------
// Rows are dealt to the workgroups in turn and each row's columns to the
// threads; with vec (W 16-byte aligned, ldw and k multiples of 8 values) a
// thread reads 8 consecutive values at a time.
template <int BF16>
__global__ __launch_bounds__(256) void amax_kernel(const void* __restrict__ W, int64_t m, int64_t k,
                                                   int64_t ldw, float* __restrict__ partial, bool vec) {
  __shared__ float red[256];
  float a = 0.0f;
  for (int64_t r = blockIdx.x; r < m; r += gridDim.x) {
    if (vec) {
      for (int64_t c = (int64_t)threadIdx.x * 8; c < k; c += 256 * 8) {
        if (BF16) {
          const u32x4 u = *(const u32x4*)((const uint16_t*)W + r * ldw + c);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            a = fmaxf(a, fmaxf(fabsf(__uint_as_float(u[q] << 16)), fabsf(__uint_as_float(u[q] & 0xFFFF0000u))));
        } else {
          const f32x4* src = (const f32x4*)((const float*)W + r * ldw + c);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const f32x4 u = src[h];
#pragma unroll
            for (int q = 0; q < 4; ++q) a = fmaxf(a, fabsf(u[q]));
          }
        }
      }
    } else {
      for (int64_t c = threadIdx.x; c < k; c += 256) a = fmaxf(a, fabsf(load_w<BF16>(W, r * ldw + c)));
    }
  }
  red[threadIdx.x] = a;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  if (threadIdx.x == 0) partial[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(256) void gscale_finish_kernel(const float* __restrict__ partial, int nparts,
                                                            float* __restrict__ g) {
  __shared__ float red[256];
  float a = 0.0f;
  for (int i = threadIdx.x; i < nparts; i += 256) a = fmaxf(a, partial[i]);
  red[threadIdx.x] = a;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    float amax = red[0];
    // fl32(amax / 2688): the fp64 quotient rounded to fp32 is the correctly
    // rounded fp32 quotient (no fp32 midpoint lies within fp64 rounding of it).
    *g = amax > 0.0f ? (float)((double)amax / 2688.0) : 1.0f;
  }
}

// ---- dequantization ---------------------------------------------------------------
// The codes [m][k/2], scales [m][k/16] and output [m][k] are dense, so they are
// one stream of half blocks (8 weights: 4 bytes of codes, half a scale byte,
// 16 bytes of bf16 or 32 of fp32 output).  A grid of a few workgroups per CU
// strides over the stream; consecutive lanes take consecutive half blocks, so
// a wave's loads and stores are contiguous, and a thread issues the loads of
// DQ_U half blocks before any of their stores.
constexpr int DQ_U = 4;
template <int OUT_BF16>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales,
                                                      const float* __restrict__ gptr, int64_t nhalf,
                                                      void* __restrict__ out) {
  const float g = *gptr;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t h0 = (int64_t)blockIdx.x * 256 + threadIdx.x; h0 < nhalf; h0 += DQ_U * stride) {
    uint32_t c[DQ_U];
    uint32_t sc[DQ_U];
#pragma unroll
    for (int u = 0; u < DQ_U; ++u) {
      const int64_t hb = min(h0 + u * stride, nhalf - 1);   // clamped: every load is valid
      c[u] = *(const uint32_t*)(codes + hb * 4);
      sc[u] = scales[hb >> 1];
    }
#pragma unroll
    for (int u = 0; u < DQ_U; ++u) {
      const int64_t hb = h0 + u * stride;
      if (hb >= nhalf) break;
      // 0x7F / 0xFF is E4M3FN's NaN (the code of a row rejected by the finite check).
      const float s = (sc[u] & 0x7F) == 0x7F ? __builtin_nanf("") : e4m3_value(sc[u] & 0x7F);
      const bool neg_scale = sc[u] & 0x80;
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = e2m1_dequant((int)((c[u] >> (4 * j)) & 0xF), s, g);
        v[j] = neg_scale ? -x : x;
      }
      if (OUT_BF16) {
        u32x4 o;
#pragma unroll
        for (int w = 0; w < 4; ++w)
          o[w] = (uint32_t)f32_to_bf16_bits(v[2 * w]) | ((uint32_t)f32_to_bf16_bits(v[2 * w + 1]) << 16);
        *(u32x4*)((uint16_t*)out + hb * 8) = o;
      } else {
        f32x4* dst = (f32x4*)((float*)out + hb * 8);
        dst[0] = f32x4{v[0], v[1], v[2], v[3]};
        dst[1] = f32x4{v[4], v[5], v[6], v[7]};
      }
    }
  }
}

// ---- round to nearest (no GPTQ updates) ------------------------------------------
// One thread per (row, block) at a time, striding over the blocks of the
// matrix (codes and scales are dense, so block b's codes are at 8 b and its
// scale at b; W's block is at row * ldw + 16 * column block).  Candidate scores
// are sum_j (w_j - q_j)^2 with separately rounded products and sums in column
// order; with one candidate (the absmax scale) there is nothing to compare,
// and no score is formed.
// vec: every block starts 16-byte aligned (W aligned, ldw a multiple of 8
// bf16 or 4 fp32 values), so it is read with 16-byte loads.
template <int BF16>
__global__ __launch_bounds__(256) void rtn_kernel(const void* __restrict__ W, int64_t m, int64_t k, int64_t ldw,
                                                  const float* __restrict__ gptr, int n_cand,
                                                  uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                  bool vec, int64_t stride_w) {
  const int64_t nbk = k / kBlock, nblk = m * nbk;
  {   // matrix e = blockIdx.y of a batch: W + e * stride_w elements, g[e], its codes and scales
    const int64_t e = blockIdx.y;
    W = (const char*)W + e * stride_w * (BF16 ? 2 : 4);
    gptr += e;
    codes += e * m * (k / 2);
    scales += e * nblk;
  }
  const float g = *gptr;
  const float r6g = 1.0f / (6.0f * g);
  // The one-test E2M1 index needs 2 / (s g) finite for every scale s >= 2^-9.
  const bool nearest = g >= kNearestMinG;
  const float rg = 1.0f / g;
  const bool dense = ldw == k;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < nblk; b += stride) {
    const int64_t base = dense ? b * 16 : (b / nbk) * ldw + (b % nbk) * 16;
    float w[16];
    if (vec) {
      if (BF16) {
        const u32x4* src = (const u32x4*)((const uint16_t*)W + base);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 u = src[h];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            w[8 * h + 2 * q] = __uint_as_float(u[q] << 16);
            w[8 * h + 2 * q + 1] = __uint_as_float(u[q] & 0xFFFF0000u);
          }
        }
      } else {
        const f32x4* src = (const f32x4*)((const float*)W + base);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 u = src[q];
#pragma unroll
          for (int t = 0; t < 4; ++t) w[4 * q + t] = u[t];
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) w[j] = load_w<BF16>(W, base + j);
    }
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) a = fmaxf(a, fabsf(w[j]));
    int best_c = 0;
    uint32_t best_lo = 0, best_hi = 0;
    if (a > 0.0f) {
      const int lo = candidate_lo(e4m3_code_of_ratio_any(a, g, r6g), n_cand);
      if (n_cand == 1 && nearest) {
        // Magnitude indices and sign bits gather into the two code words
        // separately; a sign is kept where its nibble's index is non-zero
        // (zero is always +0).
        const float s = e4m3_value_sel(lo);
        const float r2 = 2.0f * __builtin_amdgcn_rcpf(s) * rg, s8 = 0.125f * s;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float* x = &w[8 * h];
          uint32_t mag = 0;
#pragma unroll
          for (int j = 0; j < 8; ++j)
            mag |= (uint32_t)e2m1_index_nearest(fabsf(x[j]), fabsf(x[j]) * r2, g, s8) << (4 * j);
          // Code byte q holds elements 2q (bits 0-3) and 2q+1 (bits 4-7): byte
          // permutes gather byte 3 (the sign's byte) of the odd elements into
          // bytes 0-3 (sign at bit 7) and of the even ones (shifted to bit 3).
          auto b3 = [&](int a, int c) {   // byte 3 of x[a] and x[c] into bytes 0, 1 | of x[a+4], x[c+4] into 2, 3
            return __builtin_amdgcn_perm(__float_as_uint(x[c]), __float_as_uint(x[a]), 0x0C0C0703u) |
                   __builtin_amdgcn_perm(__float_as_uint(x[c + 4]), __float_as_uint(x[a + 4]), 0x07030C0Cu);
          };
          const uint32_t sgn = (b3(1, 3) & 0x80808080u) | ((b3(0, 2) >> 4) & 0x08080808u);
          const uint32_t nz = mag | (mag >> 1) | (mag >> 2);   // bit 4j: nibble j is non-zero
          (h ? best_hi : best_lo) = mag | (sgn & (nz << 3));
        }
        best_c = lo;
      } else if (n_cand == 1) {
        const float s = e4m3_value_sel(lo);
        const float ts[7] = {0.25f * s, 0.75f * s, 1.25f * s, 1.75f * s, 2.5f * s, 3.5f * s, 5.0f * s};
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int idx = e2m1_index_search(fabsf(w[j]), g, ts);
          const int code = idx | (int)(((__float_as_uint(w[j]) >> 31) & (uint32_t)(idx != 0)) << 3);
          if (j < 8) best_lo |= (uint32_t)code << (4 * j); else best_hi |= (uint32_t)code << (4 * (j - 8));
        }
        best_c = lo;
      } else {
        float best = __builtin_inff();
        for (int ci = 0; ci < n_cand; ++ci) {
          const int c = lo + ci;
          const float s = e4m3_value_sel(c);
          const float hs = 0.5f * s;
          const float ts[7] = {0.25f * s, 0.75f * s, 1.25f * s, 1.75f * s, 2.5f * s, 3.5f * s, 5.0f * s};
          float score = 0.0f;
          uint32_t plo = 0, phi = 0;
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            // e2m1_encode and e2m1_dequant's values, with the sign set by bit operations
            const int idx = e2m1_index_search(fabsf(w[j]), g, ts);
            const int code = idx | (int)(((__float_as_uint(w[j]) >> 31) & (uint32_t)(idx != 0)) << 3);
            const float dq =
                __uint_as_float(__float_as_uint(e2m1_twice_mag(idx) * hs * g) | ((uint32_t)(code & 8) << 28));
            float e = __fsub_rn(w[j], dq);
            score = __fadd_rn(score, __fmul_rn(e, e));
            if (j < 8) plo |= (uint32_t)code << (4 * j); else phi |= (uint32_t)code << (4 * (j - 8));
          }
          if (score < best) { best = score; best_c = c; best_lo = plo; best_hi = phi; }
        }
      }
    }
    *(u32x2*)(codes + b * 8) = u32x2{best_lo, best_hi};
    scales[b] = (uint8_t)best_c;
  }
}

// ---- finite checks ------------------------------------------------------------------
// Whether row r of A (cols values of type bf16 or fp32, row stride ld) holds a
// non-finite value (exponent field all ones), decided by the whole workgroup.
// vec: rows start 16-byte aligned and hold a multiple of 16 bytes.
template <int BF16>
__device__ __forceinline__ bool row_nonfinite(const void* __restrict__ A, int64_t r, int64_t cols, int64_t ld,
                                              bool vec) {
  uint32_t bad = 0;
  if (vec) {
    const int64_t nv = cols * (BF16 ? 2 : 4) / 16;
    const u32x4* row = (const u32x4*)((const char*)A + r * ld * (BF16 ? 2 : 4));
    for (int64_t v = threadIdx.x; v < nv; v += blockDim.x) {
      const u32x4 u = row[v];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (BF16) bad |= ((u[q] & 0x7F80u) == 0x7F80u) | ((u[q] & 0x7F800000u) == 0x7F800000u);
        else bad |= (u[q] & 0x7F800000u) == 0x7F800000u;
      }
    }
  } else {
    for (int64_t c = threadIdx.x; c < cols; c += blockDim.x) {
      if (BF16) bad |= (((const uint16_t*)A)[r * ld + c] & 0x7F80u) == 0x7F80u;
      else bad |= (__float_as_uint(((const float*)A)[r * ld + c]) & 0x7F800000u) == 0x7F800000u;
    }
  }
  return __syncthreads_or((int)bad) != 0;
}

__global__ void status_init_kernel(int32_t* __restrict__ status) { *status = 0x7FFFFFFF; }
__global__ void status_finish_kernel(int32_t* __restrict__ status) {
  const int32_t v = *status;
  *status = v == 0x7FFFFFFF ? 0 : v + 1;
}
// *status = min(*status, the first row holding a non-finite value); a
// workgroup visits its rows in increasing order, so it stops at its first.
template <int BF16>
__global__ __launch_bounds__(256) void nonfinite_scan_kernel(const void* __restrict__ A, int64_t rows, int64_t cols,
                                                             int64_t ld, bool vec, int32_t* __restrict__ status) {
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    if (row_nonfinite<BF16>(A, r, cols, ld, vec)) {
      if (threadIdx.x == 0) atomicMin(status, (int32_t)r);
      return;
    }
  }
}

// Rows of W that hold a non-finite value, or every row if g is not a finite
// positive number, are rejected: codes 0, scales 0x7F (E4M3FN's NaN), and NaN
// row_err / row_loss.  Runs after everything else has written the outputs.
template <int BF16>
__global__ __launch_bounds__(256) void reject_nonfinite_rows_kernel(const void* __restrict__ W, int64_t m, int64_t k,
                                                                    int64_t ldw, bool vec, const float* __restrict__ gptr,
                                                                    uint8_t* __restrict__ codes,
                                                                    uint8_t* __restrict__ scales,
                                                                    float* __restrict__ row_err,
                                                                    float* __restrict__ row_loss, int64_t stride_w) {
  {   // matrix e = blockIdx.y of a batch
    const int64_t e = blockIdx.y;
    W = (const char*)W + e * stride_w * (BF16 ? 2 : 4);
    gptr += e;
    codes += e * m * (k / 2);
    scales += e * m * (k / kBlock);
    if (row_err) row_err += e * m;
    if (row_loss) row_loss += e * m;
  }
  const float g = *gptr;
  const bool g_bad = !(g > 0.0f) || __builtin_isinf(g);
  for (int64_t r = blockIdx.x; r < m; r += gridDim.x) {
    if (!g_bad && !row_nonfinite<BF16>(W, r, k, ldw, vec)) continue;
    for (int64_t c = threadIdx.x; c < k / 2; c += blockDim.x) codes[r * (k / 2) + c] = 0;
    for (int64_t c = threadIdx.x; c < k / kBlock; c += blockDim.x) scales[r * (k / kBlock) + c] = 0x7F;
    if (threadIdx.x == 0) {
      if (row_err) row_err[r] = __builtin_nanf("");
      if (row_loss) row_loss[r] = __builtin_nanf("");
    }
  }
}

// ---- sweep helpers ------------------------------------------------------------------
template <int BF16>
__global__ void load_working_f64_kernel(const void* __restrict__ W, int64_t m, int64_t k, int64_t ldw,
                                        double* __restrict__ Wp, int64_t stride_w, int64_t stride_wp) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= m * k) return;
  W = (const char*)W + (int64_t)blockIdx.y * stride_w * (BF16 ? 2 : 4);   // matrix of a batch
  Wp += (int64_t)blockIdx.y * stride_wp;
  Wp[e] = (double)load_w<BF16>(W, (e / k) * ldw + e % k);
}

template <int BF16>
__global__ void load_working_kernel(const void* __restrict__ W, int64_t m, int64_t k, int64_t ldw,
                                    float* __restrict__ Wp, int64_t stride_w, int64_t stride_wp) {
  int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= m * k) return;
  W = (const char*)W + (int64_t)blockIdx.y * stride_w * (BF16 ? 2 : 4);   // matrix of a batch
  Wp += (int64_t)blockIdx.y * stride_wp;
  int64_t r = e / k, c = e % k;  // k % 4 == 0: the 4 elements share a row
  f32x4 v;
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = load_w<BF16>(W, r * ldw + c + q);
  *(f32x4*)(Wp + e) = v;
}

// invd[j] = 1 / U[j][j], or U[j][j] itself (copy: the diagonal of the
// Cholesky-factor form, R_jj, by which the sweep multiplies).
__global__ void inv_diag_kernel(const float* __restrict__ U, int64_t k, float* __restrict__ invd, int64_t stride_u,
                                int64_t stride_invd, int copy) {
  int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  U += (int64_t)blockIdx.y * stride_u;   // matrix of a batch
  invd += (int64_t)blockIdx.y * stride_invd;
  if (j < k) invd[j] = copy ? U[j * k + j] : 1.0f / U[j * k + j];
}

// Cholesky-factor form: for each diagonal 16x16 block of V (N its strictly
// upper part, N_ij = -R_ij / R_jj), M = (I - N)^-1, unit upper triangular,
// found column by column by substitution (no divisions) in fp64.  Thread t
// (block t / 16, column c = t % 16) writes Mt[t][i] = M_ic for i < c and 0
// for i >= c: the transposed strictly upper part the sweep reads by columns.
__global__ void chol_block_m_kernel(const float* __restrict__ V, int64_t k, float* __restrict__ Mt, int64_t stride_v,
                                    int64_t stride_m) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  V += (int64_t)blockIdx.y * stride_v;
  Mt += (int64_t)blockIdx.y * stride_m;
  if (t >= k) return;
  const int c = (int)(t % 16);
  const float* vb = V + (t - c) * k + (t - c);   // the block's top-left element
  double x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = i == c ? 1.0 : 0.0;
  // (I - N) x = e_c: x_i = sum_{j > i} N_ij x_j, taking j downwards (x_j is
  // final once every later column has added its part; x_j = 0 for j > c).
#pragma unroll
  for (int j = 15; j >= 1; --j)
#pragma unroll
    for (int i = 0; i < j; ++i) x[i] = fma((double)vb[(int64_t)i * k + j], x[j], x[i]);
#pragma unroll
  for (int i = 0; i < 16; ++i) Mt[t * 16 + i] = i < c ? (float)x[i] : 0.0f;
}

// dW = W - dequant(codes, scales, g) as fp32 [m x k].
template <int BF16>
__global__ __launch_bounds__(256) void delta_w_kernel(const void* __restrict__ W, int64_t m, int64_t k,
                                                      int64_t ldw, const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales,
                                                      const float* __restrict__ gptr, float* __restrict__ dW,
                                                      int64_t blk0, int64_t nblk, int64_t stride_w,
                                                      int64_t stride_dw) {
  const int64_t nbk = k / kBlock;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= m * nblk) return;
  {   // matrix e = blockIdx.y of a batch
    const int64_t e = blockIdx.y;
    W = (const char*)W + e * stride_w * (BF16 ? 2 : 4);
    codes += e * m * (k / 2);
    scales += e * m * nbk;
    gptr += e;
    dW += e * stride_dw;
  }
  const int64_t row = t / nblk, blk = blk0 + t % nblk, b = row * nbk + blk;
  const float g = *gptr;
  const float s = e4m3_value(scales[b] & 0x7F);
  u32x2 c = *(const u32x2*)(codes + b * 8);
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    int code = (c[j >> 3] >> (4 * (j & 7))) & 0xF;
    dW[row * k + blk * 16 + j] = load_w<BF16>(W, row * ldw + blk * 16 + j) - e2m1_dequant(code, s, g);
  }
}

__global__ void row_sum_kernel(const float* __restrict__ P, int64_t m, int64_t np, float* __restrict__ out,
                               int64_t stride_p) {
  int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= m) return;
  P += (int64_t)blockIdx.y * stride_p;   // matrix of a batch
  out += (int64_t)blockIdx.y * m;
  float s = 0.0f;
  for (int64_t t = 0; t < np; ++t) s += P[r * np + t];
  out[r] = s;
}

__global__ void fill_kernel(float* p, int64_t n, float v) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

// ---- the sweep of one lazy batch ---------------------------------------------------------
constexpr int UT_LD = kBatch + 4;

template <int G>
struct SweepCfg {
  static constexpr int ROWS = (64 / G) > 16 ? (64 / G) : 16;
  static constexpr int THREADS = ROWS * G;
  // With two or more waves per workgroup the launch applies the earlier
  // batches' errors of the 512-column block to its rows itself.
  static constexpr bool INBLOCK = G >= 8;
};

// One butterfly step of the candidate arg-min inside groups of G lanes.
// DPP moves within 16-lane rows.  The order is total, so every lane of a
// group ends with the same winner: the least score, ties to the lower
// candidate index, a NaN score (a non-finite weight in the row) above every
// number and NaN ties again to the lower index.
template <typename T>
__device__ __forceinline__ bool argmin_takes(T so, int io, T s, int i) {
  const bool sn = s != s, on = so != so;
  return (!on && (sn || so < s)) || ((so == s || (sn && on)) && io < i);
}
template <int CTRL>
__device__ __forceinline__ void argmin_step(float& s, int& i) {
  const float so = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(s), CTRL, 0xF, 0xF, false));
  const int io = __builtin_amdgcn_mov_dpp(i, CTRL, 0xF, 0xF, false);
  if (argmin_takes(so, io, s, i)) { s = so; i = io; }
}
template <int CTRL>
__device__ __forceinline__ float sum_step(float s) {
  return s + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(s), CTRL, 0xF, 0xF, false));
}
// Lane pairings: xor 1 and xor 2 (quad_perm), then 8-lane and 16-lane mirrors.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

// fp64 values move as two 32-bit halves.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = __double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)u, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
template <int CTRL>
__device__ __forceinline__ void argmin_step(double& s, int& i) {
  const double so = dpp_f64<CTRL>(s);
  const int io = __builtin_amdgcn_mov_dpp(i, CTRL, 0xF, 0xF, false);
  if (argmin_takes(so, io, s, i)) { s = so; i = io; }
}
template <int CTRL>
__device__ __forceinline__ double sum_step(double s) {
  return s + dpp_f64<CTRL>(s);
}

template <int G, typename T>
__device__ __forceinline__ void group_argmin(T& s, int& i) {
  if (G >= 2) argmin_step<kDppXor1>(s, i);
  if (G >= 4) argmin_step<kDppXor2>(s, i);
  if (G >= 8) argmin_step<kDppHalfMirror>(s, i);
  if (G >= 16) argmin_step<kDppMirror>(s, i);
}
template <int CTRL>
__device__ __forceinline__ float max_step(float s) {
  return fmaxf(s, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(s), CTRL, 0xF, 0xF, false)));
}
template <int CTRL>
__device__ __forceinline__ double max_step(double s) {
  return fmax(s, dpp_f64<CTRL>(s));
}
template <int G, typename T>
__device__ __forceinline__ T group_max(T s) {
  if (G >= 2) s = max_step<kDppXor1>(s);
  if (G >= 4) s = max_step<kDppXor2>(s);
  if (G >= 8) s = max_step<kDppHalfMirror>(s);
  if (G >= 16) s = max_step<kDppMirror>(s);
  return s;
}
template <int G, typename T>
__device__ __forceinline__ T group_sum(T s) {
  if (G >= 2) s = sum_step<kDppXor1>(s);
  if (G >= 4) s = sum_step<kDppXor2>(s);
  if (G >= 8) s = sum_step<kDppHalfMirror>(s);
  if (G >= 16) s = sum_step<kDppMirror>(s);
  return s;
}

// A row's G candidate lanes always lie in one wave, so after the initial
// loads the block loop needs no workgroup barrier: a wave's LDS accesses are
// executed in program order.  T is the working precision (fp32, or fp64 for
// layers whose Hessian spreads over many orders of magnitude); U stays fp32
// (its values are exact inputs) and is widened where it is used.  In fp32 the
// error of a column is (w' - q) times the rounded 1/U_jj; in fp64 it is the
// quotient (w' - q) / U_jj.
template <typename T>
__device__ __forceinline__ void load16(const T* p, T (&v)[16]) {
#pragma unroll
  for (int q = 0; q < 16; ++q) v[q] = p[q];
}

// CHOL: U holds V from the Cholesky factor R of H_d = R R^T (V_ij = -R_ij /
// R_jj above the diagonal, V_jj = R_jj, so invd holds R_jj), and W0 the
// weights as input.  The same updates are then taken as w'_l = w_l +
// sum_{j<l} (w_j - q_j) R_jl / R_ll: a committed column propagates its raw
// error w_j - q_j (against its input value) through V where the inverse form
// propagates e_j = (w'_j - q_j) / U_jj through U, and its score term is
// e_j = (w'_j - q_j) R_jj (U_jj = 1 / R_jj).  The error slab holds the
// propagated values, so the lazy updates are unchanged.  Mid-block the two
// forms hold different values for the columns not yet reached, and the
// candidate window is set by the absmax of the inverse form's block-start
// values a = w + P_{<c0} R_{<c0,B} U_BB.  With b the values held here and
// U_BB = R_BB^-1 = D^-1 (I - N)^-1 (D = diag R_BB, N the strictly upper part
// of V's diagonal block), a = b + (b - w)(M - I) with M = (I - N)^-1; Mb holds
// each block's M - I transposed (chol_block_m_kernel), and the candidate
// lanes of a row share the 16 columns of a before a group max.  A block whose
// a is all zero takes q = 0 and propagates its input weights.
template <int G, typename T, bool INDEP, bool CHOL>
__global__ __launch_bounds__(SweepCfg<G>::THREADS) void sweep_batch_kernel(
    T* __restrict__ Wp, const T* __restrict__ W0, const float* __restrict__ U, const float* __restrict__ invd,
    const float* __restrict__ gptr, int64_t m, int64_t k, int i1, int ncols, int n_cand,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, T* __restrict__ Eslab, int64_t lde,
    float* __restrict__ row_loss, SweepStrides bs, int pre, const float* __restrict__ Mb) {
  constexpr bool F64 = sizeof(T) == 8;
  {   // matrix e = blockIdx.y of a batch
    const int64_t e = blockIdx.y;
    Wp += e * bs.wp;
    if (CHOL) W0 += e * bs.wp;
    if (CHOL) Mb += e * bs.mb;
    U += e * bs.u;
    invd += e * bs.invd;
    gptr += e;
    codes += e * m * (k / 2);
    scales += e * m * (k / kBlock);
    Eslab += e * bs.e;
    if (row_loss) row_loss += e * m;
  }
  constexpr int ROWS = SweepCfg<G>::ROWS;
  constexpr int NT = SweepCfg<G>::THREADS;
  __shared__ __attribute__((aligned(16))) float Ut[kBatch * UT_LD];      // Ut[c][r] = U[i1+r][i1+c]
  __shared__ __attribute__((aligned(16))) float Ud[kBatch / kBlock][kBlock][kBlock];  // diagonal 16x16 blocks
  __shared__ __attribute__((aligned(16))) float id_s[kBatch];
  __shared__ __attribute__((aligned(16))) float Mt_s[CHOL ? kBatch / kBlock : 1][kBlock][kBlock];  // CHOL: M - I
  // Rows padded by 64 bytes: the four rows a wave touches fall on distinct banks.
  __shared__ __attribute__((aligned(16))) T slab[ROWS][kBatch + 64 / sizeof(T)];
  __shared__ __attribute__((aligned(16))) T eb_s[ROWS][16];

  const int tid = threadIdx.x;
  const int rl = tid / G, ci = tid % G;
  const int64_t row = (int64_t)blockIdx.x * ROWS + rl;
  const bool row_ok = row < m;
  const float g = *gptr;
  const float r6g = 1.0f / (6.0f * g);   // only locates the candidate window's centre

  // Staging: Ut[c][r] = U[i1+r][i1+c] for r <= c < ncols (0 elsewhere), the
  // diagonal 16x16 blocks, 1/U_jj and the rows' slab of W'.  Every load is a
  // 16-byte vector at a clamped (always valid) address and the loads of a
  // chunk are all issued before its LDS writes.  ncols is a multiple of 16.
  // U is staged by 16x16 tiles on or above the diagonal (the kernel reads
  // no other part): one wave-instruction loads a tile as 16 rows x 4 float4,
  // so the transposed LDS writes of its 64 lanes hit 64 distinct banks.
  constexpr int NW = NT / 64;                         // waves
  constexpr int NTILE = (kBatch / 16) * (kBatch / 16 + 1) / 2;
  constexpr int UCH = NTILE / NW < 9 ? NTILE / NW : 9;   // tiles per wave in flight
  static_assert(NTILE % (NW * UCH) == 0, "tile chunks");
  constexpr int VT = 16 / sizeof(T);                  // slab elements per vector
  constexpr int SV = ROWS * kBatch / VT;              // slab vectors
  constexpr int SCH = SV / NT < 8 ? SV / NT : 8;
  static_assert(SV % (NT * SCH) == 0, "slab chunks");
  typedef T tvec __attribute__((ext_vector_type(VT)));
  const int64_t row0 = (int64_t)blockIdx.x * ROWS;
  constexpr int IDN = (kBatch + NT - 1) / NT;
  float idv[IDN];
#pragma unroll
  for (int j = 0; j < IDN; ++j) idv[j] = invd[i1 + min(tid + j * NT, ncols - 1)];
  auto slab_load_from = [&](const T* src, int base, tvec (&w)[SCH]) {
#pragma unroll
    for (int it = 0; it < SCH; ++it) {
      const int idx = base + it * NT + tid;
      const int64_t gr = min(row0 + idx / (kBatch / VT), m - 1);
      const int c = min((idx % (kBatch / VT)) * VT, ncols - VT);
      w[it] = *(const tvec*)(src + gr * k + i1 + c);
    }
  };
  auto slab_store_to = [&](T (*dst)[kBatch + 64 / sizeof(T)], int base, const tvec (&w)[SCH]) {
#pragma unroll
    for (int it = 0; it < SCH; ++it) {
      const int idx = base + it * NT + tid;
      const int r = idx / (kBatch / VT), c = (idx % (kBatch / VT)) * VT;
      const bool ok = row0 + r < m && c < ncols;
      tvec v;
#pragma unroll
      for (int t = 0; t < VT; ++t) v[t] = ok ? w[it][t] : T(0);
      *(tvec*)&dst[r][c] = v;
    }
  };
  auto slab_load = [&](int base, tvec (&w)[SCH]) { slab_load_from(Wp, base, w); };
  auto slab_store = [&](int base, const tvec (&w)[SCH]) { slab_store_to(slab, base, w); };
  tvec w0[SCH];
  slab_load(0, w0);
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  for (int base = 0; base < NTILE; base += NW * UCH) {
    f32x4 u[UCH];
    int tr[UCH], tc[UCH];
#pragma unroll
    for (int it = 0; it < UCH; ++it) {
      // upper-triangle tile q -> (tile row, tile column), row-major
      int q = base + it * NW + wave, t_r = 0, len = kBatch / 16;
      while (q >= len) { q -= len; ++t_r; --len; }
      tr[it] = t_r; tc[it] = t_r + q;
      const int r = min(tr[it] * 16 + lane % 16, ncols - 1);
      const int c = min(tc[it] * 16 + (lane / 16) * 4, ncols - 4);
      u[it] = *(const f32x4*)(U + (int64_t)(i1 + r) * k + i1 + c);
    }
    if (base == 0) slab_store(0, w0);
#pragma unroll
    for (int it = 0; it < UCH; ++it) {
      const int r = tr[it] * 16 + lane % 16, c = tc[it] * 16 + (lane / 16) * 4;
      f32x4 v;
#pragma unroll
      for (int t = 0; t < 4; ++t) v[t] = (r < ncols && c + t < ncols && r <= c + t) ? u[it][t] : 0.0f;
#pragma unroll
      for (int t = 0; t < 4; ++t) Ut[(c + t) * UT_LD + r] = v[t];
      if (tr[it] == tc[it]) *(f32x4*)&Ud[tr[it]][r & 15][c & 15] = v;
    }
  }
#pragma unroll
  for (int j = 0; j < IDN; ++j)
    if (tid + j * NT < kBatch) id_s[tid + j * NT] = tid + j * NT < ncols ? idv[j] : 0.0f;
  if constexpr (CHOL) {   // the batch's ncols / 16 blocks of M - I, 256 floats each
    const f32x4* src = (const f32x4*)(Mb + (int64_t)i1 * kBlock);
    for (int idx = tid; idx < ncols * (kBlock / 4); idx += NT) ((f32x4*)&Mt_s[0][0][0])[idx] = src[idx];
  }
  for (int base = NT * SCH; base < SV; base += NT * SCH) {
    tvec w[SCH];
    slab_load(base, w);
    slab_store(base, w);
  }
  __syncthreads();

  // The earlier batches of this 512-column block (pre columns, whose errors
  // sit just before this batch's in the error slab) have not yet updated the
  // batch's columns: slab[r][c] -= sum_q E[r][q] U[i1-pre+q][i1+c], on
  // v_mfma_f32_16x16x4f32 tiles of 16 rows x 16 columns, each wave taking
  // 128 / NW columns.  Lane (l16, lq) supplies q = kc + 4 lq + s at step s of
  // a 16-value chunk: one 16-byte read of its row's errors, and U rows read
  // as 64-byte row pieces.  Rows past m read row m-1 (results unused);
  // columns past ncols are neither read nor written.
  if constexpr (!F64 && SweepCfg<G>::INBLOCK) {
    if (pre > 0) {
      static_assert(ROWS == 16, "one 16-row tile per workgroup");
      constexpr int TPW = kBatch / 16 / NW;   // column tiles per wave
      const int l16 = lane & 15, lq = lane >> 4;
      const float* ep = Eslab - pre + min(row0 + l16, m - 1) * lde + 4 * lq;
      const float* up = U + (int64_t)(i1 - pre + 4 * lq) * k + i1;
      int col[TPW];
#pragma unroll
      for (int t = 0; t < TPW; ++t) col[t] = min((wave * TPW + t) * 16 + l16, ncols - 1);
      f32x4 acc[TPW];
#pragma unroll
      for (int t = 0; t < TPW; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      // Stages of 64 k-values in two buffers: one stage's loads are in flight
      // during the other's products (pre is a multiple of 128; the last load
      // repeats the last stage, unused).  The scheduling barriers keep the
      // loads ahead of the products they overlap.
      constexpr int CU = 4;
      struct Stage {
        f32x4 a[CU];
        float b[CU][4][TPW];
      };
      auto load_stage = [&](int kc, Stage& o) {
#pragma unroll
        for (int c = 0; c < CU; ++c) {
          o.a[c] = *(const f32x4*)(ep + kc + 16 * c);
#pragma unroll
          for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int t = 0; t < TPW; ++t) o.b[c][st][t] = up[(int64_t)(kc + 16 * c + st) * k + col[t]];
        }
      };
      auto mfma_stage = [&](const Stage& o) {
#pragma unroll
        for (int c = 0; c < CU; ++c)
#pragma unroll
          for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int t = 0; t < TPW; ++t)
              acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(o.a[c][st], o.b[c][st][t], acc[t], 0, 0, 0);
      };
      Stage sa, sb;
      load_stage(0, sa);
      for (int kc = 0; kc < pre; kc += 32 * CU) {
        load_stage(kc + 16 * CU, sb);
        __builtin_amdgcn_sched_barrier(0);
        mfma_stage(sa);
        __builtin_amdgcn_sched_barrier(0);
        load_stage(min(kc + 32 * CU, pre - 16 * CU), sa);
        __builtin_amdgcn_sched_barrier(0);
        mfma_stage(sb);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int c = (wave * TPW + t) * 16 + l16;
        if (c < ncols) {
#pragma unroll
          for (int r = 0; r < 4; ++r) slab[4 * lq + r][c] -= acc[t][r];
        }
      }
      __syncthreads();
    }
  }

  T loss = 0;
  const int nblk = ncols / kBlock;
  // CHOL: the row's input weights of a block, read one block ahead (16-byte
  // loads; rows past m read row m-1, unused).
  const T* w0row = CHOL ? W0 + min(row, m - 1) * k + i1 : nullptr;
  auto load_w0 = [&](int c0, T (&o)[16]) {
#pragma unroll
    for (int q = 0; q < 16 / VT; ++q) {
      const tvec t = *(const tvec*)(w0row + c0 + VT * q);
#pragma unroll
      for (int u = 0; u < VT; ++u) o[VT * q + u] = t[u];
    }
  };
  T o_next[16];
  if constexpr (CHOL) load_w0(0, o_next);
  for (int b = 0; b < nblk; ++b) {
    const int c0 = b * kBlock;
    T v[16];
    if constexpr (F64) {
      load16(&slab[rl][c0], v);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4 t = *(const f32x4*)&slab[rl][c0 + 4 * q];
        v[4 * q] = t[0]; v[4 * q + 1] = t[1]; v[4 * q + 2] = t[2]; v[4 * q + 3] = t[3];
      }
    }
    T o[16];   // CHOL: the block's input weights
    if constexpr (CHOL) {
#pragma unroll
      for (int j = 0; j < 16; ++j) o[j] = o_next[j];
      load_w0(min(c0 + kBlock, ncols - kBlock), o_next);
    }
    // The block-start values the candidate window (and the block-independent
    // score) is taken on: v itself, or with CHOL a = v + (v - w)(M - I).
    T a = 0;
    T av[INDEP ? 16 : 1];
    if constexpr (!CHOL) {
#pragma unroll
      for (int j = 0; j < 16; ++j) a = fmax(a, fabs(v[j]));
      if constexpr (INDEP) {
#pragma unroll
        for (int j = 0; j < 16; ++j) av[j] = v[j];
      }
    } else {
      T d[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) d[j] = v[j] - o[j];
      auto column = [&](int c, T vc) {   // a_c (Mt_s[b][c][j] = 0 for j >= c)
        T acc = vc;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 m4 = *(const f32x4*)&Mt_s[b][c][4 * q];
#pragma unroll
          for (int u = 0; u < 4; ++u) acc = fma(d[4 * q + u], (T)m4[u], acc);
        }
        return acc;
      };
      if constexpr (INDEP) {
#pragma unroll
        for (int c = 0; c < 16; ++c) {
          av[c] = column(c, v[c]);
          a = fmax(a, fabs(av[c]));
        }
      } else {
#pragma unroll
        for (int t = 0; t < 16 / G; ++t) {
          const int c = ci + G * t;
          a = fmax(a, fabs(column(c, slab[rl][c0 + c])));
        }
        a = group_max<G>(a);
      }
    }

    T e[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) e[j] = CHOL ? o[j] : T(0);   // CHOL: the propagated values when a = 0
    uint32_t plo = 0, phi = 0;
    int cand = 0;
    T score = F64 ? T(__builtin_inf()) : T(__builtin_inff());
    T rsc = 0;   // this candidate's replay score (its damped loss)
    if (a > T(0)) {
      const int lo = candidate_lo(e4m3_code_of_ratio_any(a, g, r6g), n_cand);
      cand = lo + (ci < n_cand ? ci : 0);
      const float s = e4m3_value_sel(cand);
      const float hs = 0.5f * s;
      const float ts[7] = {0.25f * s, 0.75f * s, 1.25f * s, 1.75f * s, 2.5f * s, 3.5f * s, 5.0f * s};
      // Block-independent selection: the plain squared rounding error of the
      // block's weights at the block start, each rounded on its own.
      T isc = 0;
      if constexpr (INDEP) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          T dj;
          if constexpr (F64) dj = av[j] - e2m1_dequant_f64(e2m1_encode(av[j], s, g), s, g);
          else dj = av[j] - e2m1_dequant(e2m1_encode(av[j], s, g), s, g);
          isc = fma(dj, dj, isc);
        }
      }
      T sc = 0;
      // Row j of the block's U is read while column j - 1 is encoded, so the
      // LDS latency hides behind that work (one wave per SIMD runs here).
      f32x4 un[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) un[q] = *(const f32x4*)&Ud[b][0][4 * q];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float urow[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          urow[4 * q] = un[q][0]; urow[4 * q + 1] = un[q][1]; urow[4 * q + 2] = un[q][2]; urow[4 * q + 3] = un[q][3];
        }
        if (j + 1 < 15) {
#pragma unroll
          for (int q = 0; q < 4; ++q) un[q] = *(const f32x4*)&Ud[b][j + 1][4 * q];
          __builtin_amdgcn_sched_barrier(0x7);   // arithmetic may move across, memory accesses may not
        }
        int code;
        T ej, pj;   // the score term and the propagated value
        if constexpr (F64) {
          code = e2m1_encode(v[j], s, g);
          const T dq = e2m1_dequant_f64(code, s, g);
          ej = CHOL ? (v[j] - dq) * (T)Ud[b][j][j] : (v[j] - dq) / (T)Ud[b][j][j];
          pj = CHOL ? o[j] - dq : ej;
        } else {
          // The dequantized value e2m1_dequant gives, fl32(m * g) with the code's
          // sign set by a bit operation (m * g >= 0), then the error.  The
          // product and the difference are rounded separately (no contraction
          // into one fma).
#pragma clang fp contract(off)
          const float aw = fabsf(v[j]);
          const int idx = e2m1_index_search(aw, g, ts);
          code = idx | (int)(((__float_as_uint(v[j]) >> 31) & (uint32_t)(idx != 0)) << 3);
          const float mg = e2m1_twice_mag(idx) * hs * g;
          const float dq = __uint_as_float(__float_as_uint(mg) | ((uint32_t)(code & 8) << 28));
          ej = (v[j] - dq) * id_s[c0 + j];
          pj = CHOL ? o[j] - dq : ej;
        }
        sc = fma(ej, ej, sc);
        if (j + 1 < 16) {
#pragma unroll
          for (int l = j + 1; l < 16; ++l) v[l] = fma(-pj, (T)urow[l], v[l]);
        }
        e[j] = pj;
        if (j < 8) plo |= (uint32_t)code << (4 * j); else phi |= (uint32_t)code << (4 * (j - 8));
      }
      rsc = sc;
      if (ci < n_cand) score = INDEP ? isc : sc;
    }
    T bs = score;
    int bi = ci;
    group_argmin<G>(bs, bi);
    if (ci == bi && row_ok) {
#pragma unroll
      for (int j = 0; j < 16; ++j) eb_s[rl][j] = e[j];
      const int64_t gb = (i1 + c0) / kBlock;
      *(u32x2*)(codes + row * (k / 2) + gb * 8) = u32x2{plo, phi};
      scales[row * (k / kBlock) + gb] = (uint8_t)cand;
      T* es = Eslab + row * lde + c0;
#pragma unroll
      for (int j = 0; j < 16; ++j) es[j] = e[j];
      if (a > T(0)) loss += rsc;
    }
    // Update the later columns of the batch: w'_l -= sum_j e_j U[c0+j][l].
    if (row_ok && c0 + kBlock < ncols) {
      T eb[16];
      load16(&eb_s[rl][0], eb);
      for (int cc = c0 + kBlock + ci; cc < ncols; cc += G) {
        T acc = slab[rl][cc];
        const float* ut = &Ut[cc * UT_LD + c0];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f32x4 u4 = *(const f32x4*)(ut + 4 * q);
          acc = fma(-eb[4 * q + 0], (T)u4[0], acc);
          acc = fma(-eb[4 * q + 1], (T)u4[1], acc);
          acc = fma(-eb[4 * q + 2], (T)u4[2], acc);
          acc = fma(-eb[4 * q + 3], (T)u4[3], acc);
        }
        slab[rl][cc] = acc;
      }
    }
  }
  // Per-row loss: the winners' scores are spread over the row's lanes.
  loss = group_sum<G>(loss);
  if (ci == 0 && row_ok && row_loss) row_loss[row] += (float)loss;
}

template <int G, typename T>
hipError_t sweep_launch_g(T* Wp, const T* W0, const float* U, const float* invd, const float* g, int64_t m,
                          int64_t k, int i1, int ncols, int n_cand, bool indep, uint8_t* codes, uint8_t* scales,
                          T* Eslab, int64_t lde, float* row_loss, hipStream_t s, int64_t nb, const SweepStrides& bs,
                          int pre, const float* Mb) {
  constexpr int ROWS = SweepCfg<G>::ROWS;
  if (!SweepCfg<G>::INBLOCK || sizeof(T) != 4) pre = 0;
  dim3 grid((unsigned)((m + ROWS - 1) / ROWS), (unsigned)nb);
  const dim3 blk(SweepCfg<G>::THREADS);
#define NVQ_SWEEP_LAUNCH(IND, CH)                                                                                  \
  hipLaunchKernelGGL((sweep_batch_kernel<G, T, IND, CH>), grid, blk, 0, s, Wp, W0, U, invd, g, m, k, i1, ncols,     \
                     n_cand, codes, scales, Eslab, lde, row_loss, bs, pre, Mb)
  if (W0) {
    if (indep) NVQ_SWEEP_LAUNCH(true, true); else NVQ_SWEEP_LAUNCH(false, true);
  } else {
    if (indep) NVQ_SWEEP_LAUNCH(true, false); else NVQ_SWEEP_LAUNCH(false, false);
  }
#undef NVQ_SWEEP_LAUNCH
  return hipGetLastError();
}
template <typename T>
hipError_t sweep_launch_t(T* Wp, const T* W0, const float* U, const float* invd, const float* g, int64_t m, int64_t k, int i1,
                          int ncols, int n_cand, bool indep, uint8_t* codes, uint8_t* scales, T* Eslab, int64_t lde,
                          float* row_loss, hipStream_t s, int64_t nb, const SweepStrides& bs, int pre,
                          const float* Mb) {
  if (W0 && !Mb) return hipErrorInvalidValue;
  if (n_cand <= 1) return sweep_launch_g<1>(Wp, W0, U, invd, g, m, k, i1, ncols, n_cand, indep, codes, scales, Eslab, lde, row_loss, s, nb, bs, pre, Mb);
  if (n_cand <= 2) return sweep_launch_g<2>(Wp, W0, U, invd, g, m, k, i1, ncols, n_cand, indep, codes, scales, Eslab, lde, row_loss, s, nb, bs, pre, Mb);
  if (n_cand <= 4) return sweep_launch_g<4>(Wp, W0, U, invd, g, m, k, i1, ncols, n_cand, indep, codes, scales, Eslab, lde, row_loss, s, nb, bs, pre, Mb);
  if (n_cand <= 8) return sweep_launch_g<8>(Wp, W0, U, invd, g, m, k, i1, ncols, n_cand, indep, codes, scales, Eslab, lde, row_loss, s, nb, bs, pre, Mb);
  return sweep_launch_g<16>(Wp, W0, U, invd, g, m, k, i1, ncols, n_cand, indep, codes, scales, Eslab, lde, row_loss, s, nb, bs, pre, Mb);
}

}  // namespace

int global_scale_parts(int64_t m, int64_t k) {
  (void)k;
  int64_t blocks = m;   // one or more rows per workgroup
  if (blocks > 1024) blocks = 1024;
  return (int)(blocks < 1 ? 1 : blocks);
}

hipError_t global_scale_launch(const void* W, int bf16, int64_t m, int64_t k, int64_t ldw, float* g,
                               float* partial, int nparts, hipStream_t s) {
  const bool vec = ((uintptr_t)W % 16 == 0) && (ldw % 8 == 0) && (k % 8 == 0);
  if (bf16)
    hipLaunchKernelGGL(amax_kernel<1>, dim3(nparts), dim3(256), 0, s, W, m, k, ldw, partial, vec);
  else
    hipLaunchKernelGGL(amax_kernel<0>, dim3(nparts), dim3(256), 0, s, W, m, k, ldw, partial, vec);
  hipLaunchKernelGGL(gscale_finish_kernel, dim3(1), dim3(256), 0, s, partial, nparts, g);
  return hipGetLastError();
}

// Workgroups of a grid-stride streaming launch: enough for every CU several
// times over, never more than the items need.
static unsigned stream_grid(int64_t items_per_wg) {
  const int64_t cap = 8 * 256;
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(items_per_wg, cap));
}

hipError_t dequant_launch(const uint8_t* codes, const uint8_t* scales, const float* g, int64_t m, int64_t k,
                          void* out, int out_bf16, hipStream_t s) {
  const int64_t nhalf = 2 * m * (k / kBlock);
  if (nhalf == 0) return hipSuccess;
  const dim3 grid(stream_grid((nhalf + 256 * DQ_U - 1) / (256 * DQ_U)));
  if (out_bf16)
    hipLaunchKernelGGL(dequant_kernel<1>, grid, dim3(256), 0, s, codes, scales, g, nhalf, out);
  else
    hipLaunchKernelGGL(dequant_kernel<0>, grid, dim3(256), 0, s, codes, scales, g, nhalf, out);
  return hipGetLastError();
}

hipError_t rtn_launch(const void* W, int bf16, int64_t m, int64_t k, int64_t ldw, const float* g, int n_cand,
                      uint8_t* codes, uint8_t* scales, float* row_loss, hipStream_t s, int64_t nb, int64_t stride_w) {
  int64_t nblk = m * (k / kBlock);
  dim3 grid(stream_grid((nblk + 255) / 256), (unsigned)nb);
  const int64_t es = bf16 ? 2 : 4;
  const bool vec = ((uintptr_t)W % 16 == 0) && (ldw % (bf16 ? 8 : 4) == 0) && ((stride_w * es) % 16 == 0);
  if (bf16)
    hipLaunchKernelGGL(rtn_kernel<1>, grid, dim3(256), 0, s, W, m, k, ldw, g, n_cand, codes, scales, vec, stride_w);
  else
    hipLaunchKernelGGL(rtn_kernel<0>, grid, dim3(256), 0, s, W, m, k, ldw, g, n_cand, codes, scales, vec, stride_w);
  if (row_loss)
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((nb * m + 255) / 256)), dim3(256), 0, s, row_loss, nb * m, 0.0f);
  return hipGetLastError();
}

hipError_t load_working_copy(const void* W, int bf16, int64_t m, int64_t k, int64_t ldw, float* Wp,
                             hipStream_t s, int64_t nb, int64_t stride_w, int64_t stride_wp) {
  dim3 grid((unsigned)((m * k / 4 + 255) / 256), (unsigned)nb);
  if (bf16)
    hipLaunchKernelGGL(load_working_kernel<1>, grid, dim3(256), 0, s, W, m, k, ldw, Wp, stride_w, stride_wp);
  else
    hipLaunchKernelGGL(load_working_kernel<0>, grid, dim3(256), 0, s, W, m, k, ldw, Wp, stride_w, stride_wp);
  return hipGetLastError();
}

hipError_t inv_diag_launch(const float* U, int64_t k, float* invd, hipStream_t s, int64_t nb, int64_t stride_u,
                           int64_t stride_invd, bool copy) {
  hipLaunchKernelGGL(inv_diag_kernel, dim3((unsigned)((k + 255) / 256), (unsigned)nb), dim3(256), 0, s, U, k, invd,
                     stride_u, stride_invd, (int)copy);
  return hipGetLastError();
}

hipError_t chol_block_m_launch(const float* V, int64_t k, float* Mb, hipStream_t s, int64_t nb, int64_t stride_v,
                               int64_t stride_m) {
  if (k % kBlock) return hipErrorInvalidValue;
  hipLaunchKernelGGL(chol_block_m_kernel, dim3((unsigned)((k + 255) / 256), (unsigned)nb), dim3(256), 0, s, V, k, Mb,
                     stride_v, stride_m);
  return hipGetLastError();
}

hipError_t load_working_copy_f64(const void* W, int bf16, int64_t m, int64_t k, int64_t ldw, double* Wp,
                                 hipStream_t s, int64_t nb, int64_t stride_w, int64_t stride_wp) {
  dim3 grid((unsigned)((m * k + 255) / 256), (unsigned)nb);
  if (bf16)
    hipLaunchKernelGGL(load_working_f64_kernel<1>, grid, dim3(256), 0, s, W, m, k, ldw, Wp, stride_w, stride_wp);
  else
    hipLaunchKernelGGL(load_working_f64_kernel<0>, grid, dim3(256), 0, s, W, m, k, ldw, Wp, stride_w, stride_wp);
  return hipGetLastError();
}

hipError_t sweep_batch_launch(float* Wp, const float* U, const float* invd, const float* g, int64_t m, int64_t k,
                              int i1, int ncols, int n_cand, bool indep, uint8_t* codes, uint8_t* scales,
                              float* Eslab, int64_t lde, float* row_loss, hipStream_t s, int64_t nb,
                              const SweepStrides& bs, int pre, const float* W0, const float* Mb) {
  return sweep_launch_t<float>(Wp, W0, U, invd, g, m, k, i1, ncols, n_cand, indep, codes, scales, Eslab, lde,
                               row_loss, s, nb, bs, pre, Mb);
}
bool sweep_applies_inblock(int n_cand) { return n_cand > 4; }
hipError_t sweep_batch_launch_f64(double* Wp, const float* U, const float* g, int64_t m, int64_t k, int i1,
                                  int ncols, int n_cand, bool indep, uint8_t* codes, uint8_t* scales, double* Eslab,
                                  int64_t lde, float* row_loss, hipStream_t s, int64_t nb, const SweepStrides& bs,
                                  const double* W0, const float* Mb) {
  // the fp64 sweep divides by U_jj itself: invd is not read (U is passed in its place)
  SweepStrides b2 = bs;
  b2.invd = bs.u;
  return sweep_launch_t<double>(Wp, W0, U, U, g, m, k, i1, ncols, n_cand, indep, codes, scales, Eslab, lde, row_loss,
                                s, nb, b2, 0, Mb);
}

hipError_t delta_w_launch(const void* W, int bf16, int64_t m, int64_t k, int64_t ldw, const uint8_t* codes,
                          const uint8_t* scales, const float* g, float* dW, hipStream_t s, int64_t c0, int64_t c1,
                          int64_t nb, int64_t stride_w, int64_t stride_dw) {
  if (c1 < 0) c1 = k;
  const int64_t blk0 = c0 / kBlock, nblk = (c1 - c0) / kBlock;
  if (m <= 0 || nblk <= 0) return hipSuccess;
  dim3 grid((unsigned)((m * nblk + 255) / 256), (unsigned)nb);
  if (bf16)
    hipLaunchKernelGGL(delta_w_kernel<1>, grid, dim3(256), 0, s, W, m, k, ldw, codes, scales, g, dW, blk0, nblk,
                       stride_w, stride_dw);
  else
    hipLaunchKernelGGL(delta_w_kernel<0>, grid, dim3(256), 0, s, W, m, k, ldw, codes, scales, g, dW, blk0, nblk,
                       stride_w, stride_dw);
  return hipGetLastError();
}

hipError_t row_sum_launch(const float* P, int64_t m, int64_t np, float* out, hipStream_t s, int64_t nb,
                          int64_t stride_p) {
  hipLaunchKernelGGL(row_sum_kernel, dim3((unsigned)((m + 255) / 256), (unsigned)nb), dim3(256), 0, s, P, m, np, out,
                     stride_p);
  return hipGetLastError();
}

namespace {
int scan_grid(int64_t rows) { return (int)(rows < 4096 ? (rows < 1 ? 1 : rows) : 4096); }
bool rows_vectorizable(const void* A, int bf16, int64_t cols, int64_t ld) {
  const int64_t es = bf16 ? 2 : 4;
  return (uintptr_t)A % 16 == 0 && (cols * es) % 16 == 0 && (ld * es) % 16 == 0;
}
}  // namespace

hipError_t nonfinite_scan_launch(const void* A, int bf16, int64_t rows, int64_t cols, int64_t ld, int32_t* status,
                                 hipStream_t s) {
  hipLaunchKernelGGL(status_init_kernel, dim3(1), dim3(1), 0, s, status);
  if (rows > 0) {
    const bool vec = rows_vectorizable(A, bf16, cols, ld);
    if (bf16)
      hipLaunchKernelGGL(nonfinite_scan_kernel<1>, dim3(scan_grid(rows)), dim3(256), 0, s, A, rows, cols, ld, vec,
                         status);
    else
      hipLaunchKernelGGL(nonfinite_scan_kernel<0>, dim3(scan_grid(rows)), dim3(256), 0, s, A, rows, cols, ld, vec,
                         status);
  }
  hipLaunchKernelGGL(status_finish_kernel, dim3(1), dim3(1), 0, s, status);
  return hipGetLastError();
}

hipError_t reject_nonfinite_rows_launch(const void* W, int bf16, int64_t m, int64_t k, int64_t ldw, const float* g,
                                        uint8_t* codes, uint8_t* scales, float* row_err, float* row_loss,
                                        hipStream_t s, int64_t nb, int64_t stride_w) {
  const bool vec = rows_vectorizable(W, bf16, k, ldw) && (stride_w * (bf16 ? 2 : 4)) % 16 == 0;
  const dim3 grid((unsigned)scan_grid(m), (unsigned)nb);
  if (bf16)
    hipLaunchKernelGGL(reject_nonfinite_rows_kernel<1>, grid, dim3(256), 0, s, W, m, k, ldw, vec, g, codes, scales,
                       row_err, row_loss, stride_w);
  else
    hipLaunchKernelGGL(reject_nonfinite_rows_kernel<0>, grid, dim3(256), 0, s, W, m, k, ldw, vec, g, codes, scales,
                       row_err, row_loss, stride_w);
  return hipGetLastError();
}

hipError_t fill_f32(float* p, int64_t n, float v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

}  // namespace nvq
