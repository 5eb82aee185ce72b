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
// updated afterwards by one fp32 MFMA GEMM with the batch's error slab.
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
template <int OUT_BF16>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales,
                                                      const float* __restrict__ gptr, int64_t m, int64_t k,
                                                      void* __restrict__ out) {
  // One thread per half block (8 weights: 4 bytes of codes, 16 bytes of bf16
  // out), so that a wave's loads and stores are contiguous.
  const int64_t nhalf = m * (k / kBlock) * 2;
  const int64_t hb = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (hb >= nhalf) return;
  const float g = *gptr;
  const uint8_t sc = scales[hb >> 1];
  const float s = e4m3_value(sc & 0x7F);
  const bool neg_scale = sc & 0x80;
  const uint32_t c = *(const uint32_t*)(codes + hb * 4);
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float x = e2m1_dequant((int)((c >> (4 * j)) & 0xF), s, g);
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

// ---- round to nearest (no GPTQ updates) ------------------------------------------
// One thread per (row, block).  Candidate scores are sum_j (w_j - q_j)^2 with
// separately rounded products and sums in column order.
// vec: every block starts 16-byte aligned (W aligned, ldw a multiple of 8
// bf16 or 4 fp32 values), so it is read with 16-byte loads.
template <int BF16>
__global__ __launch_bounds__(256) void rtn_kernel(const void* __restrict__ W, int64_t m, int64_t k, int64_t ldw,
                                                  const float* __restrict__ gptr, int n_cand,
                                                  uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                  bool vec) {
  const int64_t nbk = k / kBlock;
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= m * nbk) return;
  const int64_t row = b / nbk, blk = b % nbk;
  const float g = *gptr;
  float w[16];
  const int64_t base = row * ldw + blk * 16;
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
    const int lo = candidate_lo(e4m3_code_of_ratio_any(a, g, 1.0f / (6.0f * g)), n_cand);
    float best = __builtin_inff();
    for (int ci = 0; ci < n_cand; ++ci) {
      const int c = lo + ci;
      const float s = e4m3_value(c);
      const float hs = 0.5f * s;
      const float ts[7] = {0.25f * s, 0.75f * s, 1.25f * s, 1.75f * s, 2.5f * s, 3.5f * s, 5.0f * s};
      float score = 0.0f;
      uint32_t plo = 0, phi = 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        // e2m1_encode and e2m1_dequant's values, with the sign set by bit operations
        const int idx = e2m1_index_search(fabsf(w[j]), g, ts);
        const int code = idx | (int)(((__float_as_uint(w[j]) >> 31) & (uint32_t)(idx != 0)) << 3);
        const float dq = __uint_as_float(__float_as_uint(e2m1_twice_mag(idx) * hs * g) | ((uint32_t)(code & 8) << 28));
        float e = __fsub_rn(w[j], dq);
        score = __fadd_rn(score, __fmul_rn(e, e));
        if (j < 8) plo |= (uint32_t)code << (4 * j); else phi |= (uint32_t)code << (4 * (j - 8));
      }
      if (score < best) { best = score; best_c = c; best_lo = plo; best_hi = phi; }
    }
  }
  *(u32x2*)(codes + row * (k / 2) + blk * 8) = u32x2{best_lo, best_hi};
  scales[row * nbk + blk] = (uint8_t)best_c;
}

// ---- sweep helpers ------------------------------------------------------------------
template <int BF16>
__global__ void load_working_f64_kernel(const void* __restrict__ W, int64_t m, int64_t k, int64_t ldw,
                                        double* __restrict__ Wp) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= m * k) return;
  Wp[e] = (double)load_w<BF16>(W, (e / k) * ldw + e % k);
}

template <int BF16>
__global__ void load_working_kernel(const void* __restrict__ W, int64_t m, int64_t k, int64_t ldw,
                                    float* __restrict__ Wp) {
  int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= m * k) return;
  int64_t r = e / k, c = e % k;  // k % 4 == 0: the 4 elements share a row
  f32x4 v;
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = load_w<BF16>(W, r * ldw + c + q);
  *(f32x4*)(Wp + e) = v;
}

__global__ void inv_diag_kernel(const float* __restrict__ U, int64_t k, float* __restrict__ invd) {
  int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j < k) invd[j] = 1.0f / U[j * k + j];
}

// dW = W - dequant(codes, scales, g) as fp32 [m x k].
template <int BF16>
__global__ __launch_bounds__(256) void delta_w_kernel(const void* __restrict__ W, int64_t m, int64_t k,
                                                      int64_t ldw, const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales,
                                                      const float* __restrict__ gptr, float* __restrict__ dW,
                                                      int64_t blk0, int64_t nblk) {
  const int64_t nbk = k / kBlock;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= m * nblk) return;
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

__global__ void row_sum_kernel(const float* __restrict__ P, int64_t m, int64_t np, float* __restrict__ out) {
  int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= m) return;
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
};

// One butterfly step of the candidate arg-min inside groups of G lanes
// (ties to the lower candidate index).  DPP moves within 16-lane rows.
template <int CTRL>
__device__ __forceinline__ void argmin_step(float& s, int& i) {
  const float so = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(s), CTRL, 0xF, 0xF, false));
  const int io = __builtin_amdgcn_mov_dpp(i, CTRL, 0xF, 0xF, false);
  if (so < s || (so == s && io < i)) { s = so; i = io; }
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
  if (so < s || (so == s && io < i)) { s = so; i = io; }
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

template <int G, typename T, bool INDEP>
__global__ __launch_bounds__(SweepCfg<G>::THREADS) void sweep_batch_kernel(
    T* __restrict__ Wp, const float* __restrict__ U, const float* __restrict__ invd,
    const float* __restrict__ gptr, int64_t m, int64_t k, int i1, int ncols, int n_cand,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, T* __restrict__ Eslab, int64_t lde,
    float* __restrict__ row_loss) {
  constexpr bool F64 = sizeof(T) == 8;
  constexpr int ROWS = SweepCfg<G>::ROWS;
  constexpr int NT = SweepCfg<G>::THREADS;
  __shared__ __attribute__((aligned(16))) float Ut[kBatch * UT_LD];      // Ut[c][r] = U[i1+r][i1+c]
  __shared__ __attribute__((aligned(16))) float Ud[kBatch / kBlock][kBlock][kBlock];  // diagonal 16x16 blocks
  __shared__ __attribute__((aligned(16))) float id_s[kBatch];
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
  auto slab_load = [&](int base, tvec (&w)[SCH]) {
#pragma unroll
    for (int it = 0; it < SCH; ++it) {
      const int idx = base + it * NT + tid;
      const int64_t gr = min(row0 + idx / (kBatch / VT), m - 1);
      const int c = min((idx % (kBatch / VT)) * VT, ncols - VT);
      w[it] = *(const tvec*)(Wp + gr * k + i1 + c);
    }
  };
  auto slab_store = [&](int base, const tvec (&w)[SCH]) {
#pragma unroll
    for (int it = 0; it < SCH; ++it) {
      const int idx = base + it * NT + tid;
      const int r = idx / (kBatch / VT), c = (idx % (kBatch / VT)) * VT;
      const bool ok = row0 + r < m && c < ncols;
      tvec v;
#pragma unroll
      for (int t = 0; t < VT; ++t) v[t] = ok ? w[it][t] : T(0);
      *(tvec*)&slab[r][c] = v;
    }
  };
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
  for (int base = NT * SCH; base < SV; base += NT * SCH) {
    tvec w[SCH];
    slab_load(base, w);
    slab_store(base, w);
  }
  __syncthreads();

  T loss = 0;
  const int nblk = ncols / kBlock;
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
    T a = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) a = fmax(a, fabs(v[j]));

    T e[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) e[j] = 0;
    uint32_t plo = 0, phi = 0;
    int cand = 0;
    T score = F64 ? T(__builtin_inf()) : T(__builtin_inff());
    T rsc = 0;   // this candidate's replay score (its damped loss)
    if (a > T(0)) {
      const int lo = candidate_lo(e4m3_code_of_ratio_any(a, g, r6g), n_cand);
      cand = lo + (ci < n_cand ? ci : 0);
      const float s = e4m3_value(cand);
      const float hs = 0.5f * s;
      const float ts[7] = {0.25f * s, 0.75f * s, 1.25f * s, 1.75f * s, 2.5f * s, 3.5f * s, 5.0f * s};
      // Block-independent selection: the plain squared rounding error of the
      // block's weights at the block start, each rounded on its own.
      T isc = 0;
      if constexpr (INDEP) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          T dj;
          if constexpr (F64) dj = v[j] - e2m1_dequant_f64(e2m1_encode(v[j], s, g), s, g);
          else dj = v[j] - e2m1_dequant(e2m1_encode(v[j], s, g), s, g);
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
        T ej;
        if constexpr (F64) {
          code = e2m1_encode(v[j], s, g);
          ej = (v[j] - e2m1_dequant_f64(code, s, g)) / (T)Ud[b][j][j];
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
        }
        sc = fma(ej, ej, sc);
        if (j + 1 < 16) {
#pragma unroll
          for (int l = j + 1; l < 16; ++l) v[l] = fma(-ej, (T)urow[l], v[l]);
        }
        e[j] = ej;
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
hipError_t sweep_launch_g(T* Wp, const float* U, const float* invd, const float* g, int64_t m, int64_t k,
                          int i1, int ncols, int n_cand, bool indep, uint8_t* codes, uint8_t* scales, T* Eslab,
                          int64_t lde, float* row_loss, hipStream_t s) {
  constexpr int ROWS = SweepCfg<G>::ROWS;
  dim3 grid((unsigned)((m + ROWS - 1) / ROWS));
  if (indep)
    hipLaunchKernelGGL((sweep_batch_kernel<G, T, true>), grid, dim3(SweepCfg<G>::THREADS), 0, s, Wp, U, invd, g, m,
                       k, i1, ncols, n_cand, codes, scales, Eslab, lde, row_loss);
  else
    hipLaunchKernelGGL((sweep_batch_kernel<G, T, false>), grid, dim3(SweepCfg<G>::THREADS), 0, s, Wp, U, invd, g, m,
                       k, i1, ncols, n_cand, codes, scales, Eslab, lde, row_loss);
  return hipGetLastError();
}
template <typename T>
hipError_t sweep_launch_t(T* Wp, const float* U, const float* invd, const float* g, int64_t m, int64_t k, int i1,
                          int ncols, int n_cand, bool indep, uint8_t* codes, uint8_t* scales, T* Eslab, int64_t lde,
                          float* row_loss, hipStream_t s) {
  if (n_cand <= 1) return sweep_launch_g<1>(Wp, U, invd, g, m, k, i1, ncols, n_cand, indep, codes, scales, Eslab, lde, row_loss, s);
  if (n_cand <= 2) return sweep_launch_g<2>(Wp, U, invd, g, m, k, i1, ncols, n_cand, indep, codes, scales, Eslab, lde, row_loss, s);
  if (n_cand <= 4) return sweep_launch_g<4>(Wp, U, invd, g, m, k, i1, ncols, n_cand, indep, codes, scales, Eslab, lde, row_loss, s);
  if (n_cand <= 8) return sweep_launch_g<8>(Wp, U, invd, g, m, k, i1, ncols, n_cand, indep, codes, scales, Eslab, lde, row_loss, s);
  return sweep_launch_g<16>(Wp, U, invd, g, m, k, i1, ncols, n_cand, indep, codes, scales, Eslab, lde, row_loss, s);
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

hipError_t dequant_launch(const uint8_t* codes, const uint8_t* scales, const float* g, int64_t m, int64_t k,
                          void* out, int out_bf16, hipStream_t s) {
  int64_t nblk = m * (k / kBlock);
  if (nblk == 0) return hipSuccess;
  dim3 grid((unsigned)((2 * nblk + 255) / 256));
  if (out_bf16)
    hipLaunchKernelGGL(dequant_kernel<1>, grid, dim3(256), 0, s, codes, scales, g, m, k, out);
  else
    hipLaunchKernelGGL(dequant_kernel<0>, grid, dim3(256), 0, s, codes, scales, g, m, k, out);
  return hipGetLastError();
}

hipError_t rtn_launch(const void* W, int bf16, int64_t m, int64_t k, int64_t ldw, const float* g, int n_cand,
                      uint8_t* codes, uint8_t* scales, float* row_loss, hipStream_t s) {
  int64_t nblk = m * (k / kBlock);
  dim3 grid((unsigned)((nblk + 255) / 256));
  const bool vec = ((uintptr_t)W % 16 == 0) && (ldw % (bf16 ? 8 : 4) == 0);
  if (bf16)
    hipLaunchKernelGGL(rtn_kernel<1>, grid, dim3(256), 0, s, W, m, k, ldw, g, n_cand, codes, scales, vec);
  else
    hipLaunchKernelGGL(rtn_kernel<0>, grid, dim3(256), 0, s, W, m, k, ldw, g, n_cand, codes, scales, vec);
  if (row_loss) hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, s, row_loss, m, 0.0f);
  return hipGetLastError();
}

hipError_t load_working_copy(const void* W, int bf16, int64_t m, int64_t k, int64_t ldw, float* Wp,
                             hipStream_t s) {
  dim3 grid((unsigned)((m * k / 4 + 255) / 256));
  if (bf16)
    hipLaunchKernelGGL(load_working_kernel<1>, grid, dim3(256), 0, s, W, m, k, ldw, Wp);
  else
    hipLaunchKernelGGL(load_working_kernel<0>, grid, dim3(256), 0, s, W, m, k, ldw, Wp);
  return hipGetLastError();
}

hipError_t inv_diag_launch(const float* U, int64_t k, float* invd, hipStream_t s) {
  hipLaunchKernelGGL(inv_diag_kernel, dim3((unsigned)((k + 255) / 256)), dim3(256), 0, s, U, k, invd);
  return hipGetLastError();
}

hipError_t load_working_copy_f64(const void* W, int bf16, int64_t m, int64_t k, int64_t ldw, double* Wp,
                                 hipStream_t s) {
  dim3 grid((unsigned)((m * k + 255) / 256));
  if (bf16)
    hipLaunchKernelGGL(load_working_f64_kernel<1>, grid, dim3(256), 0, s, W, m, k, ldw, Wp);
  else
    hipLaunchKernelGGL(load_working_f64_kernel<0>, grid, dim3(256), 0, s, W, m, k, ldw, Wp);
  return hipGetLastError();
}

hipError_t sweep_batch_launch(float* Wp, const float* U, const float* invd, const float* g, int64_t m, int64_t k,
                              int i1, int ncols, int n_cand, bool indep, uint8_t* codes, uint8_t* scales,
                              float* Eslab, int64_t lde, float* row_loss, hipStream_t s) {
  return sweep_launch_t<float>(Wp, U, invd, g, m, k, i1, ncols, n_cand, indep, codes, scales, Eslab, lde, row_loss, s);
}
hipError_t sweep_batch_launch_f64(double* Wp, const float* U, const float* g, int64_t m, int64_t k, int i1,
                                  int ncols, int n_cand, bool indep, uint8_t* codes, uint8_t* scales, double* Eslab,
                                  int64_t lde, float* row_loss, hipStream_t s) {
  return sweep_launch_t<double>(Wp, U, U, g, m, k, i1, ncols, n_cand, indep, codes, scales, Eslab, lde, row_loss, s);
}

hipError_t delta_w_launch(const void* W, int bf16, int64_t m, int64_t k, int64_t ldw, const uint8_t* codes,
                          const uint8_t* scales, const float* g, float* dW, hipStream_t s, int64_t c0, int64_t c1) {
  if (c1 < 0) c1 = k;
  const int64_t blk0 = c0 / kBlock, nblk = (c1 - c0) / kBlock;
  if (m <= 0 || nblk <= 0) return hipSuccess;
  dim3 grid((unsigned)((m * nblk + 255) / 256));
  if (bf16)
    hipLaunchKernelGGL(delta_w_kernel<1>, grid, dim3(256), 0, s, W, m, k, ldw, codes, scales, g, dW, blk0, nblk);
  else
    hipLaunchKernelGGL(delta_w_kernel<0>, grid, dim3(256), 0, s, W, m, k, ldw, codes, scales, g, dW, blk0, nblk);
  return hipGetLastError();
}

hipError_t row_sum_launch(const float* P, int64_t m, int64_t np, float* out, hipStream_t s) {
  hipLaunchKernelGGL(row_sum_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, s, P, m, np, out);
  return hipGetLastError();
}

hipError_t fill_f32(float* p, int64_t n, float v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

}  // namespace nvq
