// Shared device helpers of the NVFP4 quantizer (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 16;       // weights per E4M3 scale
constexpr int kBatch = 128;      // lazy-batch width of the GPTQ sweep
constexpr int kE4m3MaxCode = 0x7E;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (inputs are finite here).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------
// NVFP4 codec.  E4M3 (FN): bias 7, exponent field 0 is subnormal (m * 2^-9),
// 0x7E = 448 is the largest finite value.  E2M1 magnitudes by index:
// 0, 0.5, 1, 1.5, 2, 3, 4, 6.
//
// Every rounding decision compares a magnitude |w| with t * s * g, where t is
// a midpoint of one of the grids (at most 7 significant bits together with
// s) and g the fp32 tensor scale.  t * s is exact in fp32, and the sign of
// fmaf(-(t * s), g, |w|) is the sign of the exact difference, so decisions are
// those of exact real arithmetic (denormals must not be flushed).
// ---------------------------------------------------------------------------

// Value of a non-negative E4M3 code 0..126 (exact).
__device__ __forceinline__ float e4m3_value(int c) {
  int e = c >> 3, m = c & 7;
  return e == 0 ? (float)m * 0x1p-9f : __uint_as_float((uint32_t)(e + 120) << 23 | (uint32_t)m << 20);
}
// The same value with both forms evaluated and one selected: c 2^-9 for the
// subnormal codes c < 8, else the float bits (c << 20) + (120 << 23).  Where
// it is evaluated per block ahead of the element loop (the scale search and
// encode) this compiles without branches; the dequantization kernel keeps
// the form above, which schedules better there.
__device__ __forceinline__ float e4m3_value_sel(int c) {
  const float nrm = __uint_as_float(((uint32_t)c << 20) + (120u << 23));
  const float sub = (float)c * 0x1p-9f;
  return c < 8 ? sub : nrm;
}

// Code of the E4M3 value nearest to the real quotient a / (6 g), ties to the
// even code, saturating at 0x7E.  a >= 0.  Binary search over the 126
// midpoints m_i = (v_i + v_{i+1}) / 2; a passes midpoint i when a > 6 m_i g,
// or a >= 6 m_i g when i is odd (the tie then rounds up to the even code i+1).
__device__ __forceinline__ int e4m3_code_of_ratio(float a, float g) {
  int lo = 0, hi = kE4m3MaxCode;           // answer in [lo, hi]
#pragma unroll
  for (int it = 0; it < 7; ++it) {
    int mid = (lo + hi) >> 1;              // test midpoint between mid and mid+1
    if (lo >= hi) break;
    float six_m = 3.0f * (e4m3_value_sel(mid) + e4m3_value_sel(mid + 1));   // 6 * m_i, exact
    float d = fmaf(-six_m, g, a);
    bool pass = (mid & 1) ? (d >= 0.0f) : (d > 0.0f);
    if (pass) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// Magnitude index (0..7) of the E2M1 value nearest to |w| / (s g), ties to the
// even index, clipped at 6.  aw = |w|, s = E4M3 block-scale value.
__device__ __forceinline__ int e2m1_index(float aw, float s, float g) {
  int idx = 0;
  idx += fmaf(-0.25f * s, g, aw) > 0.0f;
  idx += fmaf(-0.75f * s, g, aw) >= 0.0f;
  idx += fmaf(-1.25f * s, g, aw) > 0.0f;
  idx += fmaf(-1.75f * s, g, aw) >= 0.0f;
  idx += fmaf(-2.50f * s, g, aw) > 0.0f;
  idx += fmaf(-3.50f * s, g, aw) >= 0.0f;
  idx += fmaf(-5.00f * s, g, aw) > 0.0f;
  return idx;
}

// The E2M1 magnitude index e2m1_index returns, found by a three-level search
// over the midpoints instead of seven tests: the first two levels test odd
// midpoints (a tie rounds up to the even index), the last an even one (a tie
// rounds down).  ts[i] = t_i * s for the midpoints t = 0.25, 0.75, 1.25,
// 1.75, 2.5, 3.5, 5 (exact products); each test is the sign of an fma, as in
// e2m1_index.
// (The selections are bit masks: written as conditionals they became branches.)
__device__ __forceinline__ float pick(uint32_t mask, float a, float b) {   // mask ? a : b, mask all ones or zero
  return __uint_as_float((__float_as_uint(a) & mask) | (__float_as_uint(b) & ~mask));
}
__device__ __forceinline__ int e2m1_index_search(float aw, float g, const float (&ts)[7]) {
  const uint32_t m2 = 0u - (uint32_t)(fmaf(-ts[3], g, aw) >= 0.0f);
  const uint32_t m1 = 0u - (uint32_t)(fmaf(-pick(m2, ts[5], ts[1]), g, aw) >= 0.0f);
  const float t0 = pick(m1, pick(m2, ts[6], ts[2]), pick(m2, ts[4], ts[0]));
  const uint32_t b0 = fmaf(-t0, g, aw) > 0.0f;
  return (int)((m2 & 4u) | (m1 & 2u) | b0);
}

// The same index from one exact test.  q2 ~ 2 aw / (s g) (any relative
// error under 10% will do) picks the midpoint t_j nearest to aw / (s g):
// j = floor(min(q2, q2 / 2 + 2, 6.5)) switches from j to j + 1 at 0.5, 1,
// 1.5, 2, 3 and 4, each well inside the gap between t_j and t_{j+1}
// (midpoints 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5).  So aw / (s g) lies
// between t_{j-1} and t_{j+1}, and the index is j, or j + 1 when aw passes
// t_j: the sign of fma(-t_j s, g, aw) as in e2m1_index (t_j s is exact:
// 8 t_j = 2, 6, 10, 14, 20, 28, 40 from a byte table, times s8 = s / 8).
// (The byte is selected by j alone: the other result bytes are ignored.)
// The tie rule rides on the integer view of that difference d: a positive
// float is an integer >= 1, +0 is 0 and every negative float (-0 too) is
// negative, so "d > 0" is int(d) > 0 and "d >= 0" (odd midpoints, ties round
// up) is int(d) > -1: both are int(d) > -(j & 1), in signed arithmetic.
__device__ __forceinline__ int e2m1_index_nearest(float aw, float q2, float g, float s8) {
  const int j = (int)fminf(fminf(q2, fmaf(0.5f, q2, 2.0f)), 6.5f);
  const float t8 = (float)(__builtin_amdgcn_perm(0x00281C14u, 0x0E0A0602u, (uint32_t)j) & 0xFFu);
  const float d = fmaf(-(t8 * s8), g, aw);
  return j + (int)(__float_as_int(d) > -(j & 1));
}
// q2 = aw * r2 with r2 = 2 / (s g) needs that quotient finite: g at least
// this for every scale s >= 2^-9 (below it the search above is used).
constexpr float kNearestMinG = 0x1p-100f;

// Twice the E2M1 magnitude of index idx: 0,1,2,3,4,6,8,12 packed in nibbles.
__device__ __forceinline__ float e2m1_twice_mag(int idx) {
  return (float)((0xC8643210u >> (4 * idx)) & 0xFu);
}

// Signed dequantized value fl32(e2m1 * s * g): the first product is exact.
__device__ __forceinline__ float e2m1_dequant(int code4, float s, float g) {
  float m = e2m1_twice_mag(code4 & 7) * 0.5f * s;
  float v = m * g;
  return (code4 & 8) ? -v : v;
}

// 4-bit code of w under scale s * g (zero is +0).
__device__ __forceinline__ int e2m1_encode(float w, float s, float g) {
  int idx = e2m1_index(fabsf(w), s, g);
  return (idx != 0 && w < 0.0f) ? (idx | 8) : idx;
}

// fp64 working values: every threshold t * s * g (t * s at most 7 significant
// bits, g 24) is exact in fp64, so plain comparisons are exact.
__device__ __forceinline__ int e4m3_code_of_ratio(double a, float g) {
  int lo = 0, hi = kE4m3MaxCode;
#pragma unroll
  for (int it = 0; it < 7; ++it) {
    int mid = (lo + hi) >> 1;
    if (lo >= hi) break;
    double thr = (double)(3.0f * (e4m3_value_sel(mid) + e4m3_value_sel(mid + 1))) * (double)g;
    bool pass = (mid & 1) ? (a >= thr) : (a > thr);
    if (pass) lo = mid + 1; else hi = mid;
  }
  return lo;
}
__device__ __forceinline__ int e2m1_index(double aw, float s, float g) {
  const double sg = (double)s * (double)g;
  int idx = 0;
  idx += aw > 0.25 * sg;
  idx += aw >= 0.75 * sg;
  idx += aw > 1.25 * sg;
  idx += aw >= 1.75 * sg;
  idx += aw > 2.50 * sg;
  idx += aw >= 3.50 * sg;
  idx += aw > 5.00 * sg;
  return idx;
}
__device__ __forceinline__ int e2m1_encode(double w, float s, float g) {
  int idx = e2m1_index(fabs(w), s, g);
  return (idx != 0 && w < 0.0) ? (idx | 8) : idx;
}
// Exact signed value e2m1 * s * g in fp64.
__device__ __forceinline__ double e2m1_dequant_f64(int code4, float s, float g) {
  double v = (double)(e2m1_twice_mag(code4 & 7) * 0.5f * s) * (double)g;
  return (code4 & 8) ? -v : v;
}

// Workgroup barrier for LDS double buffering: waits for this wave's LDS
// (and scalar) operations only, then joins the barrier, so every wave's LDS
// writes before it are visible to every wave after it, while global loads
// issued ahead stay in flight (__syncthreads would wait for those too).  The
// memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt 63 and expcnt 7 (no wait)
  asm volatile("s_barrier" ::: "memory");
}

// ---- the same decisions with shorter dependency chains (the sweep's inner loop) ----
// Whether a passes the midpoint between E4M3 codes i and i+1 (the binary
// search's test above); never past the last code.
// (Branch-free: i <= 126, and e4m3_value is defined on 127.)
__device__ __forceinline__ bool e4m3_passes(float a, float g, int i) {
  const float d = fmaf(-3.0f * (e4m3_value_sel(i) + e4m3_value_sel(i + 1)), g, a);
  return i < kE4m3MaxCode && ((i & 1) ? d >= 0.0f : d > 0.0f);
}
__device__ __forceinline__ bool e4m3_passes(double a, float g, int i) {
  const double thr = (double)(3.0f * (e4m3_value_sel(i) + e4m3_value_sel(i + 1))) * (double)g;
  return i < kE4m3MaxCode && ((i & 1) ? a >= thr : a > thr);
}
// E4M3 code whose value is at or just below q >= 0, from q's bits (q may be
// approximate or infinite; clamped to [0, 126]).
// (Both forms are evaluated and one selected; the product is clamped before
// its conversion, so that it stays in range for every q.)
__device__ __forceinline__ int e4m3_code_below(float q) {
  const int sub = (int)fminf(q * 512.0f, 8.0f);
  const int nrm = (int)(__float_as_uint(q) >> 20) - 960;   // (exponent - 120) * 8 + top mantissa bits
  return min(max(q < 0x1p-6f ? sub : nrm, 0), kE4m3MaxCode);
}
// The code e4m3_code_of_ratio returns, from one exact test.  The grid code
// i at or below an approximate quotient q = a r6g (r6g ~ 1 / (6 g), a few
// ulps off) names the midpoint m_i nearest to q; grid steps are >= 1/16
// relative, so the exact quotient lies between m_{i-1} and m_{i+1}, and the
// code is i, or i + 1 when a passes m_i (never past the last code).
template <typename T>
__device__ __forceinline__ int e4m3_code_of_ratio_fast(T a, float g, float r6g) {
  const int i = e4m3_code_below((float)a * r6g);
  return i + (int)e4m3_passes(a, g, i);
}
// The quotient above is only that close while 1 / (6 g) is a finite normal
// float; below this g (weights under ~1e-35) the binary search is used.
constexpr float kFastRatioMinG = 0x1p-120f;
template <typename T>
__device__ __forceinline__ int e4m3_code_of_ratio_any(T a, float g, float r6g) {
  return g >= kFastRatioMinG ? e4m3_code_of_ratio_fast(a, g, r6g) : e4m3_code_of_ratio(a, g);
}

// First of the n_cand consecutive candidate codes around c0, inside [1, 126].
__device__ __forceinline__ int candidate_lo(int c0, int n_cand) {
  int lo = c0 - (n_cand >> 1);
  lo = lo < 1 ? 1 : lo;
  int top = kE4m3MaxCode - n_cand + 1;
  return lo > top ? top : lo;
}

}  // namespace nvq
