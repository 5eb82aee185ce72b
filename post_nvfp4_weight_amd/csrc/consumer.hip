// NVFP4 weight-only GEMM, the consumer of the exported weights:
//   Y = X dequant(W)^T, X bf16 [T x k] activations, W NVFP4 [m x k].
//
// An element without the per-tensor scale, e2m1 * e4m3, has at most 6
// significant bits and is exact in bf16.  So the kernel expands codes and
// block scales to bf16 as it stages a weight tile into LDS, multiplies on the
// bf16 matrix cores (v_mfma_f32_32x32x16_bf16, exact products, fp32
// accumulation) and applies g once to the result: Y = g (X Q^T) with
// Q = e2m1 * e4m3.  Against X fl32(Q g)^T this differs by at most 2^-24 of
// each product.
//
// Three kernels share this: a decode-sized one for at most 32 tokens, a
// large-tile one when there is a 256 x 256 tile per CU (both further below),
// and the general one.  Its tiles are 128 (tokens) x 128 (output channels),
// four waves of 64 x 64, k in steps of 64 (four NVFP4 blocks); both operands
// are kept [row][k] in LDS (k contiguous, rows padded to 72 elements) and
// double-buffered; the next step's loads are in flight while the current
// step is multiplied.
#include <algorithm>

#include <mutex>

#include "common.h"
#include "kernels.h"

namespace nvq {

namespace {

constexpr int CT = 128, CK = 64, CLD = CK + 8;
constexpr int CBUF = 2 * CT * CLD;   // bf16 elements of one buffer: X tile, then Q tile

typedef float f32x2c __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2c __attribute__((ext_vector_type(2)));

// Byte B of word (two codes, low nibble first) under block scale value s ->
// packed bf16 pair of e2m1 * s.  The E2M1 decode is the hardware's FP4
// conversion at scale 1 (its scale operand applies only a power of two, so
// the E4M3 scale is multiplied in fp32; the product has at most 6
// significant bits and is exact, as is its bf16 conversion).
// E4M3 value of code c (0..126) without branches: (m + 8 min(e, 1)) 2^(max(e, 1) - 10)
// for c = 8 e + m, which is m 2^-9 for e = 0 and (1 + m/8) 2^(e-7) otherwise.
__device__ __forceinline__ float scale_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15, m = c & 7;
  return (float)(m + 8 * min(e, 1u)) * __uint_as_float((max(e, 1u) + 117) << 23);
}

template <int B>
__device__ __forceinline__ uint32_t dq_byte(uint32_t word, float s) {
  const f32x2c v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, B);
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2c{v.x * s, v.y * s}, bf16x2c));
}
__device__ __forceinline__ uint32_t dq_byte(uint32_t word, float s, int b) {   // b known after unrolling
  switch (b) {
    case 0: return dq_byte<0>(word, s);
    case 1: return dq_byte<1>(word, s);
    case 2: return dq_byte<2>(word, s);
    default: return dq_byte<3>(word, s);
  }
}

// OUT: 0 fp32 Y, 1 bf16 Y, 2 fp32 partial sums of k-split blockIdx.z (no g)
// at P + z * T * m.  ksplit: k per split (a multiple of CK).
template <int OUT>
__global__ __launch_bounds__(256) void nvfp4_gemm_kernel(const uint16_t* __restrict__ X, int64_t T, int64_t k,
                                                         int64_t ldx, const uint8_t* __restrict__ codes,
                                                         const uint8_t* __restrict__ scales,
                                                         const float* __restrict__ gptr, int64_t m,
                                                         void* __restrict__ Y, int64_t ldy, int64_t ksplit) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * CBUF];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int64_t t0 = (int64_t)blockIdx.y * CT, o0 = (int64_t)blockIdx.x * CT;
  const int64_t kb = k / 16;   // blocks per weight row

  // Per step: X 128 rows x 64 k = 4 x 16 B per thread; W 128 rows x 4 blocks
  // = 2 blocks (8 B of codes + 2 scale bytes) per thread.
  const int wrow = tid >> 1, wh = tid & 1;
  auto load = [&](int64_t k0, u32x4 (&xv)[4], u32x2 (&cv)[2], uint32_t (&sv)[2]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = q * 256 + tid, r = e >> 3, c8 = (e & 7) * 8;
      xv[q] = *(const u32x4*)(X + min(t0 + r, T - 1) * ldx + min(k0 + c8, k - 8));
    }
    const int64_t row = min(o0 + wrow, m - 1);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t blk = min(k0 / 16 + 2 * wh + b, kb - 1);
      cv[b] = *(const u32x2*)(codes + row * (k / 2) + blk * 8);
      sv[b] = scales[row * kb + blk];
    }
  };
  auto store = [&](uint16_t* buf, int64_t k0, const u32x4 (&xv)[4], const u32x2 (&cv)[2], const uint32_t (&sv)[2]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = q * 256 + tid, r = e >> 3, c8 = (e & 7) * 8;
      const bool ok = t0 + r < T && k0 + c8 < k;
      *(u32x4*)(buf + r * CLD + c8) = ok ? xv[q] : u32x4{0u, 0u, 0u, 0u};
    }
    uint16_t* qb = buf + CT * CLD;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const bool ok = o0 + wrow < m && k0 + 32 * wh + 16 * b < k;
      const float sb = scale_value(sv[b] & 0x7F);
      const uint32_t keep = ok ? ~0u : 0u;   // a mask, so that nothing branches
      u32x4 lo, hi;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        lo[j] = dq_byte(cv[b][0], sb, j) & keep;
        hi[j] = dq_byte(cv[b][1], sb, j) & keep;
      }
      *(u32x4*)(qb + wrow * CLD + 32 * wh + 16 * b) = lo;
      *(u32x4*)(qb + wrow * CLD + 32 * wh + 16 * b + 8) = hi;
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int64_t kbeg = (int64_t)blockIdx.z * ksplit, kend = min(k, kbeg + ksplit);
  const int64_t nsteps = (kend - kbeg + CK - 1) / CK;
  u32x4 xv[4];
  u32x2 cv[2];
  uint32_t sv[2];
  load(kbeg, xv, cv, sv);
  store(smem, kbeg, xv, cv, sv);
  __syncthreads();
  const int arow = wr * 64 + (lane & 31), brow = wc * 64 + (lane & 31), koff = 8 * (lane >> 5);
  for (int64_t st = 0; st < nsteps; ++st) {
    const int cur = (int)(st & 1);
    if (st + 1 < nsteps) load(kbeg + (st + 1) * CK, xv, cv, sv);
    const uint16_t* Xs = smem + cur * CBUF;
    const uint16_t* Qs = Xs + CT * CLD;
#pragma unroll
    for (int ks = 0; ks < CK; ks += 16) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        a[t] = *(const bf16x8*)(Xs + (arow + 32 * t) * CLD + ks + koff);
        b[t] = *(const bf16x8*)(Qs + (brow + 32 * t) * CLD + ks + koff);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (st + 1 < nsteps) store(smem + (cur ^ 1) * CBUF, kbeg + (st + 1) * CK, xv, cv, sv);
    __syncthreads();
  }

  // Accumulator layout: lane l, register r -> row 8 (r/4) + 4 (l/32) + r%4, column l%32.
  const float g = OUT == 2 ? 1.0f : *gptr;
  float* P = (float*)Y + (OUT == 2 ? (int64_t)blockIdx.z * T * m : 0);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = t0 + wr * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t col = o0 + wc * 64 + j * 32 + (lane & 31);
        if (row < T && col < m) {
          const float v = acc[i][j][r] * g;
          if (OUT == 1) ((__bf16*)Y)[row * ldy + col] = (__bf16)v;
          else if (OUT == 0) ((float*)Y)[row * ldy + col] = v;
          else P[row * m + col] = v;
        }
      }
}

// Y = g * (sum of the splits in split order).
template <bool OUT_BF16>
__global__ void nvfp4_gemm_reduce_kernel(const float* __restrict__ P, int nsplit, int64_t T, int64_t m,
                                         const float* __restrict__ gptr, void* __restrict__ Y, int64_t ldy) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= T * m) return;
  float s = 0.0f;
  for (int z = 0; z < nsplit; ++z) s += P[(int64_t)z * T * m + e];
  const float v = s * *gptr;
  const int64_t row = e / m, col = e % m;
  if (OUT_BF16) ((__bf16*)Y)[row * ldy + col] = (__bf16)v;
  else ((float*)Y)[row * ldy + col] = v;
}

// ---- few tokens (T <= 32): decode-sized products ------------------------------
// These are bound by reading the weights once, so the loads are spread wide
// and issued together.  A workgroup of 16 waves takes 16 output channels over
// all of k (k a multiple of 128); wave w takes chunks w, w + 16, ... of 128 k,
// two at a time.  v_mfma_f32_16x16x32_bf16: A = 16 tokens x 32 k, B = 32 k x
// 16 channels.  In a chunk, lane (c = l % 16, q = l / 16) supplies the 32
// consecutive k 32 q .. 32 q + 31 of the chunk over its four MFMAs, 8 per
// MFMA, for channel c (B) and token c of each 16-token group (A): both
// operands take the same k, so the four MFMAs sum every k of the chunk once
// (the order of the k inside a sum is free).  A lane's 32 codes are one
// 16-byte load and its two block scales one 2-byte load.  The waves' 16 x 16
// partial tiles are summed in wave order through LDS.
constexpr int GV_W = 16;   // waves per workgroup
typedef float f32x4c __attribute__((ext_vector_type(4)));
template <int NTG, int OUT>
__global__ __launch_bounds__(1024) void nvfp4_gemv_kernel(const uint16_t* __restrict__ X, int64_t T, int64_t k,
                                                          int64_t ldx, const uint8_t* __restrict__ codes,
                                                          const uint8_t* __restrict__ scales,
                                                          const float* __restrict__ gptr, int64_t m,
                                                          void* __restrict__ Y, int64_t ldy) {
  __shared__ float red[GV_W][NTG][16][17];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, q = lane >> 4;
  const int64_t o0 = (int64_t)blockIdx.x * 16;
  const int64_t orow = min(o0 + c, m - 1);
  const int64_t nch = k / 128;
  f32x4c acc[NTG];
#pragma unroll
  for (int tg = 0; tg < NTG; ++tg) acc[tg] = f32x4c{0.f, 0.f, 0.f, 0.f};
  for (int64_t base = wave; base < nch; base += 2 * GV_W) {
    u32x4 cw[2], xa[2][NTG][4];
    uint32_t sw[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t ch = base + u * GV_W;
      const bool ok = ch < nch;
      const int64_t kk = (ok ? ch : 0) * 128 + 32 * q;   // the lane's first k in the chunk
      cw[u] = ok ? *(const u32x4*)(codes + orow * (k / 2) + kk / 2) : u32x4{0u, 0u, 0u, 0u};
      sw[u] = ok ? (uint32_t)*(const uint16_t*)(scales + orow * (k / 16) + kk / 16) : 0u;
#pragma unroll
      for (int tg = 0; tg < NTG; ++tg) {
        const int64_t t = tg * 16 + c;
        const bool tok = ok && t < T;
        const uint16_t* xr = X + min(t, T - 1) * ldx + kk;
#pragma unroll
        for (int j = 0; j < 4; ++j) xa[u][tg][j] = tok ? *(const u32x4*)(xr + 8 * j) : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // codes of k 8 j .. 8 j + 7 of the lane's 32, under the scale of their 16-block
        const float sc = scale_value((j < 2 ? sw[u] : sw[u] >> 8) & 0x7F);
        const uint32_t w = cw[u][j];
        const u32x4 bq{dq_byte<0>(w, sc), dq_byte<1>(w, sc), dq_byte<2>(w, sc), dq_byte<3>(w, sc)};
        const bf16x8 b = __builtin_bit_cast(bf16x8, bq);
#pragma unroll
        for (int tg = 0; tg < NTG; ++tg)
          acc[tg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[u][tg][j]), b, acc[tg],
                                                            0, 0, 0);
      }
  }
  // Accumulator register r of lane l: token 4 (l / 16) + r, channel l % 16.
#pragma unroll
  for (int tg = 0; tg < NTG; ++tg)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][tg][4 * q + r][c] = acc[tg][r];
  __syncthreads();
  if (tid < NTG * 256) {
    const int tg = tid >> 8, rr = (tid >> 4) & 15, cc = tid & 15;
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < GV_W; ++w) sum += red[w][tg][rr][cc];
    const int64_t t = tg * 16 + rr, o = o0 + cc;
    if (t < T && o < m) {
      const float v = sum * *gptr;
      if (OUT == 1) ((__bf16*)Y)[t * ldy + o] = (__bf16)v;
      else ((float*)Y)[t * ldy + o] = v;
    }
  }
}

// ---- many tokens: 256 x 256 tiles ----------------------------------------------
// 256 (tokens) x 256 (output channels) per workgroup, four waves of 128 x 128
// (16 accumulators of 32 x 32), k in steps of 32 (k a multiple of 32).  A wave
// reads 8 operand fragments per 16 products, half the LDS reads per product
// of the 64 x 64 wave tiles above.
//
// X goes to LDS by direct-to-LDS buffer loads, issued two steps ahead into a
// ring of three X buffers: 256 rows of 64 bytes, 16-byte chunks XOR-swizzled
// by (row / 2) % 4, so that the 8 lanes of each fragment-read group hit
// distinct banks.  Rows past T read as zeros (the buffer bound).  The codes
// and scales of a step are loaded into registers three steps ahead (two
// register sets) and expanded to bf16 into one of two Q buffers, in small
// pieces placed between the products.
constexpr int BT = 256, BK = 32, BLD = BK + 8;
constexpr int BXBUF = BT * BK;     // bf16 elements of one X buffer (64-byte rows, no padding)
constexpr int BQBUF = BT * BLD;    // bf16 elements of one Q buffer (rows padded to 80 bytes)

__device__ __forceinline__ int bswz(int row, int c) { return c ^ ((row >> 1) & 3); }

template <int OUT>   // 0 fp32 Y, 1 bf16 Y
__global__ __launch_bounds__(256) void nvfp4_gemm_big_kernel(const uint16_t* __restrict__ X, int64_t T, int64_t k,
                                                             int64_t ldx, const uint8_t* __restrict__ codes,
                                                             const uint8_t* __restrict__ scales,
                                                             const float* __restrict__ gptr, int64_t m,
                                                             void* __restrict__ Y, int64_t ldy) {
  __shared__ __attribute__((aligned(1024))) uint16_t smem[3 * BXBUF + 2 * BQBUF];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int64_t t0 = (int64_t)blockIdx.y * BT, o0 = (int64_t)blockIdx.x * BT;
  const int64_t kb = k / 16;
  const int64_t nsteps = k / BK;
  uint16_t* const xbuf = smem;
  uint16_t* const qbuf = smem + 3 * BXBUF;

  // Direct-to-LDS loads: this wave's instruction q fills bytes [1024 i, 1024 (i+1))
  // of an X buffer, i = wave + 4 q: rows 16 i + lane / 4, physical chunk lane % 4.
  uint32_t voff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = wave + 4 * q, row = 16 * i + (lane >> 2);
    voff[q] = (uint32_t)(row * ldx * 2 + bswz(row, lane & 3) * 16);
  }
  const int64_t rows_left = T - t0;
  auto issue_x = [&](int64_t st) {   // step st into its ring buffer; zero-length past the end
#if __HIP_DEVICE_COMPILE__
    const int64_t kk = st < nsteps ? st * BK : 0;
    const int nrec = st < nsteps ? (int)min(rows_left * ldx * 2 - kk * 2, (int64_t)0x7FFFFFF0) : 0;
    __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(X + t0 * ldx + kk), (short)0, nrec, 0x00020000);
    char* dst = (char*)(xbuf + ((int)st % 3) * BXBUF);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + (wave + 4 * q) * 1024),
                                               16, voff[q], 0, 0, 0);
#endif
  };

  // Codes and scales of weight row tid: the two blocks of a step are 16
  // aligned bytes of codes and 2 of scales (k is a multiple of 32); steps
  // past the end are clamped, so that every load is valid.
  const int64_t wrow = min(o0 + tid, m - 1);
  const uint8_t* crow = codes + wrow * (k / 2);
  const uint8_t* srow = scales + wrow * kb;
  const int last = (int)(nsteps - 1);
  auto load_q = [&](int64_t st, u32x2 (&cv)[2], uint32_t (&sv)[2]) {
    const int s2 = min((int)st, last);
    const u32x4 c = *(const u32x4*)(crow + s2 * 16);
    const uint32_t sc = *(const uint16_t*)(srow + s2 * 2);
    cv[0] = u32x2{c[0], c[1]};
    cv[1] = u32x2{c[2], c[3]};
    sv[0] = sc & 0xFF;
    sv[1] = sc >> 8;
  };
  // Piece p (0..7) of expanding step st's codes into Q buffer buf: block p / 4,
  // 8-code half (p / 2) % 2; the first piece of a half expands 4 codes, the
  // second 4 more and stores the 16 bytes.
  auto q_piece = [&](uint16_t* buf, int64_t st, const u32x2 (&cv)[2], const uint32_t (&sv)[2], int p, u32x4& qv) {
    const int b = p >> 2, h = (p >> 1) & 1, part = p & 1;
    const uint32_t keep = (o0 + tid < m && st < nsteps) ? ~0u : 0u;   // a mask, so that nothing branches
    const float sb = scale_value(sv[b] & 0x7F);
    const uint32_t word = cv[b][h];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int jj = 2 * part + j;
      qv[jj] = dq_byte(word, sb, jj) & keep;
    }
    if (part == 1) *(u32x4*)(buf + tid * BLD + 16 * b + 8 * h) = qv;
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  u32x2 cv0[2], cv1[2];
  uint32_t sv0[2], sv1[2];
  u32x4 qv;
  issue_x(0);
  issue_x(1);
  load_q(0, cv0, sv0);
#pragma unroll
  for (int p = 0; p < 8; ++p) q_piece(qbuf, 0, cv0, sv0, p, qv);
  load_q(1, cv0, sv0);
  load_q(2, cv1, sv1);
  __syncthreads();   // waits for every load so far, X steps 0 and 1 included

  const int arow = wr * 128 + (lane & 31), brow = wc * 128 + (lane & 31), kc = lane >> 5;
  // Per step st: 4 loads of X step st+2 (first), 4 loads of codes step st+3
  // (product 20).  At the end, X step st+1 must have landed: after it were
  // issued the codes of st+2, X of st+2 and the codes of st+3, 12 loads.
  auto body = [&](const uint16_t* __restrict__ Xs, const uint16_t* __restrict__ Qs, uint16_t* __restrict__ nq,
                  int64_t st, u32x2 (&cv)[2], uint32_t (&sv)[2]) {
    bf16x8 a[2][4], b[2][4];
    auto read = [&](int h, int f) {
      if (f < 4) {
        const int r = arow + 32 * f;
        a[h][f] = *(const bf16x8*)(Xs + r * BK + bswz(r, 2 * h + kc) * 8);
      } else {
        b[h][f - 4] = *(const bf16x8*)(Qs + (brow + 32 * (f - 4)) * BLD + 16 * h + 8 * kc);
      }
    };
#pragma unroll
    for (int f = 0; f < 8; ++f) read(0, f);
    // Behind product g: the second k-step's fragment g (g < 8), the X loads
    // of step st+2 (g < 4, one per product), codes piece g - 4 (4 <= g < 12)
    // and, once its register set's last reader has run, the codes of step
    // st+3 (g == 20).
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int mm = 0; mm < 16; ++mm) {
        const int g = 16 * h + mm, i = mm >> 2, j = mm & 3;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[h][i], b[h][j], acc[i][j], 0, 0, 0);
        if (g < 8) read(1, g);
        if (g == 0) issue_x(st + 2);
        if (g >= 4 && g < 12) q_piece(nq, st + 1, cv, sv, g - 4, qv);
        if (g == 20) load_q(st + 3, cv, sv);
        __builtin_amdgcn_sched_barrier(0);
      }
    __builtin_amdgcn_s_waitcnt(12 | (7 << 4) | (0 << 8));   // vmcnt(12), lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
  };
  // Steps go in pairs with no branch between them (a join would make the
  // compiler copy the accumulators): with an odd step count the last pair's
  // second step multiplies zeros (its X rows read past the end as zeros and
  // its codes are masked).
  for (int64_t st = 0; st < nsteps; st += 2) {
    body(xbuf + ((int)st % 3) * BXBUF, qbuf, qbuf + BQBUF, st, cv0, sv0);
    body(xbuf + ((int)st + 1) % 3 * BXBUF, qbuf + BQBUF, qbuf, st + 1, cv1, sv1);
  }
  // The direct-to-LDS loads issued for steps past the end still write LDS
  // (zeros): none may be in flight once the workgroup's LDS is released.
  __builtin_amdgcn_s_waitcnt(0);

  // Accumulator layout: lane l, register r -> row 8 (r/4) + 4 (l/32) + r%4, column l%32.
  const float g = *gptr;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = t0 + wr * 128 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t col = o0 + wc * 128 + j * 32 + (lane & 31);
        if (row < T && col < m) {
          const float v = acc[i][j][r] * g;
          if (OUT == 1) ((__bf16*)Y)[row * ldy + col] = (__bf16)v;
          else ((float*)Y)[row * ldy + col] = v;
        }
      }
}

int num_cus_consumer() {
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
  }
  return cus;
}

// k splits so that the launch has about two workgroups per CU (at most 16,
// and each split at least one k step).
int nvfp4_gemm_splits(int64_t T, int64_t k, int64_t m) {
  const int64_t tiles = ((m + CT - 1) / CT) * ((T + CT - 1) / CT);
  const int64_t steps = (k + CK - 1) / CK;
  int64_t sp = (2 * num_cus_consumer() + tiles - 1) / tiles;
  sp = std::min<int64_t>(std::min<int64_t>(sp, 16), steps);
  return (int)std::max<int64_t>(sp, 1);
}

}  // namespace

// ---- the no-allocation variant's scratch ---------------------------------------
// The k-split partial sums of nvfp4_gemm_noalloc live in this array instead of
// a caller workspace: each device that runs the call holds its own copy until
// the process ends.  Host code never passes the array's name to a kernel (on
// the host it is only a stand-in for the symbol): the device address comes
// from hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = (float*)p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

size_t nvfp4_gemm_workspace(int64_t T, int64_t k, int64_t m) {
  if (T <= 0 || m <= 0 || k <= 0) return 0;
  const int sp = nvfp4_gemm_splits(T, k, m);
  return sp > 1 ? (size_t)sp * T * m * sizeof(float) : 0;
}

hipError_t nvfp4_gemm_launch(const uint16_t* X, int64_t T, int64_t k, int64_t ldx, const uint8_t* codes,
                             const uint8_t* scales, const float* g, int64_t m, void* Y, int out_bf16, int64_t ldy,
                             float* ws, hipStream_t s) {
  if (T <= 0 || m <= 0) return hipSuccess;
  if (T <= 32 && k % 128 == 0 && (uintptr_t)codes % 16 == 0 && (uintptr_t)scales % 2 == 0 &&
      (uintptr_t)X % 16 == 0 && ldx % 8 == 0) {
    // Decode-sized: one workgroup per 16 output channels (no workspace).
    const dim3 grid((unsigned)((m + 15) / 16));
    if (T <= 16) {
      if (out_bf16) hipLaunchKernelGGL((nvfp4_gemv_kernel<1, 1>), grid, dim3(1024), 0, s, X, T, k, ldx, codes, scales, g, m, Y, ldy);
      else hipLaunchKernelGGL((nvfp4_gemv_kernel<1, 0>), grid, dim3(1024), 0, s, X, T, k, ldx, codes, scales, g, m, Y, ldy);
    } else {
      if (out_bf16) hipLaunchKernelGGL((nvfp4_gemv_kernel<2, 1>), grid, dim3(1024), 0, s, X, T, k, ldx, codes, scales, g, m, Y, ldy);
      else hipLaunchKernelGGL((nvfp4_gemv_kernel<2, 0>), grid, dim3(1024), 0, s, X, T, k, ldx, codes, scales, g, m, Y, ldy);
    }
    return hipGetLastError();
  }
  if (k % BK == 0 && (uintptr_t)codes % 16 == 0 && (uintptr_t)scales % 2 == 0 &&
      ((T + BT - 1) / BT) * ((m + BT - 1) / BT) >= num_cus_consumer()) {
    // Enough 256 x 256 tiles for every CU (k a multiple of 32, codes 16-byte and
    // scales 2-byte aligned): the large-tile kernel, no k split.
    dim3 grid((unsigned)((m + BT - 1) / BT), (unsigned)((T + BT - 1) / BT));
    if (out_bf16)
      hipLaunchKernelGGL(nvfp4_gemm_big_kernel<1>, grid, dim3(256), 0, s, X, T, k, ldx, codes, scales, g, m, Y, ldy);
    else
      hipLaunchKernelGGL(nvfp4_gemm_big_kernel<0>, grid, dim3(256), 0, s, X, T, k, ldx, codes, scales, g, m, Y, ldy);
    return hipGetLastError();
  }
  const int sp = nvfp4_gemm_splits(T, k, m);
  const int64_t steps = (k + CK - 1) / CK;
  const int64_t ksplit = ((steps + sp - 1) / sp) * CK;
  const int nz = (int)((k + ksplit - 1) / ksplit);
  dim3 grid((unsigned)((m + CT - 1) / CT), (unsigned)((T + CT - 1) / CT), (unsigned)nz);
  if (nz > 1) {
    hipLaunchKernelGGL(nvfp4_gemm_kernel<2>, grid, dim3(256), 0, s, X, T, k, ldx, codes, scales, g, m, (void*)ws,
                       ldy, ksplit);
    const dim3 rg((unsigned)((T * m + 255) / 256));
    if (out_bf16)
      hipLaunchKernelGGL(nvfp4_gemm_reduce_kernel<true>, rg, dim3(256), 0, s, ws, nz, T, m, g, Y, ldy);
    else
      hipLaunchKernelGGL(nvfp4_gemm_reduce_kernel<false>, rg, dim3(256), 0, s, ws, nz, T, m, g, Y, ldy);
  } else if (out_bf16) {
    hipLaunchKernelGGL(nvfp4_gemm_kernel<1>, grid, dim3(256), 0, s, X, T, k, ldx, codes, scales, g, m, Y, ldy, ksplit);
  } else {
    hipLaunchKernelGGL(nvfp4_gemm_kernel<0>, grid, dim3(256), 0, s, X, T, k, ldx, codes, scales, g, m, Y, ldy, ksplit);
  }
  return hipGetLastError();
}

}  // namespace nvq
