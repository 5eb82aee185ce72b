// fp32 GEMMs on CDNA4 matrix cores: v_mfma_f32_32x32x2_f32, and for large
// non-transposed products the bf16 matrix cores with operands split into
// three bf16 parts (gemm_x6_kernel below).
//
// One 256-thread workgroup computes a 128x128 tile of C; its four waves hold
// 64x64 sub-tiles as 2x2 MFMA 32x32 accumulators.  Launches that would give
// fewer than two such tiles per CU use 64x64 tiles (one 32x32 accumulator
// per wave) instead.  K is consumed in chunks of
// 32 staged through two LDS buffers (the next chunk is loaded into registers
// while the current one is multiplied).  Used for the GPTQ trailing
// update, the Cholesky panel/trailing updates, the triangular inverse and the
// weighted error (row-dot epilogue).
#include "common.h"
#include "kernels.h"

namespace nvq {

namespace {

constexpr int BK = 32;
// LDS layouts.  An operand whose k index is contiguous in memory is kept as
// [row][BK + 1] (scalar stores; the odd stride makes both the stores and the
// MFMA reads of 32 consecutive rows conflict free); one whose row index is
// contiguous is kept as [BK][T + 4] (16-byte stores, conflict-free reads).
// T is the tile edge: 128, or 64 for launches that would otherwise leave
// most CUs idle.
constexpr int KSTRIDE = BK + 1;           // [row][k] layout
template <int T> struct TileCfg {
  static constexpr int RSTRIDE = T + 4;                       // [k][row] layout
  static constexpr int OPER = T * KSTRIDE > BK * RSTRIDE ? T * KSTRIDE : BK * RSTRIDE;
  static constexpr int LQ = T * BK / 4 / 256;                  // float4 per thread per operand tile
  static constexpr int NI = T / 64;                            // 32x32 accumulators per wave per dimension
};

// Global -> registers for one operand tile of T rows x BK k-values.
// kmajor: element (r, kk) at src[r * ld + kk] (k contiguous); otherwise at
// src[kk * ld + r] (rows contiguous).
template <int T, bool KMAJOR>
__device__ __forceinline__ void load_tile(const float* __restrict__ src, int64_t ld, int64_t r0, int64_t nrows,
                                          int64_t k0, int64_t K, int tid, f32x4 (&v)[TileCfg<T>::LQ]) {
#pragma unroll
  for (int q = 0; q < TileCfg<T>::LQ; ++q) {
    int e = q * 256 + tid;
    // Unconditional loads from clamped addresses (so that all of them are
    // in flight together), zeroed outside the matrix afterwards.
    if (KMAJOR) {
      int r = e >> 3, kk = (e & 7) * 4;            // 8 lanes cover 32 k of a row
      int64_t gr = r0 + r, gk = k0 + kk;
      const f32x4 t = *(const f32x4*)(src + min(gr, nrows - 1) * ld + min(gk, K - 4));
      v[q] = (gr < nrows && gk < K) ? t : f32x4{0.f, 0.f, 0.f, 0.f};
    } else {
      int kk = e / (T / 4), r = (e % (T / 4)) * 4;   // T/4 lanes cover the T rows of a k
      int64_t gr = r0 + r, gk = k0 + kk;
      const f32x4 t = *(const f32x4*)(src + min(gk, K - 1) * ld + min(gr, nrows - 4));
      v[q] = (gr < nrows && gk < K) ? t : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
}

// B' = 2 triu(B, 1) + diag(B) on a B tile (k-index k0 + kk, column n0 + r).
template <int T, bool KMAJOR>
__device__ __forceinline__ void sym_upper(f32x4 (&v)[TileCfg<T>::LQ], int tid, int64_t k0, int64_t n0) {
#pragma unroll
  for (int q = 0; q < TileCfg<T>::LQ; ++q) {
    const int e = q * 256 + tid;
    const int r = KMAJOR ? e >> 3 : (e % (T / 4)) * 4, kk = KMAJOR ? (e & 7) * 4 : e / (T / 4);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t kg = k0 + kk + (KMAJOR ? u : 0), jg = n0 + r + (KMAJOR ? 0 : u);
      v[q][u] *= kg < jg ? 2.0f : (kg == jg ? 1.0f : 0.0f);
    }
  }
}

template <int T, bool KMAJOR>
__device__ __forceinline__ void store_tile(float* dst, int tid, f32x4 (&v)[TileCfg<T>::LQ], float scale = 1.0f) {
#pragma unroll
  for (int q = 0; q < TileCfg<T>::LQ; ++q) {
    if (scale != 1.0f) v[q] = v[q] * scale;
    int e = q * 256 + tid;
    if (KMAJOR) {
      int r = e >> 3, kk = (e & 7) * 4;
      float* d = dst + r * KSTRIDE + kk;
      d[0] = v[q][0]; d[1] = v[q][1]; d[2] = v[q][2]; d[3] = v[q][3];
    } else {
      int kk = e / (T / 4), r = (e % (T / 4)) * 4;
      *(f32x4*)(dst + kk * TileCfg<T>::RSTRIDE + r) = v[q];
    }
  }
}

template <int T, bool KMAJOR>
__device__ __forceinline__ float read_operand(const float* tile, int row, int kk) {
  return KMAJOR ? tile[row * KSTRIDE + kk] : tile[kk * TileCfg<T>::RSTRIDE + row];
}

template <int T, bool TA, bool TB, bool LOWER, int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs p) {
  constexpr int BM = T, BN = T, WT = T / 2, NI = TileCfg<T>::NI, OPER = TileCfg<T>::OPER, LQ = TileCfg<T>::LQ;
  // Tile of this workgroup.  With a triangular k range the tiles differ in
  // length: they are dealt out longest first, so that the last ones to start
  // are short.
  const int nt = (int)gridDim.x, mt = (int)gridDim.y;
  const int lin = (int)blockIdx.y * nt + (int)blockIdx.x;
  int tn = (int)blockIdx.x, tm = (int)blockIdx.y;
  if (p.kmode == kGemmKSymUpperB) { tn = nt - 1 - lin / mt; tm = lin % mt; }
  else if (p.kmode == kGemmKLowerB) { tn = lin / mt; tm = lin % mt; }
  else if (p.kmode == kGemmKLowerA) { tm = mt - 1 - lin / nt; tn = lin % nt; }
  if (LOWER && tn > tm) return;
  // [buffer][A | B] operand tiles; reused by the row-dot epilogue.  64-wide
  // tiles have four buffers (see the short-k path below).
  constexpr int NBUF = T == 64 ? 4 : 2;
  __shared__ __attribute__((aligned(16))) float smem[NBUF * 2 * OPER];
  constexpr bool AK = !TA;   // A stored [M][K]: k contiguous
  constexpr bool BKM = TB;   // B stored [N][K]: k contiguous

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t z = blockIdx.z;
  const int64_t zi = p.bi > 0 ? z % p.bi : z, zo = p.bi > 0 ? z / p.bi : 0;
  const float* A = p.A + zi * p.sA + zo * p.sA2;
  const float* B = p.B + zi * p.sB + zo * p.sB2;
  float* C = p.C + zi * p.sC + zo * p.sC2;
  const float* Dz = EPI == kEpiRowDot ? p.D + zi * p.sD + zo * p.sD2 : nullptr;
  float* Pz = EPI == kEpiRowDot ? p.P + zi * p.sP + zo * p.sP2 : nullptr;

  // Accumulator layout of a 32x32 MFMA tile: lane l, register r holds
  // row 8*(r/4) + 4*(l/32) + r%4, column l%32.  With beta != 0 the tile of C
  // is loaded into the accumulators up front (its latency overlaps the first
  // operand loads) and alpha is applied to A on its way into LDS, so the
  // epilogue only stores: C = beta*C + (alpha*A) op(B).
  f32x16 acc[NI][NI];
  const bool load_c = EPI == kEpiAxpby && p.beta != 0.0f;
  // Wave-uniform base of this wave's WT x WT sub-tile of C plus a 32-bit lane
  // offset; a whole tile inside C needs no per-element bounds checks.
  const int64_t wrow0 = m0 + wr * WT, wcol0 = n0 + wc * WT;
  float* Cw = C + wrow0 * p.ldc + wcol0;
  const int lane_off = 4 * (lane >> 5) * (int)p.ldc + (lane & 31);
  const bool full = wrow0 + WT <= p.M && wcol0 + WT <= p.N;
  // Unconditional loads (clamped addresses at the matrix edge), so that all
  // of them are in flight together.
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  if (load_c && full) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          acc[i][j][r] = p.beta * Cw[(i * 32 + 8 * (r >> 2) + (r & 3)) * p.ldc + j * 32 + lane_off];
  } else if (load_c) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t gr = wrow0 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int64_t gc = wcol0 + j * 32 + (lane & 31);
          const float v = C[min(gr, p.M - 1) * p.ldc + min(gc, p.N - 1)];
          acc[i][j][r] = (gr < p.M && gc < p.N) ? p.beta * v : 0.0f;
        }
  }
  const float alpha_a = EPI == kEpiAxpby ? p.alpha : 1.0f;

  // The chunks of k this tile needs (all of them unless a triangular operand
  // makes the rest zero).
  int64_t klo = 0, khi = p.K;
  if (p.kmode == kGemmKLowerA) khi = min(p.K, m0 + BM);
  if (p.kmode == kGemmKLowerB) klo = p.noff + n0;
  if (p.kmode == kGemmKSymUpperB) khi = min(p.K, p.noff + n0 + BN);
  const int64_t c0 = klo / BK, nk = (khi + BK - 1) / BK;
  const bool sym = p.kmode == kGemmKSymUpperB;
  // The products of one chunk of BK k-values from the operand tiles at As.
  auto mma_chunk = [&](const float* As) {
    const float* Bs = As + OPER;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 2) {
      float a[NI], b[NI];
#pragma unroll
      for (int t = 0; t < NI; ++t) {
        a[t] = read_operand<T, AK>(As, wr * WT + t * 32 + (lane & 31), kk + (lane >> 5));
        b[t] = read_operand<T, BKM>(Bs, wc * WT + t * 32 + (lane & 31), kk + (lane >> 5));
      }
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };
  bool done = false;
  if constexpr (T == 64) {
    if (nk > c0 && nk - c0 <= NBUF) {
      // At most four chunks (the lazy batch updates, K = 128): with one chunk
      // of look-ahead each chunk would wait for its own loads, so all of them
      // are loaded together (chunks past the end repeat the last, unused),
      // stored, and then multiplied in chunk order, as in the loop below.
      f32x4 ra4[NBUF][LQ], rb4[NBUF][LQ];
#pragma unroll
      for (int u = 0; u < NBUF; ++u) {
        const int64_t cu = min(c0 + u, nk - 1);
        load_tile<T, AK>(A, p.lda, m0, p.M, cu * BK, p.K, tid, ra4[u]);
        load_tile<T, BKM>(B, p.ldb, n0, p.N, cu * BK, p.K, tid, rb4[u]);
      }
#pragma unroll
      for (int u = 0; u < NBUF; ++u)
        if (c0 + u < nk) {
          if (sym) sym_upper<T, BKM>(rb4[u], tid, (c0 + u) * BK, p.noff + n0);
          store_tile<T, AK>(smem + u * 2 * OPER, tid, ra4[u], alpha_a);
          store_tile<T, BKM>(smem + u * 2 * OPER + OPER, tid, rb4[u]);
        }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < NBUF; ++u)
        if (c0 + u < nk) mma_chunk(smem + u * 2 * OPER);
      __syncthreads();
      done = true;
    }
  }
  f32x4 ra[LQ], rb[LQ];
  if (!done) {
    if (c0 < nk) {
      load_tile<T, AK>(A, p.lda, m0, p.M, c0 * BK, p.K, tid, ra);
      load_tile<T, BKM>(B, p.ldb, n0, p.N, c0 * BK, p.K, tid, rb);
      if (sym) sym_upper<T, BKM>(rb, tid, c0 * BK, p.noff + n0);
      store_tile<T, AK>(smem, tid, ra, alpha_a);
      store_tile<T, BKM>(smem + OPER, tid, rb);
    }
    __syncthreads();
    for (int64_t c = c0; c < nk; ++c) {
      const int cur = (int)((c - c0) & 1);
      if (c + 1 < nk) {
        load_tile<T, AK>(A, p.lda, m0, p.M, (c + 1) * BK, p.K, tid, ra);
        load_tile<T, BKM>(B, p.ldb, n0, p.N, (c + 1) * BK, p.K, tid, rb);
      }
      mma_chunk(smem + cur * 2 * OPER);
      if (c + 1 < nk) {
        float* nxt = smem + (cur ^ 1) * 2 * OPER;
        if (sym) sym_upper<T, BKM>(rb, tid, (c + 1) * BK, p.noff + n0);
        store_tile<T, AK>(nxt, tid, ra, alpha_a);
        store_tile<T, BKM>(nxt + OPER, tid, rb);
      }
      __syncthreads();
    }
  }

  if (EPI == kEpiAxpby) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3), col = j * 32 + (lane & 31);
          if (full || (wrow0 + row < p.M && wcol0 + col < p.N))
            Cw[(i * 32 + 8 * (r >> 2) + (r & 3)) * p.ldc + j * 32 + lane_off] = acc[i][j][r];
        }
  } else {
    // Row-dot: P[row, tile] = sum over the tile's columns of alpha*acc*D.
    float (*red)[33] = (float (*)[33])smem;   // [T][33], operand tiles are dead here
    // Unconditional loads of D (clamped at the matrix edge), all in flight
    // together.
    float part[NI][16];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int64_t gi = m0 + wr * WT + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        float s = 0.0f;
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          int64_t gj = n0 + wc * WT + j * 32 + (lane & 31);
          const float d = Dz[min(gi, p.M - 1) * p.ldd + min(gj, p.N - 1)];
          s = fmaf(p.alpha * acc[i][j][r], (gi < p.M && gj < p.N) ? d : 0.0f, s);
        }
        part[i][r] = s;
      }
    for (int half = 0; half < 2; ++half) {
      if (wc == half) {
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            int row = wr * WT + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            float prev = half ? red[row][lane & 31] : 0.0f;
            red[row][lane & 31] = prev + part[i][r];
          }
      }
      __syncthreads();
    }
    if (tid < BM) {
      float s = 0.0f;
      for (int c2 = 0; c2 < 32; ++c2) s += red[tid][c2];
      int64_t gi = m0 + tid;
      if (gi < p.M) Pz[gi * p.ldp + tn] = s;
    }
  }
}

// ---- fp32 GEMM on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16) -----------------
// Each fp32 operand x is split into three bf16 parts, x = x1 + x2 + x3 with
// x1 = bf16(x), x2 = bf16(x - x1), x3 = bf16(x - x1 - x2) (the differences
// are exact in fp32), and a product is the sum of the six part products whose
// orders add up to at most four: x1y1, x1y2, x2y1, x1y3, x2y2, x3y1.  The
// dropped terms are below 2^-24 of |x y|; bf16 products are exact in fp32 and
// accumulate in fp32, so the result has fp32 accuracy at 6/16 of the fp32
// matrix-core time.  A is [M][K] (k contiguous) and B is [K][N], or with TB
// stored [N][K]; tiles are 128 x 128, four waves of 64 x 64, k in chunks of
// 32.  In LDS every part is kept [row][k] (k contiguous, rows padded to 40
// elements), so that an MFMA operand (8 consecutive k of one row or column)
// is one 16-byte read; a [K][N] B is transposed on its way in, each thread
// turning a 4 x 4 block, and a [N][K] B is stored like A.  With LOWER the
// workgroups of tiles wholly above the diagonal exit (square C).
// With NP = 2 the operands are split into two parts, x = x1 + x2 + r with
// |r| <= 2^-16 |x|, and a product sums the three part products x1y1, x1y2,
// x2y1 (the dropped x2y2 is below 2^-16 of |x y|): half the products and
// two thirds of the operand stores of NP = 3.  Only the weighted error
// (the row-dot epilogue) takes it: an error of about 2^-16 per product there
// moves a row's dW H' dW^T by a few parts in a million, and no quantization
// decision depends on it.  NP = 2 reads the second k-step's fragments after
// the first k-step's products instead of among them, which keeps it within
// 256 registers: with its 80 KB of LDS two workgroups share a CU, and each
// hides the other's fragment reads and split stages (same products, same
// order, same bits; the weighted error 381 -> 295 us at 4096 x 4096).
constexpr int X6_T = 128, X6_LD = BK + 8;                 // bf16 row stride of a part
constexpr int X6_PART = X6_T * X6_LD;                     // bf16 elements of one part
template <int NP>
constexpr int x6_buf() { return 2 * NP * X6_PART; }     // A parts, then B parts

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// Two values -> their three bf16 parts, each pair packed as one 32-bit word
// (first value in the low half).
__device__ __forceinline__ void split_pair(float x0, float x1, uint32_t& h, uint32_t& m, uint32_t& l) {
  h = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x0, x1}, bf16x2));
  const float r0 = x0 - __uint_as_float(h << 16), r1 = x1 - __uint_as_float(h & 0xFFFF0000u);
  m = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{r0, r1}, bf16x2));
  const float s0 = r0 - __uint_as_float(m << 16), s1 = r1 - __uint_as_float(m & 0xFFFF0000u);
  l = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{s0, s1}, bf16x2));
}
// Four consecutive-k values of one row -> 8 bytes at element offset off of
// each of the NP parts (the two-part split is the first two of the three).
template <int NP>
__device__ __forceinline__ void put4(uint16_t* base, int off, const f32x4& v) {
  uint32_t h0, m0, l0, h1, m1, l1;
  split_pair(v[0], v[1], h0, m0, l0);
  split_pair(v[2], v[3], h1, m1, l1);
  *(u32x2*)(base + off) = u32x2{h0, h1};
  *(u32x2*)(base + X6_PART + off) = u32x2{m0, m1};
  if (NP == 3) *(u32x2*)(base + 2 * X6_PART + off) = u32x2{l0, l1};
}
// B is stored transposed, [column][k]; its 16-byte k chunks are XOR-swizzled
// by (column / 16) % 4, which spreads the transposing writes over the banks.
__device__ __forceinline__ int x6_boff(int n, int k) { return n * X6_LD + ((((k >> 3) ^ (n >> 4)) & 3) << 3) + (k & 7); }

template <int EPI, bool TB, bool LOWER, int NP, bool ONEBUF>
__global__ __launch_bounds__(256, (NP == 2 || ONEBUF) ? 2 : 1) void gemm_x6_kernel(GemmArgs p) {
  static_assert(NP == 2 || NP == 3, "two or three bf16 parts");
  constexpr int X6_BUF = x6_buf<NP>();
  constexpr int WT = X6_T / 2;
  const int nt = (int)gridDim.x, mt = (int)gridDim.y;
  const int lin = (int)blockIdx.y * nt + (int)blockIdx.x;
  int tn = (int)blockIdx.x, tm = (int)blockIdx.y;
  if (p.kmode == kGemmKSymUpperB) { tn = nt - 1 - lin / mt; tm = lin % mt; }
  else if (p.kmode == kGemmKLowerB) { tn = lin / mt; tm = lin % mt; }
  else if (p.kmode == kGemmKLowerA) { tm = mt - 1 - lin / nt; tn = lin % nt; }
  __shared__ __attribute__((aligned(16))) uint16_t smem[(ONEBUF ? 1 : 2) * X6_BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int64_t m0 = (int64_t)tm * X6_T, n0 = (int64_t)tn * X6_T;
  if (LOWER && n0 >= m0 + X6_T) return;
  const int half = p.ksplit == 2 ? (int)(blockIdx.z & 1) : 0;
  const int64_t z = p.ksplit == 2 ? blockIdx.z >> 1 : blockIdx.z;
  const int64_t zi = p.bi > 0 ? z % p.bi : z, zo = p.bi > 0 ? z / p.bi : 0;
  const float* A = p.A + zi * p.sA + zo * p.sA2;
  const float* B = p.B + zi * p.sB + zo * p.sB2;
  float* C = half ? p.C2 + zi * p.s2C + zo * p.s2C2 : p.C + zi * p.sC + zo * p.sC2;
  const int64_t ldc = half ? p.ldc2 : p.ldc;
  const float* Dz = EPI == kEpiRowDot ? p.D + zi * p.sD + zo * p.sD2 : nullptr;
  float* Pz = EPI == kEpiRowDot ? p.P + zi * p.sP + zo * p.sP2 : nullptr;

  f32x16 acc[2][2];
  const bool load_c = EPI == kEpiAxpby && p.beta != 0.0f;
  const int64_t wrow0 = m0 + wr * WT, wcol0 = n0 + wc * WT;
  float* Cw = C + wrow0 * ldc + wcol0;
  const int lane_off = 4 * (lane >> 5) * (int)ldc + (lane & 31);
  const bool full = wrow0 + WT <= p.M && wcol0 + WT <= p.N;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  if (load_c && full) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          acc[i][j][r] = p.beta * Cw[(i * 32 + 8 * (r >> 2) + (r & 3)) * ldc + j * 32 + lane_off];
  } else if (load_c) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t gr = wrow0 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int64_t gc = wcol0 + j * 32 + (lane & 31);
          const float v = C[min(gr, p.M - 1) * ldc + min(gc, p.N - 1)];
          acc[i][j][r] = (gr < p.M && gc < p.N) ? p.beta * v : 0.0f;
        }
  }
  const float alpha_a = EPI == kEpiAxpby ? p.alpha : 1.0f;

  int64_t klo = 0, khi = p.K;
  if (p.kmode == kGemmKLowerA) khi = min(p.K, m0 + X6_T);
  if (p.kmode == kGemmKLowerB) klo = p.noff + n0;
  if (p.kmode == kGemmKSymUpperB) khi = min(p.K, p.noff + n0 + X6_T);
  if (p.ksplit == 2) {   // halves of whole chunks: the first ends at mid, the second starts there
    const int64_t mid = (klo / BK + ((khi + BK - 1) / BK - klo / BK) / 2) * BK;
    if (half) klo = max(klo, mid); else khi = min(khi, mid);
  }
  const int64_t c0 = klo / BK, nk = max(c0, (khi + BK - 1) / BK);
  const bool sym = p.kmode == kGemmKSymUpperB;

  // Loads of one chunk: A rows (4 float4 along k per thread), B as a 4 x 4
  // block (4 k x 4 columns) per thread, or with TB as rows like A, raw from clamped addresses so that
  // all eight are in flight while the previous chunk is multiplied; masking,
  // alpha and the symmetric weights are applied when the chunk is stored.
  const int bk = (tid >> 5) * 4, bn = (tid & 31) * 4;
  auto load_a = [&](int64_t k0, f32x4 (&ra)[4], int q) {
    const int e = q * 256 + tid, r = e >> 3, kk = (e & 7) * 4;
    ra[q] = *(const f32x4*)(A + min(m0 + r, p.M - 1) * p.lda + min(k0 + kk, p.K - 4));
  };
  auto load_b = [&](int64_t k0, f32x4 (&rb)[4], int i) {
    if (TB) {
      const int e = i * 256 + tid, r = e >> 3, kk = (e & 7) * 4;
      rb[i] = *(const f32x4*)(B + min(n0 + r, p.N - 1) * p.ldb + min(k0 + kk, p.K - 4));
    } else {
      rb[i] = *(const f32x4*)(B + min(k0 + bk + i, p.K - 1) * p.ldb + min(n0 + bn, p.N - 4));
    }
  };
  auto load_chunk = [&](int64_t k0, f32x4 (&ra)[4], f32x4 (&rb)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) load_a(k0, ra, q);
#pragma unroll
    for (int i = 0; i < 4; ++i) load_b(k0, rb, i);
  };
  // Piece idx of storing a loaded chunk into LDS as three bf16 parts:
  // pieces 0..3 are A's row chunks q = idx, pieces 4..7 B's columns
  // bn + idx - 4 (four k values each).  Indices fit in 32 bits.
  const int sm0 = (int)m0, sn0 = (int)n0, sM = (int)p.M, sN = (int)p.N, sK = (int)p.K, snoff = (int)p.noff;
  auto store_piece = [&](uint16_t* buf, int k0, const f32x4 (&ra)[4], const f32x4 (&rb)[4], int idx) {
    if (idx < 4) {
      const int q = idx, e = q * 256 + tid, r = e >> 3, kk = (e & 7) * 4;
      const bool ok = sm0 + r < sM && k0 + kk < sK;
      put4<NP>(buf, r * X6_LD + kk, ok ? ra[q] * alpha_a : f32x4{0.f, 0.f, 0.f, 0.f});
    } else if (TB) {
      const int q = idx - 4, e = q * 256 + tid, r = e >> 3, kk = (e & 7) * 4;
      const bool ok = sn0 + r < sN && k0 + kk < sK;
      put4<NP>(buf + NP * X6_PART, x6_boff(r, kk), ok ? rb[q] : f32x4{0.f, 0.f, 0.f, 0.f});
    } else {
      const int j = idx - 4, gn = sn0 + bn;
      f32x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int gk = k0 + bk + i;
        float x = (gk < sK && gn < sN) ? rb[i][j] : 0.0f;
        if (sym) {
          const int jg = snoff + gn + j;
          x *= gk < jg ? 2.0f : (gk == jg ? 1.0f : 0.0f);
        }
        v[i] = x;
      }
      put4<NP>(buf + NP * X6_PART, x6_boff(bn + j, bk), v);
    }
  };
  auto store_chunk = [&](uint16_t* buf, int k0, const f32x4 (&ra)[4], const f32x4 (&rb)[4]) {
#pragma unroll
    for (int idx = 0; idx < 8; ++idx) store_piece(buf, k0, ra, rb, idx);
  };
  // Stage st (0..5) of piece idx, the same arithmetic as store_piece spread
  // over six calls: the input, its high parts, the first residual, the
  // middle parts (and the high store), the low parts, the last two stores.
  auto store_stage = [&](uint16_t* buf, int k0, const f32x4 (&ra)[4], const f32x4 (&rb)[4], int idx, int st,
                         f32x4& v, uint32_t& h0, uint32_t& h1, uint32_t& mm0, uint32_t& mm1, float (&r)[4]) {
    uint16_t* base;
    int off;
    if (idx < 4) {
      const int e = idx * 256 + tid;
      base = buf; off = (e >> 3) * X6_LD + (e & 7) * 4;
    } else if (TB) {
      const int e = (idx - 4) * 256 + tid;
      base = buf + NP * X6_PART; off = x6_boff(e >> 3, (e & 7) * 4);
    } else {
      base = buf + NP * X6_PART; off = x6_boff(bn + idx - 4, bk);
    }
    if (st == 0) {
      if (idx < 4) {
        const int q = idx, e = q * 256 + tid, rr = e >> 3, kk = (e & 7) * 4;
        const bool ok = sm0 + rr < sM && k0 + kk < sK;
        v = ok ? ra[q] * alpha_a : f32x4{0.f, 0.f, 0.f, 0.f};
      } else if (TB) {
        const int q = idx - 4, e = q * 256 + tid, rr = e >> 3, kk = (e & 7) * 4;
        const bool ok = sn0 + rr < sN && k0 + kk < sK;
        v = ok ? rb[q] : f32x4{0.f, 0.f, 0.f, 0.f};
      } else {
        const int j = idx - 4, gn = sn0 + bn;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int gk = k0 + bk + i;
          float x = (gk < sK && gn < sN) ? rb[i][j] : 0.0f;
          if (sym) {
            const int jg = snoff + gn + j;
            x *= gk < jg ? 2.0f : (gk == jg ? 1.0f : 0.0f);
          }
          v[i] = x;
        }
      }
    } else if (st == 1) {
      h0 = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{v[0], v[1]}, bf16x2));
      h1 = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{v[2], v[3]}, bf16x2));
    } else if (st == 2) {
      r[0] = v[0] - __uint_as_float(h0 << 16); r[1] = v[1] - __uint_as_float(h0 & 0xFFFF0000u);
      r[2] = v[2] - __uint_as_float(h1 << 16); r[3] = v[3] - __uint_as_float(h1 & 0xFFFF0000u);
    } else if (st == 3) {
      mm0 = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{r[0], r[1]}, bf16x2));
      mm1 = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{r[2], r[3]}, bf16x2));
      *(u32x2*)(base + off) = u32x2{h0, h1};
    } else if (NP == 2) {   // stage 4 stores the second (last) parts; stage 5 has nothing left
      if (st == 4) *(u32x2*)(base + X6_PART + off) = u32x2{mm0, mm1};
    } else if (st == 4) {
      r[0] -= __uint_as_float(mm0 << 16); r[1] -= __uint_as_float(mm0 & 0xFFFF0000u);
      r[2] -= __uint_as_float(mm1 << 16); r[3] -= __uint_as_float(mm1 & 0xFFFF0000u);
      h0 = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{r[0], r[1]}, bf16x2));   // low parts
      h1 = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{r[2], r[3]}, bf16x2));
    } else {
      *(u32x2*)(base + X6_PART + off) = u32x2{mm0, mm1};
      *(u32x2*)(base + 2 * X6_PART + off) = u32x2{h0, h1};
    }
  };

  // Two register sets of raw chunks: while chunk c is multiplied, chunk c+1
  // (loaded two steps earlier) is split into the other LDS buffer, in eight
  // pieces placed among the products, and then the loads of chunk c+3 take
  // its registers.  Loads past the end read clamped addresses and stores past
  // the end go to the idle buffer, so no step branches.
  if constexpr (ONEBUF) {
    // One LDS buffer (two workgroups share a CU): per chunk, the split parts
    // are stored, the next chunk's loads issued into the same registers, and
    // after a barrier both k-steps are multiplied; another barrier frees the
    // buffer.  The other workgroup on the CU runs its products while this one
    // splits and stores.
    f32x4 ra[4], rb[4];
    load_chunk(c0 * BK, ra, rb);
    const int arow = wr * WT + (lane & 31), brow = wc * WT + (lane & 31), koff = 8 * (lane >> 5);
    constexpr int NPR = NP == 3 ? 6 : 3;
    constexpr int PA[6] = {NP == 3 ? 2 : 1, NP == 3 ? 1 : 0, 0, 1, 0, 0};
    constexpr int PB[6] = {0, 1, NP == 3 ? 2 : 0, 0, 1, 0};
    static_assert(BK == 32, "two 16-deep k-steps per chunk");
    const uint16_t* Bs = smem + NP * X6_PART;
    for (int64_t c = c0; c < nk; ++c) {
      store_chunk(smem, (int)(c * BK), ra, rb);
      load_chunk((c + 1) * BK, ra, rb);   // clamped addresses past the end
      lds_barrier();
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bf16x8 a[NP][2], b[NP][2];
#pragma unroll
        for (int f = 0; f < 4 * NP; ++f) {
          const int pt = f >> 2, t = (f >> 1) & 1, ks = 16 * h;
          if (f & 1) b[pt][t] = *(const bf16x8*)(Bs + pt * X6_PART + x6_boff(brow + 32 * t, ks + koff));
          else a[pt][t] = *(const bf16x8*)(smem + pt * X6_PART + (arow + 32 * t) * X6_LD + ks + koff);
        }
#pragma unroll
        for (int m = 0; m < 4 * NPR; ++m) {
          const int pp = m >> 2, i = (m >> 1) & 1, j = m & 1;
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[PA[pp]][i], b[PB[pp]][j], acc[i][j], 0, 0, 0);
        }
      }
      lds_barrier();
    }
  } else {
    f32x4 ra0[4], rb0[4], ra1[4], rb1[4];
    load_chunk(c0 * BK, ra0, rb0);
    store_chunk(smem, (int)(c0 * BK), ra0, rb0);
    load_chunk((c0 + 1) * BK, ra0, rb0);
    load_chunk((c0 + 2) * BK, ra1, rb1);
    __syncthreads();
    // Lane l reads rows (l % 32) and k offset 8 (l / 32) of each 32-row block.
    const int arow = wr * WT + (lane & 31), brow = wc * WT + (lane & 31), koff = 8 * (lane >> 5);
    // Part products, smallest first: NPR of them per 32 x 32 accumulator and
    // k-step, 4 NPR MFMAs per k-step, each followed by SPS of the 48 store
    // stages of the next chunk (8 pieces of 6).
    constexpr int NPR = NP == 3 ? 6 : 3, SPS = 48 / (8 * NPR);
    constexpr int PA[6] = {NP == 3 ? 2 : 1, NP == 3 ? 1 : 0, 0, 1, 0, 0};
    constexpr int PB[6] = {0, 1, NP == 3 ? 2 : 0, 0, 1, 0};
    static_assert(BK == 32, "two 16-deep k-steps per chunk");
    // As (the buffer being multiplied) and nbuf (the idle one) are distinct,
    // which the restrict qualifiers state: the stores into nbuf need not wait
    // for the fragment reads from As.
    auto body = [&](const uint16_t* __restrict__ As, uint16_t* __restrict__ nbuf, int64_t c, f32x4 (&ra)[4],
                    f32x4 (&rb)[4]) {
      const uint16_t* Bs = As + NP * X6_PART;
      const int kn = (int)((c + 1) * BK);
      bf16x8 a[2][NP][2], b[2][NP][2];   // [k-step][part][32-row block]
      auto read = [&](int h, int f) {   // fragment f (0..4 NP - 1) of k-step h
        const int pt = f >> 2, t = (f >> 1) & 1, ks = 16 * h;
        if (f & 1) b[h][pt][t] = *(const bf16x8*)(Bs + pt * X6_PART + x6_boff(brow + 32 * t, ks + koff));
        else a[h][pt][t] = *(const bf16x8*)(As + pt * X6_PART + (arow + 32 * t) * X6_LD + ks + koff);
      };
  #pragma unroll
      for (int f = 0; f < 4 * NP; ++f) read(0, f);
      // Per k-step: 24 products (the four accumulators take turns, so that no
      // MFMA waits for the one before it).  Behind each product comes one stage
      // of the next chunk's store (6 stages for each of its 8 pieces, a few
      // vector instructions each, which run while the MFMA does); the first
      // k-step also reads the second one's fragments, and each load of chunk
      // c+3 follows the stage that last reads the registers it fills (A's row
      // chunk q: piece q's first stage; B's rows: piece 7's, or with TB B's row
      // chunk q: piece 4 + q's).
      f32x4 sv;
      uint32_t sh0, sh1, sm0_, sm1_;
      float sr[4];
  #pragma unroll
      for (int h = 0; h < 2; ++h)
  #pragma unroll
        for (int m = 0; m < 4 * NPR; ++m) {
          if (NP == 2 && h == 1 && m == 0) {
  #pragma unroll
            for (int f = 0; f < 4 * NP; ++f) read(1, f);
          }
          const int pp = m >> 2, i = (m >> 1) & 1, j = m & 1;
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[h][PA[pp]][i], b[h][PB[pp]][j], acc[i][j], 0, 0, 0);
          if (NP == 3 && h == 0 && m < 4 * NP) read(1, m);
  #pragma unroll
          for (int u = 0; u < SPS; ++u) {
            const int g = SPS * (4 * NPR * h + m) + u;
            store_stage(nbuf, kn, ra, rb, g / 6, g % 6, sv, sh0, sh1, sm0_, sm1_, sr);
            if (g % 6 == 1 && g < 24) load_a((c + 3) * BK, ra, g / 6);
            if (TB && g % 6 == 1 && g >= 24) load_b((c + 3) * BK, rb, g / 6 - 4);
            if (!TB && g >= 43 && g < 47) load_b((c + 3) * BK, rb, g - 43);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto step = [&](int64_t c, f32x4 (&ra)[4], f32x4 (&rb)[4]) {
      const int cur = (int)((c - c0) & 1);
      body(smem + cur * X6_BUF, smem + (cur ^ 1) * X6_BUF, c, ra, rb);
      lds_barrier();
    };
    for (int64_t c = c0; c < nk; c += 2) {
      step(c, ra0, rb0);
      if (c + 1 < nk) step(c + 1, ra1, rb1);
    }
  }

  if (EPI == kEpiAxpby) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3), col = j * 32 + (lane & 31);
          if (full || (wrow0 + row < p.M && wcol0 + col < p.N))
            Cw[(i * 32 + 8 * (r >> 2) + (r & 3)) * ldc + j * 32 + lane_off] = acc[i][j][r];
        }
  } else {
    float (*red)[33] = (float (*)[33])smem;   // [128][33], operand tiles are dead here
    float part[2][16];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int64_t gi = m0 + wr * WT + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        float sacc = 0.0f;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          int64_t gj = n0 + wc * WT + j * 32 + (lane & 31);
          const float d = Dz[min(gi, p.M - 1) * p.ldd + min(gj, p.N - 1)];
          sacc = fmaf(p.alpha * acc[i][j][r], (gi < p.M && gj < p.N) ? d : 0.0f, sacc);
        }
        part[i][r] = sacc;
      }
    for (int half = 0; half < 2; ++half) {
      if (wc == half) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            int row = wr * WT + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            float prev = half ? red[row][lane & 31] : 0.0f;
            red[row][lane & 31] = prev + part[i][r];
          }
      }
      __syncthreads();
    }
    if (tid < X6_T) {
      float sacc = 0.0f;
      for (int c2 = 0; c2 < 32; ++c2) sacc += red[tid][c2];
      int64_t gi = m0 + tid;
      if (gi < p.M) Pz[gi * p.ldp + tn] = sacc;
    }
  }
}

// C += C2 elementwise over M x N (row strides ldc, ldc2), matrix z = blockIdx.y;
// 4 columns per thread, as 16-byte vectors when both rows allow.
__global__ __launch_bounds__(256) void add_into_kernel(float* __restrict__ C, int64_t ldc, const float* __restrict__ C2,
                                                       int64_t ldc2, int64_t M, int64_t N, int64_t sC, int64_t sC2) {
  C += (int64_t)blockIdx.y * sC;
  C2 += (int64_t)blockIdx.y * sC2;
  const int64_t n4 = (N + 3) / 4, items = M * n4;
  const bool vec = ((ldc | ldc2 | sC | sC2) & 3) == 0 && ((uintptr_t)C & 15) == 0 && ((uintptr_t)C2 & 15) == 0;
  for (int64_t it = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; it < items; it += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = it / n4, j = (it % n4) * 4;
    if (vec && j + 4 <= N) {
      f32x4 a = *(const f32x4*)(C + i * ldc + j);
      const f32x4 b = *(const f32x4*)(C2 + i * ldc2 + j);
      a += b;
      *(f32x4*)(C + i * ldc + j) = a;
    } else {
      for (int64_t t = j; t < min(N, j + 4); ++t) C[i * ldc + t] += C2[i * ldc2 + t];
    }
  }
}

int gemm_num_cus() {
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
  }
  return cus;
}

template <int T, bool TA, bool TB, bool LOWER, int EPI>
hipError_t launch_t(const GemmArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((a.N + T - 1) / T), (unsigned)((a.M + T - 1) / T), (unsigned)a.batch);
  hipLaunchKernelGGL((gemm_f32_kernel<T, TA, TB, LOWER, EPI>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// 64-wide fp32 tiles when 128-wide ones would give fewer than one per two CUs
// (the row-dot keeps 128: its partial sums are laid out per 128 columns);
// otherwise the split-bf16 kernel for A [M][K] times B [K][N] or [N][K].  Measured on
// the 4096-column layer: the crossover between 1/4 and 1 tile per CU.  The
// choice counts the tiles of one outer batch item only, so a matrix of a
// batch gets the same kernel, and the same bits, as when it is alone.
template <bool TA, bool TB, bool LOWER, int EPI>
hipError_t launch(const GemmArgs& a, hipStream_t s) {
  const int64_t inner = a.bi > 0 ? a.bi : a.batch;
  const int64_t tiles128 = ((a.N + 127) / 128) * ((a.M + 127) / 128) * inner;
  if (a.ksplit == 2 && (TA || TB || LOWER || EPI != kEpiAxpby || a.beta != 0.0f)) return hipErrorInvalidValue;
  if (a.ksplit != 2 && EPI == kEpiAxpby && 2 * tiles128 < gemm_num_cus()) return launch_t<64, TA, TB, LOWER, EPI>(a, s);
  if constexpr (!TA && (TB || !LOWER) && (!TB || EPI == kEpiAxpby)) {
    if (!TB || a.kmode == kGemmKFull) {
      dim3 grid((unsigned)((a.N + X6_T - 1) / X6_T), (unsigned)((a.M + X6_T - 1) / X6_T),
                (unsigned)(a.batch * (a.ksplit == 2 ? 2 : 1)));
      // Three parts: the one-buffer kernel (two workgroups per CU) once there
      // are more live tiles than CUs; below that it has no partner on the CU
      // and the double-buffered kernel is faster.  Both give the same bits.
      const int64_t mt = (a.M + X6_T - 1) / X6_T, nt = (a.N + X6_T - 1) / X6_T;
      int64_t live = mt * nt;
      if (LOWER) {   // tiles wholly above the diagonal exit
        live = 0;
        for (int64_t t = 0; t < mt; ++t) live += std::min<int64_t>(nt, t + 1);
      }
      live *= a.batch * (a.ksplit == 2 ? 2 : 1);
      if (EPI == kEpiRowDot)
        hipLaunchKernelGGL((gemm_x6_kernel<EPI, TB, LOWER, 2, false>), grid, dim3(256), 0, s, a);
      else if (live > gemm_num_cus())
        hipLaunchKernelGGL((gemm_x6_kernel<EPI, TB, LOWER, 3, true>), grid, dim3(256), 0, s, a);
      else
        hipLaunchKernelGGL((gemm_x6_kernel<EPI, TB, LOWER, 3, false>), grid, dim3(256), 0, s, a);
      return hipGetLastError();
    }
  }
  return launch_t<128, TA, TB, LOWER, EPI>(a, s);
}

// ---- fp64 rank update: C -= A B with A, C fp64 and B fp32 (widened) ------------
// 64 x 64 tiles, 4 waves of 32 x 32 (2 x 2 v_mfma_f64_16x16x4f64 tiles), k in
// chunks of 16.  MFMA f64 16x16x4: lane l supplies A[l%16][l/16] and
// B[l/16][l%16]; result register r of lane l is row l/16 + 4r, column l%16.
constexpr int F64_T = 64, F64_BK = 16;
__global__ __launch_bounds__(256) void rank_update_f64_kernel(const double* __restrict__ A, int64_t lda,
                                                              const float* __restrict__ B, int64_t ldb,
                                                              double* __restrict__ C, int64_t ldc, int64_t M,
                                                              int64_t N, int64_t K, int64_t sA, int64_t sB,
                                                              int64_t sC) {
  __shared__ double As[F64_T][F64_BK + 1];   // -A tile, [row][k]
  A += (int64_t)blockIdx.z * sA;   // matrix of a batch
  B += (int64_t)blockIdx.z * sB;
  C += (int64_t)blockIdx.z * sC;
  __shared__ double Bs[F64_BK][F64_T + 1];   // B tile, [k][column]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * F64_T, n0 = (int64_t)blockIdx.x * F64_T;
  f64x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = m0 + wr * 32 + 16 * i + (lane >> 4) + 4 * r;
        const int64_t col = n0 + wc * 32 + 16 * j + (lane & 15);
        const double v = C[min(row, M - 1) * ldc + min(col, N - 1)];
        acc[i][j][r] = (row < M && col < N) ? v : 0.0;
      }
  for (int64_t k0 = 0; k0 < K; k0 += F64_BK) {
    double av[4];
    float bv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid + 256 * q;
      const int64_t gr = m0 + (e >> 4), gk = k0 + (e & 15);
      const double x = A[min(gr, M - 1) * lda + min(gk, K - 1)];
      av[q] = (gr < M && gk < K) ? -x : 0.0;
      const int64_t gk2 = k0 + (e >> 6), gc = n0 + (e & 63);
      const float y = B[min(gk2, K - 1) * ldb + min(gc, N - 1)];
      bv[q] = (gk2 < K && gc < N) ? y : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid + 256 * q;
      As[e >> 4][e & 15] = av[q];
      Bs[e >> 6][e & 63] = (double)bv[q];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < F64_BK; kk += 4) {
      double a[2], b[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        a[t] = As[wr * 32 + 16 * t + (lane & 15)][kk + (lane >> 4)];
        b[t] = Bs[kk + (lane >> 4)][wc * 32 + 16 * t + (lane & 15)];
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = m0 + wr * 32 + 16 * i + (lane >> 4) + 4 * r;
        const int64_t col = n0 + wc * 32 + 16 * j + (lane & 15);
        if (row < M && col < N) C[row * ldc + col] = acc[i][j][r];
      }
}

}  // namespace

hipError_t rank_update_f64(const double* A, int64_t lda, const float* B, int64_t ldb, double* C, int64_t ldc,
                           int64_t M, int64_t N, int64_t K, hipStream_t s, int64_t nb, int64_t sA, int64_t sB,
                           int64_t sC) {
  if (M <= 0 || N <= 0 || K <= 0 || nb <= 0) return hipSuccess;
  dim3 grid((unsigned)((N + F64_T - 1) / F64_T), (unsigned)((M + F64_T - 1) / F64_T), (unsigned)nb);
  hipLaunchKernelGGL(rank_update_f64_kernel, grid, dim3(256), 0, s, A, lda, B, ldb, C, ldc, M, N, K, sA, sB, sC);
  return hipGetLastError();
}

hipError_t gemm_f32(const GemmArgs& a, bool ta, bool tb, bool lower, GemmEpi epi, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0 || a.batch <= 0) return hipSuccess;
  if (epi == kEpiRowDot) {
    if (!ta && !tb && !lower) return launch<false, false, false, kEpiRowDot>(a, s);
    return hipErrorInvalidValue;
  }
  if (!ta && !tb) return lower ? launch<false, false, true, kEpiAxpby>(a, s) : launch<false, false, false, kEpiAxpby>(a, s);
  if (!ta && tb) return lower ? launch<false, true, true, kEpiAxpby>(a, s) : launch<false, true, false, kEpiAxpby>(a, s);
  if (ta && !tb) return lower ? launch<true, false, true, kEpiAxpby>(a, s) : launch<true, false, false, kEpiAxpby>(a, s);
  return launch<true, true, false, kEpiAxpby>(a, s);
}

hipError_t add_into(float* C, int64_t ldc, const float* C2, int64_t ldc2, int64_t M, int64_t N, hipStream_t s,
                    int64_t nb, int64_t sC, int64_t sC2) {
  if (M <= 0 || N <= 0 || nb <= 0) return hipSuccess;
  const int64_t items = M * ((N + 3) / 4);
  const unsigned blocks = (unsigned)min((items + 255) / 256, (int64_t)2048);
  hipLaunchKernelGGL(add_into_kernel, dim3(blocks, (unsigned)nb), dim3(256), 0, s, C, ldc, C2, ldc2, M, N, sC, sC2);
  return hipGetLastError();
}

}  // namespace nvq
