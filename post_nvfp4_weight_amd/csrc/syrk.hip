// Hessian accumulation H += X^T X for bf16 activations on CDNA4 matrix cores
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation; bf16 x bf16 products are exact).
//
// Work decomposition.  Only the upper triangle of H is computed, in three
// kinds of tiles, each owned by a 4-wave workgroup for a contiguous token
// range:
//   quad    256x256 off-diagonal block of H (waves hold 128x128 each);
//   strip   128x256: the top half of a diagonal 256-block (its diagonal
//           128-block plus the 128x128 block right of it; waves 64x128);
//   single  128x128: the bottom-right diagonal 128-block of a diagonal
//           256-block (waves 64x64).
// A quad moves 512 channels per token for 65536 products, a strip 384 for
// 32768: the big tile halves the load traffic per flop.  Quads over half of
// the tokens and strips over all of them are the same amount of work, so the
// first launch runs both side by side (for a 4096-channel layer: 240 quad
// halves + 16 strips = 256 equal items); the small singles follow, split over
// tokens.  Split tiles write partial sums to the workspace, summed in a
// fixed order by a second kernel, so results are reproducible.
//
// Operand staging.  X is row-major [tokens][channels]; an MFMA operand needs
// 8 consecutive tokens of one channel per lane.  Tokens are streamed in
// 32-token stages through a ring of LDS buffers filled by buffer loads that
// write LDS directly (no registers, no per-load address arithmetic; the
// buffer bound returns zeros past the last token).  The tile keeps X's layout,
// [token][channel], and operands are fetched with ds_read_b64_tr_b16: within
// each 16-lane group, lane j addresses token T + j/4, channels C + 4(j%4),
// and lane i receives channel C + i for tokens T..T+3.  16-byte chunks of a
// row are XOR-swizzled by the row index so that the transposed reads of 32
// lanes hit 64 distinct banks.
#include "common.h"
#include "kernels.h"

namespace nvq {

namespace {

#ifndef NVQ_SYRK_ST
#define NVQ_SYRK_ST 32
#endif
#ifndef NVQ_SYRK_NS
#define NVQ_SYRK_NS 4
#endif
constexpr int ST = NVQ_SYRK_ST;   // tokens per stage
constexpr int NS = NVQ_SYRK_NS;   // ring depth (stages in flight + the one being multiplied)

typedef short s16x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

// Physical 16-byte chunk of logical chunk p in tile row r, and its inverse.
// g(p) = p ^ ((p & 2) << 2) moves chunk bit 1 into bit 3 (an involution);
// the row index then XORs bits 1..3.
__device__ __forceinline__ int swz(int p, int r) { return (p ^ ((p & 2) << 2)) ^ (2 * (r & 7)); }
__device__ __forceinline__ int unswz(int pc, int r) {
  const int y = pc ^ (2 * (r & 7));
  return y ^ ((y & 2) << 2);
}

template <int TM, int TN>
struct Tile {
  static constexpr int A_ROWB = TM * 2, B_ROWB = TN * 2;    // bytes per token row
  static constexpr int A_BYTES = ST * A_ROWB, B_BYTES = ST * B_ROWB;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int PER_WAVE = STAGE_BYTES / 4096;         // 1 KB direct-to-LDS loads per wave
  static constexpr int NI = TM / 64, NJ = TN / 64;            // 32x32 MFMA tiles per wave
};

constexpr int QUAD = 256, HALF = 128;
constexpr size_t kSlotFloats = (size_t)QUAD * QUAD;

// Enqueue one stage's direct-to-LDS loads: the lane's 16-byte chunks of the
// stage's token rows (voff: byte offsets from src) into the buffer at dst.
// Offsets at or past nrec bytes read as zero.
template <int PER_WAVE>
__device__ __forceinline__ void issue_loads(char* dst, const void* src, int nrec, const uint32_t (&voff)[PER_WAVE],
                                            const int (&ldsoff)[PER_WAVE]) {
#if __HIP_DEVICE_COMPILE__   // buffer resources exist only in device code
  __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, nrec, 0x00020000);
#pragma unroll
  for (int q = 0; q < PER_WAVE; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(dst + ldsoff[q]), 16, voff[q], 0, 0, 0);
#endif
}

// One pipeline step: enqueue the direct-to-LDS loads of a later stage into
// `dst` and multiply the stage already resident in `buf`.  The two slots never
// overlap, which the restrict qualifiers state; the completion of the loads is
// tracked by explicit vmcnt waits and a barrier in the caller, so the compiler
// need not wait on them before the operand reads here.
template <int TM, int TN>
__device__ __forceinline__ void stage_step(char* __restrict__ dst, bool issue, const void* src, int nrec,
                                           const uint32_t (&voff)[Tile<TM, TN>::PER_WAVE],
                                           const int (&ldsoff)[Tile<TM, TN>::PER_WAVE], const char* __restrict__ buf,
                                           const int (&aoff)[Tile<TM, TN>::NI][2],
                                           const int (&boff)[Tile<TM, TN>::NJ][2],
                                           f32x16 (&acc)[Tile<TM, TN>::NI][Tile<TM, TN>::NJ]) {
  using T = Tile<TM, TN>;
  if (issue) issue_loads<T::PER_WAVE>(dst, src, nrec, voff, ldsoff);
#pragma unroll
  for (int kk = 0; kk < ST / 16; ++kk) {
    bf16x8 a[T::NI], b[T::NJ];
#pragma unroll
    for (int f = 0; f < T::NI; ++f) {
      s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(buf + aoff[f][0] + kk * 16 * T::A_ROWB));
      s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(buf + aoff[f][1] + kk * 16 * T::A_ROWB));
      a[f] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
#pragma unroll
    for (int f = 0; f < T::NJ; ++f) {
      s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(buf + boff[f][0] + kk * 16 * T::B_ROWB));
      s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(buf + boff[f][1] + kk * 16 * T::B_ROWB));
      b[f] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
#pragma unroll
    for (int i = 0; i < T::NI; ++i)
#pragma unroll
      for (int f = 0; f < T::NJ; ++f)
        acc[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[f], acc[i][f], 0, 0, 0);
  }
}

// One tile job: rows [rowc0, rowc0+TM) x columns [colc0, colc0+TN) of H over
// tokens [t_begin, t_end).  P == nullptr: add into H (upper triangle + mirror);
// otherwise store the partial sums into P [TM x TN].  Channels at or past k
// may be read (they only feed accumulators of rows/columns >= k, which are
// never stored); reads stay inside X's rows thanks to the buffer bound.
template <int TM, int TN>
__device__ __forceinline__ void tile_job(char* lds, const uint16_t* __restrict__ X, int64_t k, int64_t ldx,
                                         int64_t rowc0, int64_t colc0, int64_t t_begin, int64_t t_end,
                                         float* __restrict__ H, float* __restrict__ P) {
  using T = Tile<TM, TN>;
  const int nstages = t_end > t_begin ? (int)((t_end - t_begin + ST - 1) / ST) : 0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;

  // This lane's source offset (bytes from the stage's first token row) for
  // each of the wave's load instructions, and the LDS chunk it fills.
  uint32_t voff[T::PER_WAVE];
  int ldsoff[T::PER_WAVE];
#pragma unroll
  for (int q = 0; q < T::PER_WAVE; ++q) {
    const int ins = wave + 4 * q;
    const int off = ins * 1024 + lane * 16;
    const bool is_b = off >= T::A_BYTES;
    const int toff = is_b ? off - T::A_BYTES : off;
    const int rowb = is_b ? T::B_ROWB : T::A_ROWB;
    const int r = toff / rowb, pc = (toff % rowb) / 16;
    const int p = unswz(pc, r);                         // logical chunk: channels 8p..8p+7
    const int64_t ch = (is_b ? colc0 : rowc0) + 8 * p;
    voff[q] = (uint32_t)(r * ldx * 2 + ch * 2);
    ldsoff[q] = ins * 1024;
  }

  // Per-lane LDS byte offsets of the transposed operand reads, for each
  // fragment f and half h (tokens 4h..4h+3 of the lane group's 8), k-step 0.
  const int g = lane >> 4, j = lane & 15;
  int aoff[T::NI][2], boff[T::NJ][2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = 8 * (g >> 1) + 4 * h + (j >> 2);
#pragma unroll
    for (int f = 0; f < T::NI; ++f) {
      const int ch = wr * (TM / 2) + f * 32 + 16 * (g & 1) + 4 * (j & 3);
      aoff[f][h] = r * T::A_ROWB + swz(ch >> 3, r) * 16 + 8 * (j & 1);
    }
#pragma unroll
    for (int f = 0; f < T::NJ; ++f) {
      const int ch = wc * (TN / 2) + f * 32 + 16 * (g & 1) + 4 * (j & 3);
      boff[f][h] = T::A_BYTES + r * T::B_ROWB + swz(ch >> 3, r) * 16 + 8 * (j & 1);
    }
  }

  f32x16 acc[T::NI][T::NJ];
#pragma unroll
  for (int i = 0; i < T::NI; ++i)
#pragma unroll
    for (int f = 0; f < T::NJ; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][f][r] = 0.0f;

  for (int s = 0; s < NS - 1 && s < nstages; ++s) {
    const int64_t t0 = t_begin + (int64_t)s * ST;
    issue_loads<T::PER_WAVE>(lds + (s % NS) * T::STAGE_BYTES, (const void*)(X + t0 * ldx),
                             (int)min((t_end - t0) * ldx * 2, (int64_t)0x7FFFFFF0), voff, ldsoff);
  }
  // Steady state: NS-2 later stages stay in flight while stage s is used.
  constexpr int kWait = (NS - 2) * T::PER_WAVE;
  static_assert(kWait < 64, "vmcnt range");
  auto step = [&](int s, bool steady) {
    // Wait until this wave's loads of stage s have landed, then make every
    // wave's loads visible with a plain workgroup barrier (the memory clobber
    // keeps the compiler from moving LDS accesses across it; __syncthreads()
    // would add a release fence that drains the stages still in flight).
    if (steady) __builtin_amdgcn_s_waitcnt((kWait & 15) | (7 << 4) | (15 << 8) | ((kWait >> 4) << 14));
    else __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
    asm volatile("s_barrier" ::: "memory");
    const int sn = s + NS - 1;
    const bool issue = sn < nstages;
    const int64_t t0 = t_begin + (int64_t)sn * ST;
    const int64_t rem = issue ? (t_end - t0) * ldx * 2 : 0;
    stage_step<TM, TN>(lds + (sn % NS) * T::STAGE_BYTES, issue, (const void*)(X + (issue ? t0 : t_begin) * ldx),
                       (int)min(rem, (int64_t)0x7FFFFFF0), voff, ldsoff, lds + (s % NS) * T::STAGE_BYTES, aoff,
                       boff, acc);
  };
  int s = 0;
  for (; s + NS - 2 < nstages; ++s) step(s, true);    // stages s+1..s+NS-2 exist
  for (; s < nstages; ++s) step(s, false);            // drain: wait for everything

  // Epilogue.  Accumulator element (lane l, register r) of a 32x32 tile is at
  // row 8*(r/4) + 4*(l/32) + r%4, column l%32.
  if (P == nullptr) {
    // Per 32x32 tile: read the old upper-triangle values, then store (stores
    // to H would otherwise serialize the loads behind them).
#pragma unroll
    for (int i = 0; i < T::NI; ++i)
#pragma unroll
      for (int f = 0; f < T::NJ; ++f) {
        const int64_t gj = colc0 + wc * (TN / 2) + f * 32 + (lane & 31);
        float old[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t gi = rowc0 + wr * (TM / 2) + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          old[r] = (gi < k && gj < k && gi <= gj) ? H[gi * k + gj] : 0.0f;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t gi = rowc0 + wr * (TM / 2) + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (gi < k && gj < k && gi <= gj) {
            const float v = old[r] + acc[i][f][r];
            H[gi * k + gj] = v;
            if (gi != gj) H[gj * k + gi] = v;
          }
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < T::NI; ++i)
#pragma unroll
      for (int f = 0; f < T::NJ; ++f) {
        const int col = wc * (TN / 2) + f * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wr * (TM / 2) + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          P[row * TN + col] = acc[i][f][r];
        }
      }
  }
}

// Quad q (a < b over 256-blocks, row-major) -> (a, b).
__device__ __forceinline__ void quad_coords(int q, int nb2, int& a, int& b) {
  for (a = 0; a < nb2; ++a) {
    const int cnt = nb2 - 1 - a;
    if (q < cnt) { b = a + 1 + q; return; }
    q -= cnt;
  }
  a = b = 0;
}

// Launch 1: items [0, nquad * qsplit) are quad token-splits (split-major: the
// quads of token range 0 first), the next nb2 items are strips (all tokens).
__global__ __launch_bounds__(256) void syrk_main_kernel(const uint16_t* __restrict__ X, int64_t n, int64_t k,
                                                        int64_t ldx, float* __restrict__ H,
                                                        float* __restrict__ partial, int nquad, int qsplit,
                                                        int64_t qtokens) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int nb2 = (int)((k + QUAD - 1) / QUAD);
  const int item = blockIdx.x;
  if (item < nquad * qsplit) {
    const int sp = item / nquad, q = item % nquad;
    int a, b;
    quad_coords(q, nb2, a, b);
    const int64_t t0 = (int64_t)sp * qtokens;
    float* P = qsplit > 1 ? partial + (size_t)item * kSlotFloats : nullptr;
    tile_job<QUAD, QUAD>(lds, X, k, ldx, (int64_t)a * QUAD, (int64_t)b * QUAD, t0, min(n, t0 + qtokens), H, P);
  } else {
    const int a = item - nquad * qsplit;
    tile_job<HALF, QUAD>(lds, X, k, ldx, (int64_t)a * QUAD, (int64_t)a * QUAD, 0, n, H, nullptr);
  }
}

// Launch 2: singles (bottom-right diagonal 128-block of 256-block a), split
// over tokens when they are too few to fill the device.
__global__ __launch_bounds__(256) void syrk_single_kernel(const uint16_t* __restrict__ X, int64_t n, int64_t k,
                                                          int64_t ldx, float* __restrict__ H,
                                                          float* __restrict__ partial, int nsplit,
                                                          int64_t stokens, size_t slot_base) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int a = blockIdx.x;
  const int64_t c0 = (int64_t)a * QUAD + HALF;
  const int64_t t0 = (int64_t)blockIdx.y * stokens;
  float* P = nsplit > 1 ? partial + (slot_base + (size_t)blockIdx.x * nsplit + blockIdx.y) * kSlotFloats : nullptr;
  tile_job<HALF, HALF>(lds, X, k, ldx, c0, c0, t0, min(n, t0 + stokens), H, P);
}

// Sum the token splits of a tile in split order and add into H (upper
// triangle + mirror).  Partial slot of split sp of tile t:
// slot_base + sp * sstride + t * tstride.
__global__ __launch_bounds__(256) void syrk_reduce_kernel(int64_t k, float* __restrict__ H,
                                                          const float* __restrict__ partial, int kind, int nsplit,
                                                          size_t slot_base, size_t sstride, size_t tstride) {
  const int nb2 = (int)((k + QUAD - 1) / QUAD);
  int64_t r0, c0;
  int TM, TN;
  if (kind == 0) {
    int a, b;
    quad_coords(blockIdx.x, nb2, a, b);
    r0 = (int64_t)a * QUAD; c0 = (int64_t)b * QUAD; TM = QUAD; TN = QUAD;
  } else {
    r0 = c0 = (int64_t)blockIdx.x * QUAD + HALF; TM = HALF; TN = HALF;
  }
  const float* P = partial + (slot_base + (size_t)blockIdx.x * tstride) * kSlotFloats;
  const int rows_per = TM / gridDim.y;
  for (int e = threadIdx.x; e < rows_per * TN; e += 256) {
    const int row = blockIdx.y * rows_per + e / TN, col = e % TN;
    const int64_t gi = r0 + row, gj = c0 + col;
    if (gi >= k || gj >= k || gi > gj) continue;
    float s = 0.0f;
    for (int sp = 0; sp < nsplit; ++sp) s += P[(size_t)sp * sstride * kSlotFloats + row * TN + col];
    const float v = H[gi * k + gj] + s;
    H[gi * k + gj] = v;
    if (gi != gj) H[gj * k + gi] = v;
  }
}

__global__ void symmetrize_kernel(float* H, int64_t k) {
  int64_t i = blockIdx.y, j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j < k && j < i) H[i * k + j] = H[j * k + i];
}

struct SyrkPlan {
  int nb2, nquad, qsplit, nsingle, ssplit;
  int64_t qtokens, stokens;
  size_t slots;
};

int num_cus() {
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
  }
  return cus;
}

SyrkPlan plan(int64_t n, int64_t k, int cus) {
  SyrkPlan p;
  p.nb2 = (int)((k + QUAD - 1) / QUAD);
  p.nquad = p.nb2 * (p.nb2 - 1) / 2;
  p.nsingle = 0;
  for (int a = 0; a < p.nb2; ++a)
    if ((int64_t)a * QUAD + HALF < k) ++p.nsingle;
  int64_t nstages = (n + ST - 1) / ST;
  if (nstages < 1) nstages = 1;
  // A quad over half the tokens and a strip are equal work.  Split the quads
  // over tokens while the first launch would not give every CU an item.
  p.qsplit = 1;
  if (p.nquad > 0 && p.nquad + p.nb2 < cus) {
    int64_t s = (cus - p.nb2 + p.nquad - 1) / p.nquad;
    if (s > nstages) s = nstages;
    p.qsplit = (int)(s < 1 ? 1 : s);
  }
  p.ssplit = 1;
  if (p.nsingle > 0 && p.nsingle < cus) {
    int64_t s = cus / p.nsingle;
    if (s > nstages) s = nstages;
    p.ssplit = (int)(s < 1 ? 1 : s);
  }
  p.qtokens = ((nstages + p.qsplit - 1) / p.qsplit) * ST;
  p.stokens = ((nstages + p.ssplit - 1) / p.ssplit) * ST;
  p.slots = (p.qsplit > 1 ? (size_t)p.nquad * p.qsplit : 0) + (p.ssplit > 1 ? (size_t)p.nsingle * p.ssplit : 0);
  return p;
}

}  // namespace

size_t syrk_bf16_workspace(int64_t n, int64_t k) {
  SyrkPlan p = plan(n, k, num_cus());
  return p.slots * kSlotFloats * sizeof(float);
}

hipError_t syrk_bf16(const uint16_t* X, int64_t n, int64_t k, int64_t ldx, float* H, void* ws, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  SyrkPlan p = plan(n, k, num_cus());
  float* partial = (float*)ws;
  constexpr int main_stage = Tile<QUAD, QUAD>::STAGE_BYTES > Tile<HALF, QUAD>::STAGE_BYTES
                                 ? Tile<QUAD, QUAD>::STAGE_BYTES
                                 : Tile<HALF, QUAD>::STAGE_BYTES;
  const size_t lds_main = (size_t)NS * main_stage;
  const size_t lds_single = (size_t)NS * Tile<HALF, HALF>::STAGE_BYTES;
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute((const void*)syrk_main_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds_main);
    (void)hipFuncSetAttribute((const void*)syrk_single_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds_single);
    attr = true;
  }
  const int items = p.nquad * p.qsplit + p.nb2;
  hipLaunchKernelGGL(syrk_main_kernel, dim3(items), dim3(256), lds_main, s, X, n, k, ldx, H, partial, p.nquad,
                     p.qsplit, p.qtokens);
  size_t slot = 0;
  if (p.qsplit > 1) {
    // split sp of quad q sits in slot sp * nquad + q
    hipLaunchKernelGGL(syrk_reduce_kernel, dim3(p.nquad, 16), dim3(256), 0, s, k, H, partial, 0, p.qsplit, (size_t)0,
                       (size_t)p.nquad, (size_t)1);
    slot += (size_t)p.nquad * p.qsplit;
  }
  if (p.nsingle > 0) {
    hipLaunchKernelGGL(syrk_single_kernel, dim3(p.nsingle, p.ssplit), dim3(256), lds_single, s, X, n, k, ldx, H,
                       partial, p.ssplit, p.stokens, slot);
    if (p.ssplit > 1)
      hipLaunchKernelGGL(syrk_reduce_kernel, dim3(p.nsingle, 8), dim3(256), 0, s, k, H, partial, 1, p.ssplit, slot,
                         (size_t)1, (size_t)p.ssplit);
  }
  return hipGetLastError();
}

hipError_t symmetrize_from_upper(float* H, int64_t k, hipStream_t s) {
  hipLaunchKernelGGL(symmetrize_kernel, dim3((unsigned)((k + 255) / 256), (unsigned)k), dim3(256), 0, s, H, k);
  return hipGetLastError();
}

}  // namespace nvq
