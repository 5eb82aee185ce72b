// Hessian accumulation H += X^T X for bf16 activations on CDNA4 matrix cores
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation; bf16 x bf16 products are exact).
//
// Work decomposition.  H is cut into 128x128 blocks; only blocks on or above
// the diagonal are computed.  In each block row I the blocks I..nb-1 are
// paired left to right into 128x256 "pair" jobs; an odd count leaves one
// 128x128 "single" job (always in the last block column).  A workgroup (4
// waves, each a 64x128 sub-tile = 2x4 MFMA 32x32 accumulators) owns one job
// for a contiguous token range.  When the jobs alone cannot fill the device
// the token range is split, partial tiles go to the workspace, and a second
// kernel sums the splits in a fixed order, so results are reproducible.
//
// Operand staging.  X is row-major [tokens][channels]; an MFMA operand needs
// 8 consecutive tokens of one channel per lane.  Tokens are streamed in
// 32-token stages through a ring of six LDS buffers filled by buffer loads
// that write LDS directly (no registers, no per-load address arithmetic; the
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

constexpr int ST = 32;        // tokens per stage
constexpr int NS = 6;         // ring depth (stages in flight + the one being multiplied)
constexpr int TM = 128;       // rows (channels) of a job tile
constexpr int SLOT_FLOATS = 128 * 256;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
#define LDS_AS __attribute__((address_space(3)))

// Physical 16-byte chunk of logical chunk p in tile row r, and its inverse.
// g(p) = p ^ ((p & 2) << 2) moves chunk bit 1 into bit 3 (an involution);
// the row index then XORs bits 1..3.
__device__ __forceinline__ int swz(int p, int r) { return (p ^ ((p & 2) << 2)) ^ (2 * (r & 7)); }
__device__ __forceinline__ int unswz(int pc, int r) {
  const int y = pc ^ (2 * (r & 7));
  return y ^ ((y & 2) << 2);
}

// (I, J) of pair job p: block row I, first block column J (covers J, J+1).
__device__ __forceinline__ void pair_job(int p, int nb, int& I, int& J) {
  for (I = 0; I < nb; ++I) {
    int np = (nb - I) >> 1;
    if (p < np) { J = I + 2 * p; return; }
    p -= np;
  }
  I = J = 0;
}

template <bool WIDE>
struct Cfg {
  static constexpr int TN = WIDE ? 256 : 128;          // columns of the job tile
  static constexpr int A_ROWB = TM * 2, B_ROWB = TN * 2; // bytes per token row
  static constexpr int A_BYTES = ST * A_ROWB, B_BYTES = ST * B_ROWB;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int INSTR = STAGE_BYTES / 1024;        // 1 KB direct-to-LDS loads per stage
  static constexpr int PER_WAVE = INSTR / 4;
  static constexpr int NJ = TN / 64;                      // 32-col MFMA tiles per wave
};

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
template <int NJ, int PER_WAVE, int A_ROWB, int B_ROWB>
__device__ __forceinline__ void stage_step(char* __restrict__ dst, bool issue, const void* src, int nrec,
                                           const uint32_t (&voff)[PER_WAVE], const int (&ldsoff)[PER_WAVE],
                                           const char* __restrict__ buf, const int (&aoff)[2][2],
                                           const int (&boff)[NJ][2], f32x16 (&acc)[2][NJ]) {
  if (issue) issue_loads<PER_WAVE>(dst, src, nrec, voff, ldsoff);
#pragma unroll
  for (int kk = 0; kk < ST / 16; ++kk) {
    bf16x8 a[2], b[NJ];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(buf + aoff[f][0] + kk * 16 * A_ROWB));
      s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(buf + aoff[f][1] + kk * 16 * A_ROWB));
      a[f] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
#pragma unroll
    for (int f = 0; f < NJ; ++f) {
      s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(buf + boff[f][0] + kk * 16 * B_ROWB));
      s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(buf + boff[f][1] + kk * 16 * B_ROWB));
      b[f] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int f = 0; f < NJ; ++f)
        acc[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[f], acc[i][f], 0, 0, 0);
  }
}

template <bool WIDE>
__global__ __launch_bounds__(256) void syrk_bf16_kernel(const uint16_t* __restrict__ X, int64_t n,
                                                        int64_t k, int64_t ldx, float* __restrict__ H,
                                                        float* __restrict__ partial, int nsplit,
                                                        int64_t split_tokens, int slot_base) {
  using C = Cfg<WIDE>;
  extern __shared__ __attribute__((aligned(1024))) char lds[];

  const int nb = (int)((k + 127) / 128);
  int I, J;
  if (WIDE) {
    pair_job(blockIdx.x, nb, I, J);
  } else {
    I = nb - 1 - 2 * (int)blockIdx.x;
    J = nb - 1;
  }
  const int64_t rowc0 = (int64_t)I * 128, colc0 = (int64_t)J * 128;
  const int64_t t_begin = (int64_t)blockIdx.y * split_tokens;
  const int64_t t_end = min(n, t_begin + split_tokens);
  const int nstages = t_end > t_begin ? (int)((t_end - t_begin + ST - 1) / ST) : 0;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;

  // This lane's source offset (bytes from the stage's first token row) for
  // each of the wave's load instructions, and the LDS chunk it fills.
  uint32_t voff[C::PER_WAVE];
  int ldsoff[C::PER_WAVE];
#pragma unroll
  for (int q = 0; q < C::PER_WAVE; ++q) {
    const int ins = wave + 4 * q;                       // instruction index in the stage
    const int off = ins * 1024 + lane * 16;             // byte offset in the stage buffer
    const bool is_b = off >= C::A_BYTES;
    const int toff = is_b ? off - C::A_BYTES : off;
    const int rowb = is_b ? C::B_ROWB : C::A_ROWB;
    const int r = toff / rowb, pc = (toff % rowb) / 16;
    const int p = unswz(pc, r);                         // logical chunk: channels 8p..8p+7
    const int64_t ch = (is_b ? colc0 : rowc0) + 8 * p;
    voff[q] = (uint32_t)(r * ldx * 2 + ch * 2);
    ldsoff[q] = ins * 1024;
  }
  // Per-lane LDS byte offsets of the transposed operand reads, for each
  // fragment f and half h (tokens 4h..4h+3 of the lane group's 8), k-step 0.
  const int g = lane >> 4, j = lane & 15;
  int aoff[2][2], boff[C::NJ][2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = 8 * (g >> 1) + 4 * h + (j >> 2);
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int ch = wr * 64 + f * 32 + 16 * (g & 1) + 4 * (j & 3);
      aoff[f][h] = r * C::A_ROWB + swz(ch >> 3, r) * 16 + 8 * (j & 1);
    }
#pragma unroll
    for (int f = 0; f < C::NJ; ++f) {
      const int ch = wc * (C::TN / 2) + f * 32 + 16 * (g & 1) + 4 * (j & 3);
      boff[f][h] = C::A_BYTES + r * C::B_ROWB + swz(ch >> 3, r) * 16 + 8 * (j & 1);
    }
  }

  f32x16 acc[2][C::NJ];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int f = 0; f < C::NJ; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][f][r] = 0.0f;

  for (int s = 0; s < NS - 1 && s < nstages; ++s) {
    const int64_t t0 = t_begin + (int64_t)s * ST;
    issue_loads<C::PER_WAVE>(lds + (s % NS) * C::STAGE_BYTES, (const void*)(X + t0 * ldx),
                             (int)min((t_end - t0) * ldx * 2, (int64_t)0x7FFFFFF0), voff, ldsoff);
  }
  for (int s = 0; s < nstages; ++s) {
    // Wait until this wave's loads of stage s have landed (later stages may
    // stay in flight), then make every wave's loads visible.
    const int ahead = min(NS - 2, nstages - 1 - s);     // stages issued after s
    switch (ahead * C::PER_WAVE) {
#define NVQ_WAIT(N) case N: __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14)); break;
      NVQ_WAIT(0) NVQ_WAIT(4) NVQ_WAIT(6) NVQ_WAIT(8) NVQ_WAIT(12) NVQ_WAIT(16) NVQ_WAIT(18) NVQ_WAIT(24)
#undef NVQ_WAIT
      default: __builtin_amdgcn_s_waitcnt(0); break;
    }
    // Plain workgroup barrier (the memory clobber keeps the compiler from
    // moving LDS accesses across it).  __syncthreads() would add a release
    // fence that drains the loads of the stages still in flight.
    asm volatile("s_barrier" ::: "memory");
    const int sn = s + NS - 1;
    const bool issue = sn < nstages;
    const int64_t t0 = t_begin + (int64_t)sn * ST;
    const int64_t rem = issue ? (t_end - t0) * ldx * 2 : 0;
    stage_step<C::NJ, C::PER_WAVE, C::A_ROWB, C::B_ROWB>(lds + (sn % NS) * C::STAGE_BYTES, issue,
                                                        (const void*)(X + (issue ? t0 : t_begin) * ldx),
                                                        (int)min(rem, (int64_t)0x7FFFFFF0), voff, ldsoff,
                                                        lds + (s % NS) * C::STAGE_BYTES, aoff, boff, acc);
  }

  // Epilogue.  Accumulator element (lane l, register r) of a 32x32 tile is at
  // row 8*(r/4) + 4*(l/32) + r%4, column l%32.
  if (nsplit == 1) {
    // Read the old upper-triangle values first, then store (stores to H would
    // otherwise serialize the loads behind them).
    float old[2][C::NJ][16];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int f = 0; f < C::NJ; ++f) {
        int64_t gj = colc0 + wc * (C::TN / 2) + f * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          int64_t gi = rowc0 + wr * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          old[i][f][r] = (gi < k && gj < k && gi <= gj) ? H[gi * k + gj] : 0.0f;
        }
      }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int f = 0; f < C::NJ; ++f) {
        int64_t gj = colc0 + wc * (C::TN / 2) + f * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          int64_t gi = rowc0 + wr * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (gi < k && gj < k && gi <= gj) {
            float v = old[i][f][r] + acc[i][f][r];
            H[gi * k + gj] = v;
            if (gi != gj) H[gj * k + gi] = v;
          }
        }
      }
  } else {
    float* P = partial + ((int64_t)slot_base + (int64_t)blockIdx.x * nsplit + blockIdx.y) * SLOT_FLOATS;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int f = 0; f < C::NJ; ++f) {
        int col = wc * (C::TN / 2) + f * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          int row = wr * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          P[row * 256 + col] = acc[i][f][r];
        }
      }
  }
}

// Sum the token splits of each job in split order and add into H (upper
// triangle + mirror).
template <bool WIDE>
__global__ __launch_bounds__(256) void syrk_reduce_kernel(int64_t k, float* __restrict__ H,
                                                          const float* __restrict__ partial,
                                                          int nsplit, int slot_base) {
  constexpr int TN = WIDE ? 256 : 128;
  const int nb = (int)((k + 127) / 128);
  int I, J;
  if (WIDE) {
    pair_job(blockIdx.x, nb, I, J);
  } else {
    I = nb - 1 - 2 * (int)blockIdx.x;
    J = nb - 1;
  }
  const float* P = partial + ((int64_t)slot_base + (int64_t)blockIdx.x * nsplit) * SLOT_FLOATS;
  const int rows_per = TM / gridDim.y;
  for (int e = threadIdx.x; e < rows_per * TN; e += 256) {
    int row = blockIdx.y * rows_per + e / TN, col = e % TN;
    int64_t gi = (int64_t)I * 128 + row, gj = (int64_t)J * 128 + col;
    if (gi >= k || gj >= k || gi > gj) continue;
    float s = 0.0f;
    for (int sp = 0; sp < nsplit; ++sp) s += P[(int64_t)sp * SLOT_FLOATS + row * 256 + col];
    float v = H[gi * k + gj] + s;
    H[gi * k + gj] = v;
    if (gi != gj) H[gj * k + gi] = v;
  }
}

__global__ void symmetrize_kernel(float* H, int64_t k) {
  int64_t i = blockIdx.y, j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j < k && j < i) H[i * k + j] = H[j * k + i];
}

struct SyrkPlan {
  int nb, npairs, nsingles, split_p, split_s;
  int64_t tok_p, tok_s;
  int64_t slots;
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
  p.nb = (int)((k + 127) / 128);
  p.npairs = 0;
  for (int I = 0; I < p.nb; ++I) p.npairs += (p.nb - I) / 2;
  p.nsingles = (p.nb + 1) / 2;
  int64_t nstages = (n + ST - 1) / ST;
  if (nstages < 1) nstages = 1;
  auto pick = [&](int jobs) -> int {
    if (jobs <= 0) return 1;
    int64_t s = jobs >= cus ? 1 : cus / jobs;
    if (s > nstages) s = nstages;
    return (int)(s < 1 ? 1 : s);
  };
  p.split_p = pick(p.npairs);
  p.split_s = pick(p.nsingles);
  p.tok_p = ((nstages + p.split_p - 1) / p.split_p) * ST;
  p.tok_s = ((nstages + p.split_s - 1) / p.split_s) * ST;
  p.slots = (p.split_p > 1 ? (int64_t)p.npairs * p.split_p : 0) +
            (p.split_s > 1 ? (int64_t)p.nsingles * p.split_s : 0);
  return p;
}

}  // namespace

size_t syrk_bf16_workspace(int64_t n, int64_t k) {
  SyrkPlan p = plan(n, k, num_cus());
  return (size_t)p.slots * SLOT_FLOATS * sizeof(float);
}

hipError_t syrk_bf16(const uint16_t* X, int64_t n, int64_t k, int64_t ldx, float* H, void* ws,
                     hipStream_t s) {
  if (n <= 0) return hipSuccess;
  SyrkPlan p = plan(n, k, num_cus());
  float* partial = (float*)ws;
  const size_t lds_wide = (size_t)NS * Cfg<true>::STAGE_BYTES;
  const size_t lds_narrow = (size_t)NS * Cfg<false>::STAGE_BYTES;
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute((const void*)syrk_bf16_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds_wide);
    (void)hipFuncSetAttribute((const void*)syrk_bf16_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds_narrow);
    attr = true;
  }
  int slot = 0;
  if (p.npairs > 0) {
    hipLaunchKernelGGL(syrk_bf16_kernel<true>, dim3(p.npairs, p.split_p), dim3(256), lds_wide, s, X, n, k,
                       ldx, H, partial, p.split_p, p.tok_p, slot);
    if (p.split_p > 1) {
      hipLaunchKernelGGL(syrk_reduce_kernel<true>, dim3(p.npairs, 8), dim3(256), 0, s, k, H, partial,
                         p.split_p, slot);
      slot += p.npairs * p.split_p;
    }
  }
  if (p.nsingles > 0) {
    hipLaunchKernelGGL(syrk_bf16_kernel<false>, dim3(p.nsingles, p.split_s), dim3(256), lds_narrow, s, X, n,
                       k, ldx, H, partial, p.split_s, p.tok_s, slot);
    if (p.split_s > 1)
      hipLaunchKernelGGL(syrk_reduce_kernel<false>, dim3(p.nsingles, 8), dim3(256), 0, s, k, H, partial,
                         p.split_s, slot);
  }
  return hipGetLastError();
}

hipError_t symmetrize_from_upper(float* H, int64_t k, hipStream_t s) {
  hipLaunchKernelGGL(symmetrize_kernel, dim3((unsigned)((k + 255) / 256), (unsigned)k), dim3(256), 0, s, H, k);
  return hipGetLastError();
}

}  // namespace nvq
