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
// Operand staging.  X is row-major [tokens][channels] but an MFMA operand
// needs 8 consecutive tokens of one channel per lane, so every 64-token stage
// is transposed on the way into LDS: each thread loads 8 tokens x 4 channels
// with 8-byte loads (coalesced along channels), regroups them with v_perm into
// four 16-byte channel fragments and stores those into [channel][token] rows.
// Rows are 128 bytes with the 16-byte slot index rotated by a function of the
// channel, which keeps both the fragment stores and the MFMA operand reads
// free of bank conflicts.  Two LDS buffers alternate so the global loads of
// stage s+1 are in flight while stage s is multiplied.
#include "common.h"
#include "kernels.h"

namespace nvq {

namespace {

constexpr int ST = 64;        // tokens per stage
constexpr int TM = 128;       // rows (channels) of a job tile
constexpr int SLOT_FLOATS = 128 * 256;

__device__ __forceinline__ int rot(int c) { return (c + (c >> 3)) & 7; }

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
  static constexpr int TN = WIDE ? 256 : 128;              // columns of the job tile
  static constexpr int UNITS = (TM / 4) * 8 + (TN / 4) * 8; // (quad, token-group) units
  static constexpr int UPT = UNITS / 256;                    // units per thread
  static constexpr int A_WORDS = TM * 32;                    // u32 words per stage
  static constexpr int B_WORDS = TN * 32;
  static constexpr int NJ = TN / 64;                         // 32-col MFMA tiles per wave
};

template <bool WIDE>
__global__ __launch_bounds__(256) void syrk_bf16_kernel(const uint16_t* __restrict__ X, int64_t n,
                                                        int64_t k, int64_t ldx, float* __restrict__ H,
                                                        float* __restrict__ partial, int nsplit,
                                                        int64_t split_tokens, int slot_base) {
  using C = Cfg<WIDE>;
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  constexpr int STAGE_WORDS = C::A_WORDS + C::B_WORDS;   // [A rows | B rows] per buffer

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

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;

  // Per-unit source description (constant over stages).
  int u_is_b[C::UPT], u_quad[C::UPT], u_tg[C::UPT];
  const uint16_t* u_src[C::UPT];
  bool u_chan_ok[C::UPT];
#pragma unroll
  for (int u = 0; u < C::UPT; ++u) {
    int gu = u * 256 + tid;
    int isb = gu >= 256;
    int lu = isb ? gu - 256 : gu;
    int nq = isb ? C::TN / 4 : TM / 4;
    u_is_b[u] = isb;
    u_quad[u] = lu % nq;
    u_tg[u] = lu / nq;
    int64_t ch = (isb ? colc0 : rowc0) + 4 * u_quad[u];
    u_chan_ok[u] = ch < k;
    u_src[u] = X + ch;
  }

  u32x2 pre[C::UPT][8];
  auto load_stage = [&](int64_t t0) {
#pragma unroll
    for (int u = 0; u < C::UPT; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        int64_t t = t0 + u_tg[u] * 8 + i;
        u32x2 v = {0u, 0u};
        if (u_chan_ok[u] && t < t_end) v = *(const u32x2*)(u_src[u] + t * ldx);
        pre[u][i] = v;
      }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int u = 0; u < C::UPT; ++u) {
      uint32_t* base = lds + buf * STAGE_WORDS + (u_is_b[u] ? C::A_WORDS : 0);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        // channel c of the quad: low (c even) or high (c odd) half of word c/2
        const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
        u32x4 f;
#pragma unroll
        for (int w = 0; w < 4; ++w)
          f[w] = __builtin_amdgcn_perm(pre[u][2 * w + 1][c >> 1], pre[u][2 * w][c >> 1], sel);
        int row = 4 * u_quad[u] + c;
        int slot = (u_tg[u] + rot(row)) & 7;
        *(u32x4*)(base + row * 32 + slot * 4) = f;
      }
    }
  };

  f32x16 acc[2][C::NJ];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < C::NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nstages = (int)((t_end - t_begin + ST - 1) / ST);
  if (nstages > 0) {
    load_stage(t_begin);
    store_stage(0);
  }
  __syncthreads();
  for (int s = 0; s < nstages; ++s) {
    const int cur = s & 1;
    if (s + 1 < nstages) load_stage(t_begin + (int64_t)(s + 1) * ST);
    const uint32_t* A = lds + cur * STAGE_WORDS;
    const uint32_t* B = A + C::A_WORDS;
#pragma unroll
    for (int kk = 0; kk < ST / 16; ++kk) {
      const int tg = 2 * kk + (lane >> 5);
      bf16x8 a[2], b[C::NJ];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        int row = wr * 64 + i * 32 + (lane & 31);
        u32x4 w = *(const u32x4*)(A + row * 32 + ((tg + rot(row)) & 7) * 4);
        a[i] = __builtin_bit_cast(bf16x8, w);
      }
#pragma unroll
      for (int j = 0; j < C::NJ; ++j) {
        int row = wc * (C::TN / 2) + j * 32 + (lane & 31);
        u32x4 w = *(const u32x4*)(B + row * 32 + ((tg + rot(row)) & 7) * 4);
        b[j] = __builtin_bit_cast(bf16x8, w);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < C::NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (s + 1 < nstages) store_stage(cur ^ 1);
    __syncthreads();
  }

  // Epilogue.  Accumulator element (lane l, register r) of a 32x32 tile is at
  // row 8*(r/4) + 4*(l/32) + r%4, column l%32.
  if (nsplit == 1) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < C::NJ; ++j) {
        int64_t gj = colc0 + wc * (C::TN / 2) + j * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          int64_t gi = rowc0 + wr * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (gi < k && gj < k && gi <= gj) {
            float v = H[gi * k + gj] + acc[i][j][r];
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
      for (int j = 0; j < C::NJ; ++j) {
        int col = wc * (C::TN / 2) + j * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          int row = wr * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          P[row * 256 + col] = acc[i][j][r];
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
  const size_t lds_wide = 2 * (Cfg<true>::A_WORDS + Cfg<true>::B_WORDS) * sizeof(uint32_t);
  const size_t lds_narrow = 2 * (Cfg<false>::A_WORDS + Cfg<false>::B_WORDS) * sizeof(uint32_t);
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
