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
// A quad moves 512 channels per token for 65536 products.  Strips and
// singles lie on the diagonal (their rows are the first of their columns), so
// they load only their columns' channels and read both operands from them:
// 256 channels for 32768 products, and 128 for 16384.  The first launch runs
// quads and strip pairs (two strips one after the other), split over token
// ranges until there is an item per CU (for a 4096-channel layer: 2 ranges x
// (120 quads + 8 strip pairs) = 256 items).  A strip pair still takes longer
// than a quad (half its products per LDS read and per barrier), so it covers
// only the head of its range there; the rest of the range runs as pieces in
// the second launch, beside the singles, which are split over tokens.  Items
// are ordered so that each XCD holds one token range and a compact group of
// tiles, which keeps most operand reads inside its L2.  Split tiles write
// partial sums to the workspace, summed in a fixed order by a reduction
// kernel, so results are reproducible.
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
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace nvq {

namespace {

constexpr int ST = 32;       // tokens per stage
constexpr int NS = 4;        // ring depth (stages in flight + the one being multiplied)
constexpr int HEAD16 = 13;   // sixteenths of a token range a strip pair covers in the first launch
constexpr int TSPLIT = 4;                 // tail pieces per (range, strip pair)

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

// A TM x TN tile of H: a stage holds ST token rows of the A operand (TM
// channels) and then of the B operand (TN channels).  A diagonal tile (D:
// rows and columns start at the same channel, TM <= TN) loads only B and
// reads A from B's first TM channels.
template <int TM, int TN, bool D = false>
struct Tile {
  static_assert(!D || TM <= TN, "a diagonal tile's rows are a prefix of its columns");
  static constexpr int A_ROWB = D ? TN * 2 : TM * 2, B_ROWB = TN * 2;   // bytes per token row of A's and B's region
  static constexpr int A_BYTES = D ? 0 : ST * A_ROWB, B_BYTES = ST * B_ROWB;
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

// Operand fragments of k-step kk (16 tokens) of the stage in buf.
template <int TM, int TN, bool D>
__device__ __forceinline__ void read_frags(const char* buf, int kk, const int (&aoff)[Tile<TM, TN, D>::NI][2],
                                           const int (&boff)[Tile<TM, TN, D>::NJ][2], bf16x8 (&a)[Tile<TM, TN, D>::NI],
                                           bf16x8 (&b)[Tile<TM, TN, D>::NJ]) {
  using T = Tile<TM, TN, D>;
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
}

// Fragment f of k-step kk of the stage in buf: f < NI is A fragment f,
// otherwise B fragment f - NI.
template <int TM, int TN, bool D>
__device__ __forceinline__ void read_one(const char* buf, int kk, int f, const int (&aoff)[Tile<TM, TN, D>::NI][2],
                                         const int (&boff)[Tile<TM, TN, D>::NJ][2], bf16x8 (&a)[Tile<TM, TN, D>::NI],
                                         bf16x8 (&b)[Tile<TM, TN, D>::NJ]) {
  using T = Tile<TM, TN, D>;
  if (f < T::NI) {
    s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(buf + aoff[f][0] + kk * 16 * T::A_ROWB));
    s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(buf + aoff[f][1] + kk * 16 * T::A_ROWB));
    a[f] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  } else {
    const int g = f - T::NI;
    s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(buf + boff[g][0] + kk * 16 * T::B_ROWB));
    s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(buf + boff[g][1] + kk * 16 * T::B_ROWB));
    b[g] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
}

// One stage's direct-to-LDS load q of this wave (see issue_loads).
__device__ __forceinline__ void issue_load_one(char* dst, const void* src, int nrec, uint32_t voff, int ldsoff) {
#if __HIP_DEVICE_COMPILE__
  __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, nrec, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(dst + ldsoff), 16, voff, 0, 0, 0);
#endif
}

// One pipeline step over stage s, whose LDS slot is `slot`; on entry (a0, b0)
// hold the operand fragments of its first k-step.  First half: the products
// of the first k-step, interleaved with the reads of the second k-step's
// fragments (one fragment per product, early in the half).  Then the wave
// waits for those reads and for its own loads of stage s+1 (vmcnt <= WAIT)
// and joins the workgroup barrier: every wave's loads of stage s+1 have
// landed and every wave is done reading stage s.  Second half: the products
// of the second k-step, interleaved with the refill of `slot` (direct-to-LDS
// loads of stage s+NS, zero-length past the end, so every step issues the
// same number of loads) and the reads of stage s+1's first fragments (from
// `nxt` into (a0, b0)).  Scheduling fences keep this order, so the matrix
// cores are never left waiting behind a burst of memory instructions.
// `slot` and `nxt` are distinct, which the restrict qualifiers state: the
// compiler then need not wait on the loads in flight before operand reads.
template <int TM, int TN, bool D, int WAIT, bool has_next>
__device__ __forceinline__ void pipe_step(char* __restrict__ slot, const char* __restrict__ nxt,
                                          const void* src, int nrec, const uint32_t (&voff)[Tile<TM, TN, D>::PER_WAVE],
                                          const int (&ldsoff)[Tile<TM, TN, D>::PER_WAVE],
                                          const int (&aoff)[Tile<TM, TN, D>::NI][2],
                                          const int (&boff)[Tile<TM, TN, D>::NJ][2], bf16x8 (&a0)[Tile<TM, TN, D>::NI],
                                          bf16x8 (&b0)[Tile<TM, TN, D>::NJ],
                                          f32x16 (&acc)[Tile<TM, TN, D>::NI][Tile<TM, TN, D>::NJ]) {
  using T = Tile<TM, TN, D>;
  static_assert(ST == 32, "two k-steps per stage");
  constexpr int NM = T::NI * T::NJ, NF = T::NI + T::NJ, NL = T::PER_WAVE;
  constexpr int N1 = NM > NF ? NM : NF;
  constexpr int N2 = N1 > NL ? N1 : NL;
  bf16x8 a1[T::NI], b1[T::NJ];
#pragma unroll
  for (int m = 0; m < N1; ++m) {
    if (m < NF) read_one<TM, TN, D>(slot, 1, m, aoff, boff, a1, b1);
    if (m < NM) acc[m / T::NJ][m % T::NJ] =
        __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[m / T::NJ], b0[m % T::NJ], acc[m / T::NJ][m % T::NJ], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (has_next) {
    constexpr int w = WAIT;
    __builtin_amdgcn_s_waitcnt((w & 15) | (7 << 4) | (0 << 8) | ((w >> 4) << 14));
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int m = 0; m < N2; ++m) {
    if constexpr (has_next) {
      if (m < NL) issue_load_one(slot, src, nrec, voff[m], ldsoff[m]);
      if (m < NF) read_one<TM, TN, D>(nxt, 0, m, aoff, boff, a0, b0);
    }
    if (m < NM) acc[m / T::NJ][m % T::NJ] =
        __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[m / T::NJ], b1[m % T::NJ], acc[m / T::NJ][m % T::NJ], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One tile job: rows [rowc0, rowc0+TM) x columns [colc0, colc0+TN) of H over
// tokens [t_begin, t_end).  P == nullptr: add into H (upper triangle + mirror);
// otherwise store the partial sums into P [TM x TN].  Channels at or past k
// may be read (they only feed accumulators of rows/columns >= k, which are
// never stored); reads stay inside X's rows thanks to the buffer bound.
template <int TM, int TN, bool D>
__device__ __forceinline__ void tile_job(char* lds, const uint16_t* __restrict__ X, int64_t k, int64_t ldx,
                                         int64_t rowc0, int64_t colc0, int64_t t_begin, int64_t t_end,
                                         float* __restrict__ H, float* __restrict__ P) {
  using T = Tile<TM, TN, D>;
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
  // Byte bound of the buffer that starts at stage `st` (0 past the end).
  auto stage_nrec = [&](int st) -> int {
    const int64_t t0 = t_begin + (int64_t)st * ST;
    return st < nstages ? (int)min((t_end - t0) * ldx * 2, (int64_t)0x7FFFFFF0) : 0;
  };
  auto stage_src = [&](int st) -> const void* {
    return (const void*)(X + (st < nstages ? t_begin + (int64_t)st * ST : t_begin) * ldx);
  };

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

  // Prologue: fill every slot (zero-length loads past the end), then read
  // stage 0's first fragments (the compiler also waits here for the other
  // prologue loads).
  for (int s = 0; s < NS; ++s)
    issue_loads<T::PER_WAVE>(lds + s * T::STAGE_BYTES, stage_src(s), stage_nrec(s), voff, ldsoff);
  bf16x8 a0[T::NI], b0[T::NJ];
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
  asm volatile("s_barrier" ::: "memory");
  read_frags<TM, TN, D>(lds, 0, aoff, boff, a0, b0);
  // Every step issues one stage of loads, so while the wave waits for stage
  // s+1 the loads of stages s+2..s+NS-1 are the ones it leaves in flight.
  constexpr int kWait = (NS - 2) * T::PER_WAVE;
  static_assert(NS >= 2 && kWait < 64, "ring depth");
  for (int s = 0; s + 1 < nstages; ++s) {
    const int sn = s + NS;
    pipe_step<TM, TN, D, kWait, true>(lds + (s % NS) * T::STAGE_BYTES, lds + ((s + 1) % NS) * T::STAGE_BYTES,
                                   stage_src(sn), stage_nrec(sn), voff, ldsoff, aoff, boff, a0, b0, acc);
  }
  if (nstages > 0) {
    const int s = nstages - 1;
    pipe_step<TM, TN, D, kWait, false>(lds + (s % NS) * T::STAGE_BYTES, lds, stage_src(s), 0, voff, ldsoff, aoff, boff,
                                    a0, b0, acc);
  }

  // The zero-length loads issued for stages past the end write LDS too: wait
  // for them, so that none is in flight once the workgroup's LDS is reused
  // (the next tile job) or released.
  __builtin_amdgcn_s_waitcnt(0);

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

// ---- Four-group tiles (layers of 16 segments) ---------------------------------
// A quad moves 4 groups of 128 channels per token for 4 group pairs.  A
// workgroup that loads 4 groups can instead multiply all 6 of their pairs
// (98304 products, 384 accumulator registers per lane), a third fewer bytes
// per product.  For 16 segments of 256 channels (32 groups, segment m holding
// groups 2m and 2m+1), the pairs of groups in different segments are covered
// exactly once by 80 such tiles: a group divisible design with block size 4
// and 16 groups of size 2 (Brouwer, Schrijver and Hanani, "Group divisible
// designs with block-size four", Discrete Math. 1977, show that it exists).
// This one was found by computer search as a design invariant under the shift
// x -> x + 4 (mod 32) of group indices: nine base blocks give orbits of 8
// blocks, and two blocks fixed by x -> x + 16 give orbits of 4.  The pairs
// inside a segment (its diagonal 256-block) stay with the strips and singles.
constexpr int K4_SEGS = 16, K4_TILES = 80, K4G = 128;
struct K4Table { uint8_t g[K4_TILES][4]; };
constexpr uint8_t kK4Base[9][4] = {{2, 12, 20, 29}, {0, 4, 7, 10}, {3, 11, 12, 24}, {0, 21, 27, 29}, {2, 4, 17, 30},
                                   {1, 11, 21, 28}, {1, 22, 29, 30}, {3, 15, 21, 30}, {3, 10, 22, 31}};
constexpr uint8_t kK4Fixed[2][4] = {{0, 2, 16, 18}, {1, 3, 17, 19}};
// Order of the tiles in the launch: consecutive items go to one XCD (32 per
// XCD, 80 per token range), so the order was chosen (by annealing) to keep
// the groups that each XCD's run of tiles touches few: 27-28 of the 32 for
// the runs of 32 and 20-21 for the runs of 16 (31-32 and 27-32 in orbit order).
// Entry i is the orbit-order index (8 shifts of the nine base blocks, then 4
// shifts of the two fixed ones) of tile i.
constexpr uint8_t kK4Order[K4_TILES] = {
    65, 8,  45, 61, 56, 49, 71, 38, 18, 36, 64, 11, 43, 1,  42, 74, 19, 40, 50, 79, 31, 75, 41, 52, 73, 51, 3,
    47, 68, 21, 27, 34, 16, 33, 57, 59, 7,  26, 20, 72, 39, 30, 32, 2,  67, 17, 69, 14, 22, 10, 24, 76, 23, 63,
    25, 37, 13, 44, 6,  15, 53, 28, 0,  9,  70, 5,  35, 12, 4,  77, 55, 48, 29, 46, 60, 78, 66, 58, 54, 62};
constexpr K4Table make_k4_table() {
  K4Table o{}, t{};
  int n = 0;
  for (int s = 0; s < 8; ++s)
    for (int b = 0; b < 9; ++b, ++n)
      for (int q = 0; q < 4; ++q) o.g[n][q] = (uint8_t)((kK4Base[b][q] + 4 * s) % 32);
  for (int s = 0; s < 4; ++s)
    for (int b = 0; b < 2; ++b, ++n)
      for (int q = 0; q < 4; ++q) o.g[n][q] = (uint8_t)(kK4Fixed[b][q] + 4 * s);
  for (int i = 0; i < K4_TILES; ++i)
    for (int q = 0; q < 4; ++q) t.g[i][q] = o.g[kK4Order[i]][q];
  for (int i = 0; i < K4_TILES; ++i)   // increasing group order within a tile
    for (int a = 1; a < 4; ++a)
      for (int c = a; c > 0 && t.g[i][c - 1] > t.g[i][c]; --c) {
        const uint8_t x = t.g[i][c];
        t.g[i][c] = t.g[i][c - 1];
        t.g[i][c - 1] = x;
      }
  return t;
}
// Every pair of groups in different segments lies in exactly one tile, and no
// tile holds both groups of a segment.
constexpr bool k4_table_ok(const K4Table& t) {
  int cnt[32][32] = {};
  for (int i = 0; i < K4_TILES; ++i)
    for (int a = 0; a < 4; ++a)
      for (int b = a + 1; b < 4; ++b) {
        if (t.g[i][a] / 2 == t.g[i][b] / 2 || t.g[i][a] >= t.g[i][b]) return false;
        ++cnt[t.g[i][a]][t.g[i][b]];
      }
  for (int a = 0; a < 32; ++a)
    for (int b = a + 1; b < 32; ++b)
      if (cnt[a][b] != (a / 2 == b / 2 ? 0 : 1)) return false;
  return true;
}
constexpr K4Table kK4Host = make_k4_table();
static_assert(k4_table_ok(kK4Host), "the four-group tiles must cover every cross-segment group pair once");
__constant__ K4Table kK4 = make_k4_table();

// Index of the pair of regions (a, b), a < b, in a tile's partial sums.
__host__ __device__ constexpr int k4_pair(int a, int b) { return a == 0 ? b - 1 : (a == 1 ? b + 1 : 5); }
constexpr size_t kK4SlotFloats = (size_t)6 * K4G * K4G;   // 1.5 quad slots
constexpr int K4_ROWB = K4G * 2;                          // bytes of a group's token row
constexpr int K4_REGION = ST * K4_ROWB;                   // one group's rows of a stage
constexpr int K4_STAGE = 4 * K4_REGION;
static_assert(K4_STAGE == Tile<QUAD, QUAD>::STAGE_BYTES, "same LDS ring as a quad");

// Wave roles.  A stage holds the tile's four groups as regions 0..3 (in
// increasing channel order).  Each wave multiplies one whole 128x128 block
// (rows region X, columns region Y) and half of another: with HALF 0 rows X
// times columns 0..63 of region Z, with HALF 1 rows Z times columns 64..127
// of region Y, with HALF 2 rows Z times columns 64..127 of region Z.  FB and
// HB number the two blocks in the tile's partial sums.
//   Four-group tiles (blocks numbered by k4_pair): wave 0 (0,1) and the left
//   half of (0,3); wave 1 (1,3) and the left half of (1,2); wave 2 (2,3) and
//   the right half of (0,3); wave 3 (0,2) and the right half of (1,2).  They
//   read 10, 10, 12 and 12 operand fragments per k-step for 24 products.
//   Diagonal tiles (the diagonal 256-blocks of two segments: regions 0,1 are
//   the first segment's groups, 2,3 the second's; blocks 0 (0,1), 1 (2,3),
//   2..5 the diagonal 128-blocks of regions 0..3): wave 0 (0,1) and the left
//   half of (0,0); wave 1 (2,3) and the left half of (2,2); wave 2 (1,1) and
//   the right half of (0,0); wave 3 (3,3) and the right half of (2,2).  They
//   read 8 fragments per k-step; a quarter of their products (those below
//   the diagonal blocks' diagonals) are not needed.
// Every block has its rows at or before its columns, so it lies in H's upper
// triangle.
template <int W_, int X_, int Y_, int Z_, int HALF_, int FB_, int HB_>
struct Role {
  static constexpr int W = W_, X = X_, Y = Y_, Z = Z_, HALF = HALF_, FB = FB_, HB = HB_;
  static constexpr bool YX = X_ == Y_;                 // the whole block is diagonal: Y's fragments are X's
  static constexpr bool ZX = HALF_ == 0 && Z_ == X_;   // the half block is diagonal: Z's fragments are X's
  static constexpr int NY = YX ? 0 : 4, NZ = ZX ? 0 : (HALF_ == 0 ? 2 : 4), NF = 4 + NY + NZ;
  static constexpr int HR = HALF_ == 0 ? X_ : Z_, HC = HALF_ == 1 ? Y_ : Z_, HC0 = HALF_ == 0 ? 0 : 64;
};
using K4W0 = Role<0, 0, 1, 3, 0, 0, 2>;
using K4W1 = Role<1, 1, 3, 2, 0, 4, 3>;
using K4W2 = Role<2, 2, 3, 0, 1, 5, 2>;
using K4W3 = Role<3, 0, 2, 1, 1, 1, 3>;
using DGW0 = Role<0, 0, 1, 0, 0, 0, 2>;
using DGW1 = Role<1, 2, 3, 2, 0, 1, 4>;
using DGW2 = Role<2, 1, 1, 0, 2, 3, 2>;
using DGW3 = Role<3, 3, 3, 2, 2, 5, 4>;
// Rows and columns region of block b of a diagonal tile.
__host__ __device__ constexpr int dg_row(int b) { return b == 0 ? 0 : (b == 1 ? 2 : b - 2); }
__host__ __device__ constexpr int dg_col(int b) { return b == 0 ? 1 : (b == 1 ? 3 : b - 2); }

// Region layout: [32 token rows][128 channels], 16-byte chunk p of row r
// stored at chunk p ^ 4 (r % 4).  A transposed fragment read (16 lanes: rows
// T + j/4, 8 bytes at channel C + 4 (j % 4)) then hits 64 distinct banks per
// 32 lanes, and since r % 4 is fixed per lane (T is a multiple of 4) a lane's
// address for fragment f is its own base for f plus immediates for the
// region, the half and the k-step.
__device__ __forceinline__ bf16x8 k4_frag(const char* buf, const int (&F)[4], int region, int f, int kk) {
  const char* p = buf + F[f] + region * K4_REGION + kk * 16 * K4_ROWB;
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)p);
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(p + 4 * K4_ROWB));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <class R>
struct K4Frags {
  bf16x8 x[4], y[R::NY > 0 ? R::NY : 1], z[R::NZ > 0 ? R::NZ : 1];
  __device__ __forceinline__ const bf16x8& yf(int j) const { if constexpr (R::YX) return x[j]; else return y[j]; }
  __device__ __forceinline__ const bf16x8& zf(int j) const { if constexpr (R::ZX) return x[j]; else return z[j]; }
};

// Fragment m of k-step kk: m < 4 region X, then region Y (unless it is X),
// then region Z (unless it is X).
template <class R>
__device__ __forceinline__ void k4_read(const char* buf, const int (&F)[4], int m, int kk, K4Frags<R>& fr) {
  if (m < 4) fr.x[m] = k4_frag(buf, F, R::X, m, kk);
  else if (m < 4 + R::NY) fr.y[m - 4] = k4_frag(buf, F, R::Y, m - 4, kk);
  else fr.z[m - 4 - R::NY] = k4_frag(buf, F, R::Z, m - 4 - R::NY, kk);
}

// The half block's eight accumulators (128 registers) live in VGPRs, the
// whole block's sixteen (256) in AGPRs: the compiler would put every product
// of a builtin into AGPRs, which 384 accumulators overflow.  So the half
// block's products are written as inline assembly with VGPR operands.  The
// compiler tracks their registers but not the matrix unit's hazards, so
// k4_mfma_fence waits out the longest pass count (16 passes plus the
// margin, 24 wait states) between them and any other access to their
// accumulators: after the zeroing and before the epilogue.
__device__ __forceinline__ void k4_mfma_fence(f32x16 (&accH)[4][2]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+v"(accH[0][0]), "+v"(accH[0][1]), "+v"(accH[1][0]), "+v"(accH[1][1]), "+v"(accH[2][0]),
                 "+v"(accH[2][1]), "+v"(accH[3][0]), "+v"(accH[3][1]));
}

__device__ __forceinline__ void k4_mfma_v(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}

// Product m: m < 16 the whole block's tile (m / 4, m % 4), then the half
// block's tile ((m - 16) / 2, (m - 16) % 2).
template <class R>
__device__ __forceinline__ void k4_mfma(int m, const K4Frags<R>& fr, f32x16 (&accF)[4][4], f32x16 (&accH)[4][2]) {
  if (m < 16) {
    accF[m / 4][m % 4] =
        __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr.x[m / 4], fr.yf(m % 4), accF[m / 4][m % 4], 0, 0, 0);
  } else {
    const int q = m - 16;
    if constexpr (R::HALF == 0) k4_mfma_v(accH[q / 2][q % 2], fr.x[q / 2], fr.zf(q % 2));
    else if constexpr (R::HALF == 1) k4_mfma_v(accH[q / 2][q % 2], fr.z[q / 2], fr.yf(2 + q % 2));
    else k4_mfma_v(accH[q / 2][q % 2], fr.z[q / 2], fr.z[2 + q % 2]);
  }
}

// Load q (0..7) of wave W for the stage at src (nrec bytes to the end of the
// token range, capped): token rows 4 (W + 4 (q % 2)) .. +3 of region q / 2,
// into LDS bytes (W + 4q) * 1024 of the stage.  The buffer starts at the
// region's first channel with its bound moved by the same bytes, so rows past
// the range still read as zeros; voff[q % 2] is the lane's row and (swizzled)
// chunk within the stage.
template <int W, int q>
__device__ __forceinline__ void k4_load(char* slot, const uint16_t* src, int nrec, const int64_t (&ch)[4],
                                        const uint32_t (&voff)[2]) {
#if __HIP_DEVICE_COMPILE__
  const int left = nrec - 2 * (int)ch[q >> 1];
  __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(src + ch[q >> 1]), (short)0, left > 0 ? left : 0, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(slot + (W + 4 * q) * 1024), 16, voff[q & 1], 0, 0, 0);
#endif
}

template <int W>
__device__ __forceinline__ void k4_loads(char* slot, const uint16_t* src, int nrec, const int64_t (&ch)[4],
                                         const uint32_t (&voff)[2], int m) {
  switch (m) {
    case 0: k4_load<W, 0>(slot, src, nrec, ch, voff); break;
    case 1: k4_load<W, 1>(slot, src, nrec, ch, voff); break;
    case 2: k4_load<W, 2>(slot, src, nrec, ch, voff); break;
    case 3: k4_load<W, 3>(slot, src, nrec, ch, voff); break;
    case 4: k4_load<W, 4>(slot, src, nrec, ch, voff); break;
    case 5: k4_load<W, 5>(slot, src, nrec, ch, voff); break;
    case 6: k4_load<W, 6>(slot, src, nrec, ch, voff); break;
    case 7: k4_load<W, 7>(slot, src, nrec, ch, voff); break;
    default: break;
  }
}

// One 32x32 accumulator tile at rows r0, columns c0 of block `blk` (rows
// from channel rch, columns from cch): into the tile's partial sums P
// [block][128][128], or added into H.  Off a diagonal block (rch < cch) every
// element and its mirror are written; on one (rch == cch) the upper triangle
// and the mirror of the strict upper triangle.
__device__ __forceinline__ void k4_store(const f32x16& acc, int blk, int r0, int c0, int64_t rch, int64_t cch,
                                         int64_t k, float* __restrict__ H, float* __restrict__ P,
                                         bool mirror = true) {
  const int lane = threadIdx.x & 63, col = c0 + (lane & 31);
  if (P) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = r0 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      P[(size_t)blk * K4G * K4G + row * K4G + col] = acc[r];
    }
    return;
  }
  const int64_t gj = cch + col;
  float old[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t gi = rch + r0 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    old[r] = (gi < k && gj < k && gi <= gj) ? H[gi * k + gj] : 0.0f;
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t gi = rch + r0 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    if (gi < k && gj < k && gi <= gj) {
      const float v = old[r] + acc[r];
      H[gi * k + gj] = v;
      if (mirror && gi != gj) H[gj * k + gi] = v;
    }
  }
}

// One pipeline step over a four-group stage (the order of pipe_step): the
// first k-step's 24 products interleaved with the second k-step's fragment
// reads, then the wait for stage s+1 and the barrier, then the second
// k-step's products interleaved with the refill of `slot` and the next
// stage's first fragments.  `slot` and `nxt` are distinct, which the restrict
// qualifiers state, so operand reads need not wait on the loads in flight.
template <class R, bool has_next>
__device__ __forceinline__ void k4_step(char* __restrict__ slot, const char* __restrict__ nxt, const uint16_t* src,
                                        int nrec, const int64_t (&ch)[4], const uint32_t (&voff)[2],
                                        const int (&F)[4], K4Frags<R>& f0, f32x16 (&accF)[4][4],
                                        f32x16 (&accH)[4][2]) {
  constexpr int NM = 24, NL = 8;
  constexpr int kWait = (NS - 2) * NL;
  static_assert(NS >= 2 && kWait < 64, "ring depth");
  K4Frags<R> f1;
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    if (m < R::NF) k4_read<R>(slot, F, m, 1, f1);
    k4_mfma<R>(m, f0, accF, accH);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (has_next) {
    __builtin_amdgcn_s_waitcnt((kWait & 15) | (7 << 4) | (0 << 8) | ((kWait >> 4) << 14));
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    if constexpr (has_next) {
      if (m < NL) k4_loads<R::W>(slot, src, nrec, ch, voff, m);
      if (m < R::NF) k4_read<R>(nxt, F, m, 0, f0);
    }
    k4_mfma<R>(m, f1, accF, accH);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <class R>
__device__ __forceinline__ void k4_wave(char* lds, const uint16_t* __restrict__ X, int64_t k, int64_t ldx,
                                        const int64_t (&ch)[4], int64_t t_begin, int64_t t_end,
                                        float* __restrict__ H, float* __restrict__ P, bool mirror) {
  constexpr int NL = 8;
  const int nstages = t_end > t_begin ? (int)((t_end - t_begin + ST - 1) / ST) : 0;
  const int lane = threadIdx.x & 63, g = lane >> 4, j = lane & 15, s4 = j >> 2;
  int F[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) F[f] = (8 * (g >> 1) + s4) * K4_ROWB + 64 * (f ^ s4) + 32 * (g & 1) + 8 * (j & 3);
  uint32_t voff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
    voff[h] = (uint32_t)((4 * (R::W + 4 * h) + (lane >> 4)) * ldx * 2 + 16 * ((lane & 15) ^ (4 * (lane >> 4))));
  auto stage_nrec = [&](int st) -> int {
    return st < nstages ? (int)min((t_end - t_begin - (int64_t)st * ST) * ldx * 2, (int64_t)0x7FFFFFF0) : 0;
  };
  auto stage_src = [&](int st) -> const uint16_t* {
    return X + (st < nstages ? t_begin + (int64_t)st * ST : t_begin) * ldx;
  };

  f32x16 accF[4][4], accH[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
#pragma unroll
      for (int c = 0; c < 4; ++c) accF[i][c][r] = 0.0f;
      accH[i][0][r] = 0.0f;
      accH[i][1][r] = 0.0f;
    }

  // Prologue: fill every slot (zero-length loads past the end), then read
  // stage 0's first fragments.
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int m = 0; m < NL; ++m) k4_loads<R::W>(lds + s * K4_STAGE, stage_src(s), stage_nrec(s), ch, voff, m);
  K4Frags<R> f0;
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
  asm volatile("s_barrier" ::: "memory");
#pragma unroll
  for (int m = 0; m < R::NF; ++m) k4_read<R>(lds, F, m, 0, f0);
  k4_mfma_fence(accH);
  for (int s = 0; s + 1 < nstages; ++s)
    k4_step<R, true>(lds + (s % NS) * K4_STAGE, lds + ((s + 1) % NS) * K4_STAGE, stage_src(s + NS),
                     stage_nrec(s + NS), ch, voff, F, f0, accF, accH);
  if (nstages > 0) {
    const int s = nstages - 1;
    k4_step<R, false>(lds + (s % NS) * K4_STAGE, lds, stage_src(s), 0, ch, voff, F, f0, accF, accH);
  }
  __builtin_amdgcn_s_waitcnt(0);   // the zero-length loads past the end write LDS too
  k4_mfma_fence(accH);

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) k4_store(accF[i][c], R::FB, 32 * i, 32 * c, ch[R::X], ch[R::Y], k, H, P, mirror);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < 2; ++c)
      k4_store(accH[i][c], R::HB, 32 * i, R::HC0 + 32 * c, ch[R::HR], ch[R::HC], k, H, P, mirror);
}

// Tile t over tokens [t_begin, t_end), into H or into its partial sums P
// (kK4SlotFloats): t < K4_TILES a four-group tile of the table, otherwise
// diagonal tile t - K4_TILES (segments 2d and 2d + 1, groups 4d .. 4d + 3).
__device__ __forceinline__ void k4_job(char* lds, const uint16_t* __restrict__ X, int64_t k, int64_t ldx, int t,
                                       int64_t t_begin, int64_t t_end, float* __restrict__ H, float* __restrict__ P,
                                       bool mirror = true) {
  int64_t ch[4];
  const int wave = threadIdx.x >> 6;
  if (t < K4_TILES) {
#pragma unroll
    for (int q = 0; q < 4; ++q) ch[q] = (int64_t)kK4.g[t][q] * K4G;
    switch (wave) {
      case 0: k4_wave<K4W0>(lds, X, k, ldx, ch, t_begin, t_end, H, P, mirror); break;
      case 1: k4_wave<K4W1>(lds, X, k, ldx, ch, t_begin, t_end, H, P, mirror); break;
      case 2: k4_wave<K4W2>(lds, X, k, ldx, ch, t_begin, t_end, H, P, mirror); break;
      default: k4_wave<K4W3>(lds, X, k, ldx, ch, t_begin, t_end, H, P, mirror); break;
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) ch[q] = (int64_t)(4 * (t - K4_TILES) + q) * K4G;
    switch (wave) {
      case 0: k4_wave<DGW0>(lds, X, k, ldx, ch, t_begin, t_end, H, P, mirror); break;
      case 1: k4_wave<DGW1>(lds, X, k, ldx, ch, t_begin, t_end, H, P, mirror); break;
      case 2: k4_wave<DGW2>(lds, X, k, ldx, ch, t_begin, t_end, H, P, mirror); break;
      default: k4_wave<DGW3>(lds, X, k, ldx, ch, t_begin, t_end, H, P, mirror); break;
    }
  }
}

// Order of the first launch's items within one token range.  256-blocks are
// grouped into super-blocks of SB; for each super-block A in turn come the
// quads inside A (row-major), then A's strips in pairs (2p, 2p+1), then the
// quads of A against each later super-block B (row-major over A x B).  Runs
// of consecutive items therefore touch few distinct 256-channel segments:
// for a 4096-channel layer, each run of 32 items reads 8 or 12 of the 16.
// Returns kind 0 (quad a < b), 1 (strip pair a, b; b = -1 if a is alone) or
// -1 past the end.
constexpr int SB = 8;
__host__ __device__ inline void item_coords(int r, int nb2, int& kind, int& a, int& b) {
  const int nsb = (nb2 + SB - 1) / SB;
  for (int A = 0; A < nsb; ++A) {
    const int a0 = A * SB, na = min(SB, nb2 - a0);
    const int nq = na * (na - 1) / 2, np = (na + 1) / 2;
    if (r < nq) {
      int aa = 0;
      while (r >= na - 1 - aa) { r -= na - 1 - aa; ++aa; }
      kind = 0; a = a0 + aa; b = a0 + aa + 1 + r;
      return;
    }
    r -= nq;
    if (r < np) {
      kind = 1; a = a0 + 2 * r; b = a + 1 < a0 + na ? a + 1 : -1;
      return;
    }
    r -= np;
    for (int B = A + 1; B < nsb; ++B) {
      const int b0 = B * SB, nbb = min(SB, nb2 - b0);
      if (r < na * nbb) {
        kind = 0; a = a0 + r / nbb; b = b0 + r % nbb;
        return;
      }
      r -= na * nbb;
    }
  }
  kind = -1; a = b = 0;
}

__host__ __device__ inline int items_per_range(int nb2) {
  int nsp = 0;
  for (int a0 = 0; a0 < nb2; a0 += SB) nsp += (min(SB, nb2 - a0) + 1) / 2;
  return nb2 * (nb2 - 1) / 2 + nsp;
}
__host__ __device__ inline int pairs_per_range(int nb2) { return items_per_range(nb2) - nb2 * (nb2 - 1) / 2; }

// Strip-pair tails.  With token splits every first-launch item covers one
// token range, but a strip pair takes longer than a quad (half a quad's
// products per LDS read and per barrier) and would finish last.  So it covers
// only the first `head` tokens of its range there, and the rest of the range
// is cut into tsplit pieces that run in the second launch beside the singles
// (npairs == 0: no tails).
struct TailArgs {
  int npairs;        // strip-pair items per range
  int tsplit;        // pieces per (range, pair)
  int64_t head;      // tokens of a range covered by the first launch
  int64_t ttokens;   // tokens per piece
  int64_t base;      // first partial slot of the pieces, ordered by (range, pair, piece)
};
// Item index (within a range) of the p-th strip pair, and the pair number of
// item r (the number of pairs before it), from the order of item_coords: per
// super-block, its quads, its pairs, then its quads against later ones.
__host__ __device__ inline int pair_item(int p, int nb2) {
  int base = 0;
  for (int a0 = 0; a0 < nb2; a0 += SB) {
    const int na = min(SB, nb2 - a0), nq = na * (na - 1) / 2, np = (na + 1) / 2;
    if (p < np) return base + nq + p;
    p -= np;
    base += nq + np + na * (nb2 - a0 - na);
  }
  return 0;
}
__host__ __device__ inline int pair_of_item(int r, int nb2) {
  int q = 0, base = 0;
  for (int a0 = 0; a0 < nb2; a0 += SB) {
    const int na = min(SB, nb2 - a0), nq = na * (na - 1) / 2, np = (na + 1) / 2;
    const int len = nq + np + na * (nb2 - a0 - na);
    if (r < base + len) {
      const int x = r - base - nq;
      return q + (x < 0 ? 0 : min(x, np));
    }
    q += np;
    base += len;
  }
  return q;
}

// Workgroups are dealt to the XCDs round-robin by id (id % 8).  Give each
// XCD a contiguous run of logical items, so the items sharing an XCD's L2
// share a token range and channel segments.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_logical(int id, int G) {
  const int per = G / kXcds, rem = G % kXcds, x = id % kXcds, i = id / kXcds;
  return (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + i;
}

// First-launch parameters of the quads: qsplit * per_range items; logical
// item L covers token range L / per_range and item L % per_range of the order
// above (a strip pair only the head of the range when there are tail
// pieces), and with qsplit > 1 writes its partial sums to slot L (a strip
// pair's two 128x256 strips fill the two halves of the slot).
struct MainArgs {
  int per_range, qsplit;
  int64_t qtokens;
};

__global__ __launch_bounds__(256) void syrk_main_kernel(const uint16_t* __restrict__ X, int64_t n, int64_t k,
                                                        int64_t ldx, float* __restrict__ H,
                                                        float* __restrict__ partial, MainArgs m, TailArgs tail) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int nb2 = (int)((k + QUAD - 1) / QUAD);
  const int L = xcd_logical(blockIdx.x, gridDim.x);
  int kind, a, b;
  item_coords(L % m.per_range, nb2, kind, a, b);
  const int64_t t0 = (int64_t)(L / m.per_range) * m.qtokens, t1 = min(n, t0 + m.qtokens);
  float* P = m.qsplit > 1 ? partial + (size_t)L * kSlotFloats : nullptr;
  if (kind == 0) {
    tile_job<QUAD, QUAD, false>(lds, X, k, ldx, (int64_t)a * QUAD, (int64_t)b * QUAD, t0, t1, H, P);
  } else if (kind == 1) {
    const int64_t te = tail.npairs > 0 ? min(t1, t0 + tail.head) : t1;   // the rest is tail work
    tile_job<HALF, QUAD, true>(lds, X, k, ldx, (int64_t)a * QUAD, (int64_t)a * QUAD, t0, te, H, P);
    if (b >= 0) {
      __syncthreads();   // the LDS ring is reused
      tile_job<HALF, QUAD, true>(lds, X, k, ldx, (int64_t)b * QUAD, (int64_t)b * QUAD, t0, te, H,
                                 P ? P + HALF * QUAD : nullptr);
    }
  }
}

// Four-group and diagonal tiles (16 segments).  First launch: K4_TILES * q4
// four-group tiles (tile L % K4_TILES over token range L / K4_TILES of
// k4tokens), then K4_DTILES * qd diagonal tiles (tile d of range sp is item
// sp * K4_DTILES + d over the first `head` tokens of its range of dtokens,
// all of it without tail pieces).  Second launch: the diagonal tiles' tail
// pieces, ts per (range, tile) of ttokens each, item u = (sp * K4_DTILES + d)
// * ts + piece.  A diagonal tile costs what a four-group tile does, so with
// head = k4tokens both kinds of first-launch item take the same time.
// Partial sums (kK4SlotFloats each) at slot L for the four-group tiles,
// dbase + that item for the diagonal heads, tbase + u for the tail pieces;
// with direct = 1 (one token range for every tile, no tails) each tile adds
// into H itself.
constexpr int K4_DTILES = K4_SEGS / 2;
constexpr int K4_TSPLIT = 16;
struct K4Args {
  int q4, qd, ts, direct;
  int64_t k4tokens, dtokens, head, ttokens, dbase, tbase;
};

constexpr int K4_ALL = K4_TILES + K4_DTILES;   // tiles of one k = 4096 Hessian
static_assert(sizeof(K4Grouped::nx) == kXcds, "one expert list per XCD");

__global__ __launch_bounds__(256) void syrk_k4_kernel(const uint16_t* __restrict__ X, int64_t n, int64_t k,
                                                      int64_t ldx, float* __restrict__ H,
                                                      float* __restrict__ partial, K4Args a, int tails) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int L = xcd_logical(blockIdx.x, gridDim.x);
  const int nk = K4_TILES * a.q4;
  int t;
  int64_t t0, t1;
  size_t slot;
  if (tails) {
    const int sp = L / (K4_DTILES * a.ts), piece = L % a.ts;
    const int64_t r0 = (int64_t)sp * a.dtokens, r1 = min(n, r0 + a.dtokens);
    t = K4_TILES + (L / a.ts) % K4_DTILES;
    t0 = min(r1, r0 + a.head + (int64_t)piece * a.ttokens);
    t1 = min(r1, t0 + a.ttokens);
    slot = (size_t)a.tbase + L;
  } else if (L < nk) {
    t = L % K4_TILES;
    t0 = (int64_t)(L / K4_TILES) * a.k4tokens;
    t1 = min(n, t0 + a.k4tokens);
    slot = L;
  } else {
    const int e = L - nk;
    t = K4_TILES + e % K4_DTILES;
    t0 = (int64_t)(e / K4_DTILES) * a.dtokens;
    t1 = min(n, t0 + a.dtokens);
    if (a.ts > 0) t1 = min(t1, t0 + a.head);
    slot = (size_t)a.dbase + e;
  }
  k4_job(lds, X, k, ldx, t, t0, t1, H, a.direct ? nullptr : partial + slot * kK4SlotFloats);
}

// Grouped Hessians of small experts (one H per expert, k = 4096 layout): one
// launch runs every four-group and diagonal tile of every expert of the
// group, each over its expert's whole token range (rows gathered one expert
// after another), adding straight into that expert's H.  Workgroup b runs on
// XCD b % 8 (ids are dealt round-robin), item (b / 8) of that XCD's list:
// expert xe[x][(b / 8) / K4_ALL], tile (b / 8) % K4_ALL.  The host gives each
// XCD whole experts, largest first and balanced by tokens, so an expert's rows
// are read into one XCD's L2 and the XCDs finish together; workgroups past
// an XCD's list exit.  No tile of an expert shares an H entry with another,
// so the direct stores do not race.
__global__ __launch_bounds__(256) void syrk_k4_grouped_kernel(const uint16_t* __restrict__ X, int64_t k,
                                                              float* __restrict__ H, K4Grouped g) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int x = (int)(blockIdx.x % kXcds), i = (int)(blockIdx.x / kXcds);
  const int j = i / K4_ALL, t = i % K4_ALL;
  if (j >= g.nx[x]) return;
  const int e = g.xe[x][j];
  k4_job(lds, X + (int64_t)g.beg[e] * k, k, k, t, 0, g.cnt[e], H + (int64_t)g.hexp[e] * k * k, nullptr, false);
}

// The lower triangle of each grouped expert's H from its upper triangle (the
// grouped tiles add into the upper triangle only: their column-strided mirror
// stores would touch a cache line per element).  One 64 x 64 tile per
// workgroup: tile (bi, bj), bi >= bj, of expert blockIdx.y is the transpose of
// upper tile (bj, bi), read by rows into LDS and written by rows; a diagonal
// tile writes only below its diagonal.  k % 64 == 0.
__global__ __launch_bounds__(256) void k4_mirror_kernel(float* __restrict__ H, int64_t k, K4Grouped g) {
  __shared__ float T[64][65];
  const int64_t t = blockIdx.x;
  int64_t bi = (int64_t)((sqrt(8.0 * (double)t + 1.0) - 1.0) / 2.0);
  while (bi * (bi + 1) / 2 > t) --bi;
  while ((bi + 1) * (bi + 2) / 2 <= t) ++bi;
  const int64_t bj = t - bi * (bi + 1) / 2;
  float* He = H + (int64_t)g.hexp[blockIdx.y] * k * k;
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = q * 256 + tid, r = e >> 4, c4 = (e & 15) * 4;
    const f32x4 v = *(const f32x4*)(He + (bj * 64 + r) * k + bi * 64 + c4);
#pragma unroll
    for (int u = 0; u < 4; ++u) T[r][c4 + u] = v[u];
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = q * 256 + tid, r = e >> 4, c4 = (e & 15) * 4;
    float* dst = He + (bi * 64 + r) * k + bj * 64 + c4;
    if (bi != bj) {
      *(f32x4*)dst = f32x4{T[c4][r], T[c4 + 1][r], T[c4 + 2][r], T[c4 + 3][r]};
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (c4 + u < r) dst[u] = T[c4 + u][r];
    }
  }
}

// Launch 2: singles (bottom-right diagonal 128-block of 256-block a), split
// over tokens when they are too few to fill the device (workgroups
// 0 .. nsingle * nsplit - 1), then the strip-pair tail pieces.
__global__ __launch_bounds__(256) void syrk_single_kernel(const uint16_t* __restrict__ X, int64_t n, int64_t k,
                                                          int64_t ldx, float* __restrict__ H,
                                                          float* __restrict__ partial, int nsingle, int nsplit,
                                                          int64_t stokens, size_t slot_base, int64_t qtokens,
                                                          TailArgs tail) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int id = blockIdx.x, nsi = nsingle * nsplit;
  if (id < nsi) {
    const int a = id / nsplit, sp = id % nsplit;
    const int64_t c0 = (int64_t)a * QUAD + HALF;
    const int64_t t0 = (int64_t)sp * stokens;
    float* P = nsplit > 1 ? partial + (slot_base + (size_t)a * nsplit + sp) * kSlotFloats : nullptr;
    tile_job<HALF, HALF, true>(lds, X, k, ldx, c0, c0, t0, min(n, t0 + stokens), H, P);
    return;
  }
  // Tail piece u: token range sp, strip pair p, piece t (an empty token range
  // stores zeros).
  const int u = id - nsi;
  const int sp = u / (tail.npairs * tail.tsplit), p = (u / tail.tsplit) % tail.npairs, t = u % tail.tsplit;
  const int nb2 = (int)((k + QUAD - 1) / QUAD);
  int kind, a, b;
  item_coords(pair_item(p, nb2), nb2, kind, a, b);
  const int64_t r1 = min(n, (int64_t)sp * qtokens + qtokens);
  const int64_t ts = min(r1, (int64_t)sp * qtokens + tail.head + (int64_t)t * tail.ttokens);
  const int64_t te = min(r1, ts + tail.ttokens);
  float* P = partial + ((size_t)tail.base + u) * kSlotFloats;
  tile_job<HALF, QUAD, true>(lds, X, k, ldx, (int64_t)a * QUAD, (int64_t)a * QUAD, ts, te, H, P);
  if (b >= 0) {
    __syncthreads();   // the LDS ring is reused
    tile_job<HALF, QUAD, true>(lds, X, k, ldx, (int64_t)b * QUAD, (int64_t)b * QUAD, ts, te, H, P + HALF * QUAD);
  }
}

// Sum the token splits of one 64x64 piece of a tile in split order, add the
// sum into H's upper triangle and write the mirror.  The piece is at rows r0,
// columns c0 of H; its split sp is at P + sp * sstride with row stride ldp;
// then come n2 more partial sums (strip-pair tail pieces), the j-th at
// P2 + (j / inner2) * ostride2 + (j % inner2) * istride2.  H and P move in
// 16-byte vectors; the mirror goes through an LDS transpose so that it is
// written by rows too.  k % 16 == 0, so a vector is wholly inside or outside H.
constexpr int PIECE = 64;
__device__ __forceinline__ void reduce_piece(int64_t k, float* __restrict__ H, const float* __restrict__ P,
                                             size_t sstride, int nsplit, int ldp, int64_t r0, int64_t c0,
                                             const float* __restrict__ P2 = nullptr, int n2 = 0, int inner2 = 1,
                                             size_t ostride2 = 0, size_t istride2 = 0) {
  if (r0 >= k || c0 >= k || r0 >= c0 + PIECE) return;   // outside H, or wholly below the diagonal
  __shared__ float tr[PIECE][PIECE + 1];
  const int tid = threadIdx.x;
  const bool offdiag = r0 + PIECE <= c0;
  f32x4 s[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) s[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  int sp = 0;
  for (; sp + 2 <= nsplit; sp += 2) {
    f32x4 v[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = q * 256 + tid, row = e >> 4, c4 = (e & 15) * 4;
        v[u][q] = *(const f32x4*)(P + (size_t)(sp + u) * sstride + (size_t)row * ldp + c4);
      }
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) s[q] += v[u][q];
  }
  if (sp < nsplit) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = q * 256 + tid, row = e >> 4, c4 = (e & 15) * 4;
      s[q] += *(const f32x4*)(P + (size_t)sp * sstride + (size_t)row * ldp + c4);
    }
  }
  for (int j = 0; j < n2; ++j) {
    const float* Q = P2 + (size_t)(j / inner2) * ostride2 + (size_t)(j % inner2) * istride2;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = q * 256 + tid, row = e >> 4, c4 = (e & 15) * 4;
      s[q] += *(const f32x4*)(Q + (size_t)row * ldp + c4);
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = q * 256 + tid, row = e >> 4, c4 = (e & 15) * 4;
    const int64_t gi = r0 + row, gj = c0 + c4;
    const bool in = gi < k && gj < k;
    const f32x4 h = *(const f32x4*)(H + min(gi, k - 1) * k + min(gj, k - 4));
    const f32x4 v = h + s[q];
    if (in) {
      if (offdiag) {
        *(f32x4*)(H + gi * k + gj) = v;
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (gi <= gj + u) H[gi * k + gj + u] = v[u];
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) tr[row][c4 + u] = v[u];
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    // mirror row c0 + a, columns r0 + b4 .. r0 + b4 + 3
    const int e = q * 256 + tid, a = e >> 4, b4 = (e & 15) * 4;
    const int64_t mi = c0 + a, mj = r0 + b4;
    if (mi >= k || mj >= k) continue;
    f32x4 v;
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = tr[b4 + u][a];
    if (offdiag) {
      *(f32x4*)(H + mi * k + mj) = v;
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (mj + u < mi) H[mi * k + mj + u] = v[u];
    }
  }
}

// kind 0: blockIdx.x is item r of the first launch's order, whose split sp
// sits in slot sp * per_range + r; blockIdx.y (0..15) is a 64x64 piece (a
// quad's 4x4, or a strip pair's two 2x4).  kind 1: blockIdx.x is single a,
// whose split sp sits in slot slot_base + a * nsplit + sp; blockIdx.y (0..3)
// is a piece of its 2x2.
__global__ __launch_bounds__(256) void syrk_reduce_kernel(int64_t k, float* __restrict__ H,
                                                          const float* __restrict__ partial, int kind, int nsplit,
                                                          int per_range, size_t slot_base, TailArgs tail) {
  const int nb2 = (int)((k + QUAD - 1) / QUAD);
  const int y = blockIdx.y;
  if (kind == 0) {
    int ik, a, b;
    item_coords(blockIdx.x, nb2, ik, a, b);
    const float* P = partial + (size_t)blockIdx.x * kSlotFloats;
    const size_t sstride = (size_t)per_range * kSlotFloats;
    const int pr = (y & 7) / 4, pc = y % 4;
    if (ik == 0) {
      reduce_piece(k, H, P + (size_t)(y / 4) * PIECE * QUAD + pc * PIECE, sstride, nsplit, QUAD,
                   (int64_t)a * QUAD + (y / 4) * PIECE, (int64_t)b * QUAD + pc * PIECE);
    } else if (ik == 1) {
      const int d = y < 8 ? a : b;
      const size_t off = (y < 8 ? 0 : (size_t)HALF * QUAD) + (size_t)pr * PIECE * QUAD + pc * PIECE;
      const float* P2 = nullptr;
      int n2 = 0;
      if (tail.npairs > 0) {   // then the pair's tail pieces, by range and piece
        P2 = partial + ((size_t)tail.base + (size_t)pair_of_item(blockIdx.x, nb2) * tail.tsplit) * kSlotFloats + off;
        n2 = nsplit * tail.tsplit;
      }
      if (d >= 0)
        reduce_piece(k, H, P + off, sstride, nsplit, QUAD, (int64_t)d * QUAD + pr * PIECE,
                     (int64_t)d * QUAD + pc * PIECE, P2, n2, tail.tsplit,
                     (size_t)tail.npairs * tail.tsplit * kSlotFloats, kSlotFloats);
    }
  } else {
    const int64_t c0 = (int64_t)blockIdx.x * QUAD + HALF;
    const float* P = partial + (slot_base + (size_t)blockIdx.x * nsplit) * kSlotFloats;
    reduce_piece(k, H, P + (size_t)(y / 2) * PIECE * HALF + (y % 2) * PIECE, kSlotFloats, nsplit, HALF,
                 c0 + (y / 2) * PIECE, c0 + (y % 2) * PIECE);
  }
}

// Four-group and diagonal tiles.  kind 0: blockIdx.x is four-group tile t,
// whose range sp sits at slot sp * K4_TILES + t; kind 1: blockIdx.x is
// diagonal tile d, whose range sp sits at slot dbase + sp * K4_DTILES + d,
// followed by its tail pieces (slot tbase + (sp * K4_DTILES + d) * ts +
// piece), summed by range and piece.  blockIdx.y (0..23) is a 64x64 piece of
// the tile's six 128x128 blocks (2x2 each); pieces wholly below a diagonal
// block's diagonal are skipped.
__global__ __launch_bounds__(256) void syrk_reduce_k4_kernel(int64_t k, float* __restrict__ H,
                                                             const float* __restrict__ partial, int kind,
                                                             K4Args a) {
  const int t = blockIdx.x, y = blockIdx.y, b = y / 4, pr = (y % 4) / 2, pc = y % 2;
  const size_t off = (size_t)b * K4G * K4G + pr * PIECE * K4G + pc * PIECE;
  if (kind == 0) {
    const int ra = b < 3 ? 0 : (b < 5 ? 1 : 2), rb = b < 3 ? b + 1 : (b < 5 ? b - 1 : 3);
    reduce_piece(k, H, partial + (size_t)t * kK4SlotFloats + off, (size_t)K4_TILES * kK4SlotFloats, a.q4, K4G,
                 (int64_t)kK4.g[t][ra] * K4G + pr * PIECE, (int64_t)kK4.g[t][rb] * K4G + pc * PIECE);
    return;
  }
  const float* P2 = a.ts > 0 ? partial + ((size_t)a.tbase + (size_t)t * a.ts) * kK4SlotFloats + off : nullptr;
  reduce_piece(k, H, partial + ((size_t)a.dbase + t) * kK4SlotFloats + off, (size_t)K4_DTILES * kK4SlotFloats,
               a.qd, K4G, (int64_t)(4 * t + dg_row(b)) * K4G + pr * PIECE,
               (int64_t)(4 * t + dg_col(b)) * K4G + pc * PIECE, P2, a.qd * a.ts, a.ts > 0 ? a.ts : 1,
               (size_t)K4_DTILES * a.ts * kK4SlotFloats, kK4SlotFloats);
}

__global__ void symmetrize_kernel(float* H, int64_t k) {
  int64_t i = blockIdx.y, j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j < k && j < i) H[i * k + j] = H[j * k + i];
}

struct SyrkPlan {
  int nb2, k4, nsingle, ssplit;
  MainArgs m;        // quads and strip pairs (k4 = 0)
  K4Args a;          // four-group and diagonal tiles (k4 = 1)
  int64_t stokens;
  TailArgs tail;
  size_t slots;      // partial slots of kSlotFloats
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

// Four-group and diagonal tiles: as many token ranges of the four-group
// tiles as give each (tile, range) a CU; the diagonal tiles split over the
// CUs left (at least one range), their heads as long as a four-group item
// and the rest of each range in up to K4_TSPLIT tail pieces.  Each split
// writes a partial slot (384 KB) that the reduction reads again, so ranges
// and tail pieces keep at least K4_MIN_STAGES stages each.  The range counts
// grow with n up to their caps and never shrink.
constexpr int K4_MIN_STAGES = 16;
K4Args k4_plan(int64_t nstages, int cus) {
  K4Args a{};
  const int64_t most = nstages / K4_MIN_STAGES < 1 ? 1 : nstages / K4_MIN_STAGES;
  int64_t q4 = cus / K4_TILES;
  a.q4 = (int)(q4 > most ? most : (q4 < 1 ? 1 : q4));
  int64_t qd = (cus - (int64_t)K4_TILES * (cus / K4_TILES)) / K4_DTILES;
  a.qd = (int)(qd > most ? most : (qd < 1 ? 1 : qd));
  a.k4tokens = ((nstages + a.q4 - 1) / a.q4) * ST;
  a.dtokens = ((nstages + a.qd - 1) / a.qd) * ST;
  a.head = a.k4tokens < a.dtokens ? a.k4tokens : a.dtokens;
  a.ts = 0;
  a.ttokens = 0;
  if (a.head < a.dtokens) {
    const int64_t tail_stages = (a.dtokens - a.head) / ST;
    const int64_t ts = tail_stages / K4_MIN_STAGES;
    a.ts = (int)(ts > K4_TSPLIT ? K4_TSPLIT : (ts < 1 ? 1 : ts));
    const int64_t per = (a.dtokens - a.head + a.ts - 1) / a.ts;
    a.ttokens = (per + ST - 1) / ST * ST;
  }
  a.direct = a.q4 == 1 && a.qd == 1 && a.ts == 0;
  a.dbase = (int64_t)K4_TILES * a.q4;
  a.tbase = a.dbase + (int64_t)K4_DTILES * a.qd;
  return a;
}
// Partial slots (of kSlotFloats) the four-group plan uses: every tile range,
// diagonal head and tail piece (the tails at their cap, so that the count
// never shrinks as n grows).
size_t k4_slots(const K4Args& a) {
  if (a.direct) return 0;
  const size_t k4s = (size_t)a.tbase + (size_t)K4_DTILES * a.qd * K4_TSPLIT;
  return (k4s * kK4SlotFloats + kSlotFloats - 1) / kSlotFloats;
}

SyrkPlan plan(int64_t n, int64_t k, int cus) {
  SyrkPlan p{};
  p.nb2 = (int)((k + QUAD - 1) / QUAD);
  int64_t nstages = (n + ST - 1) / ST;
  if (nstages < 1) nstages = 1;
  p.k4 = p.nb2 == K4_SEGS;
  if (p.k4) {
    p.a = k4_plan(nstages, cus);
    p.slots = k4_slots(p.a);
    return p;
  }
  p.nsingle = 0;
  for (int a = 0; a < p.nb2; ++a)
    if ((int64_t)a * QUAD + HALF < k) ++p.nsingle;
  MainArgs& m = p.m;
  // Split the first launch's items over token ranges while they would not
  // give every CU an item.
  m.per_range = items_per_range(p.nb2);
  m.qsplit = 1;
  if (m.per_range < cus) {
    int64_t s = (cus + m.per_range - 1) / m.per_range;
    if (s > nstages) s = nstages;
    m.qsplit = (int)(s < 1 ? 1 : s);
  }
  m.qtokens = ((nstages + m.qsplit - 1) / m.qsplit) * ST;
  // Strip-pair tails (only with token splits, whose partial sums the tails
  // join): the pairs keep HEAD16/16 of each range, whole stages, when the
  // pieces leave at least half the device to the singles.
  p.tail = TailArgs{0, 1, 0, 0, 0};
  if (m.qsplit > 1) {
    const int npairs = pairs_per_range(p.nb2);
    const int64_t head = m.qtokens * HEAD16 / 16 / ST * ST;
    if (npairs > 0 && head > 0 && head < m.qtokens && (int64_t)npairs * m.qsplit * TSPLIT <= cus / 2) {
      const int64_t per = (m.qtokens - head + TSPLIT - 1) / TSPLIT;
      p.tail = TailArgs{npairs, TSPLIT, head, (per + ST - 1) / ST * ST, 0};
    }
  }
  const int tail_items = p.tail.npairs * m.qsplit * p.tail.tsplit;
  p.ssplit = 1;
  if (p.nsingle > 0 && p.nsingle < cus - tail_items) {
    int64_t s = (cus - tail_items) / p.nsingle;
    if (s > nstages) s = nstages;
    p.ssplit = (int)(s < 1 ? 1 : s);
  }
  p.stokens = ((nstages + p.ssplit - 1) / p.ssplit) * ST;
  // Slots: first-launch items, then the singles' splits, then the tail pieces.
  p.slots = (m.qsplit > 1 ? (size_t)m.per_range * m.qsplit : 0) + (p.ssplit > 1 ? (size_t)p.nsingle * p.ssplit : 0) +
            (size_t)tail_items;
  if (tail_items > 0) p.tail.base = (int64_t)(p.slots - tail_items);
  return p;
}

}  // namespace

// An upper bound of the plan's slots that does not decrease with n, since
// callers size one workspace for several token counts (groups, chunks): the
// singles' splits as if there were no tail pieces, plus every tail piece the
// token splits allow.
size_t syrk_bf16_workspace(int64_t n, int64_t k) {
  const int cus = num_cus();
  SyrkPlan p = plan(n, k, cus);
  if (p.k4) return p.slots * kSlotFloats * sizeof(float);
  size_t slots = 0;
  if (p.m.qsplit > 1) slots += ((size_t)p.m.per_range + (size_t)pairs_per_range(p.nb2) * TSPLIT) * p.m.qsplit;
  if (p.nsingle > 0 && p.nsingle < cus) {
    const int64_t nstages = n > ST ? (n + ST - 1) / ST : 1;
    const int64_t sp = cus / p.nsingle < nstages ? cus / p.nsingle : nstages;
    if (sp > 1) slots += (size_t)p.nsingle * sp;
  }
  return (slots > p.slots ? slots : p.slots) * kSlotFloats * sizeof(float);
}

hipError_t syrk_bf16(const uint16_t* X, int64_t n, int64_t k, int64_t ldx, float* H, void* ws, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  SyrkPlan p = plan(n, k, num_cus());
  float* partial = (float*)ws;
  constexpr int main_stage = Tile<QUAD, QUAD>::STAGE_BYTES > Tile<HALF, QUAD>::STAGE_BYTES
                                 ? Tile<QUAD, QUAD>::STAGE_BYTES
                                 : Tile<HALF, QUAD>::STAGE_BYTES;
  static_assert(K4_STAGE <= main_stage, "the first launch's LDS ring holds a four-group stage");
  const size_t lds_main = (size_t)NS * main_stage;
  const size_t lds_single = (size_t)NS * (Tile<HALF, QUAD>::STAGE_BYTES > Tile<HALF, HALF>::STAGE_BYTES
                                              ? Tile<HALF, QUAD>::STAGE_BYTES
                                              : Tile<HALF, HALF>::STAGE_BYTES);
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute((const void*)syrk_main_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds_main);
    (void)hipFuncSetAttribute((const void*)syrk_k4_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds_main);
    (void)hipFuncSetAttribute((const void*)syrk_single_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds_single);
    attr = true;
  }
  if (p.k4) {
    // Tiles, tail pieces, then the reductions (a diagonal tile sums its tail
    // pieces too).
    const K4Args& a = p.a;
    hipLaunchKernelGGL(syrk_k4_kernel, dim3(K4_TILES * a.q4 + K4_DTILES * a.qd), dim3(256), lds_main, s, X, n, k,
                       ldx, H, partial, a, 0);
    if (a.ts > 0)
      hipLaunchKernelGGL(syrk_k4_kernel, dim3(K4_DTILES * a.qd * a.ts), dim3(256), lds_main, s, X, n, k, ldx, H,
                         partial, a, 1);
    if (!a.direct) {
      hipLaunchKernelGGL(syrk_reduce_k4_kernel, dim3(K4_TILES, 24), dim3(256), 0, s, k, H, partial, 0, a);
      hipLaunchKernelGGL(syrk_reduce_k4_kernel, dim3(K4_DTILES, 24), dim3(256), 0, s, k, H, partial, 1, a);
    }
    return hipGetLastError();
  }
  const MainArgs& m = p.m;
  // Order: first launch, second launch (singles and tail pieces), then the
  // reductions, since a strip pair's tiles sum the tail pieces too.
  hipLaunchKernelGGL(syrk_main_kernel, dim3(m.per_range * m.qsplit), dim3(256), lds_main, s, X, n, k, ldx, H,
                     partial, m, p.tail);
  const size_t single_base = m.qsplit > 1 ? (size_t)m.per_range * m.qsplit : 0;
  const int second = p.nsingle * p.ssplit + p.tail.npairs * m.qsplit * p.tail.tsplit;
  if (second > 0)
    hipLaunchKernelGGL(syrk_single_kernel, dim3(second), dim3(256), lds_single, s, X, n, k, ldx, H, partial,
                       p.nsingle, p.ssplit, p.stokens, single_base, m.qtokens, p.tail);
  if (m.qsplit > 1)
    hipLaunchKernelGGL(syrk_reduce_kernel, dim3(m.per_range, 16), dim3(256), 0, s, k, H, partial, 0, m.qsplit,
                       m.per_range, (size_t)0, p.tail);
  if (p.nsingle > 0 && p.ssplit > 1)
    hipLaunchKernelGGL(syrk_reduce_kernel, dim3(p.nsingle, 4), dim3(256), 0, s, k, H, partial, 1, p.ssplit, 0,
                       single_base, p.tail);
  return hipGetLastError();
}

bool syrk_k4_applies(int64_t k) { return (k + QUAD - 1) / QUAD == K4_SEGS; }
bool syrk_k4_grouped_applies(int64_t k) { return syrk_k4_applies(k) && k % 64 == 0; }

// Experts on XCDs: largest first, each to the XCD with the fewest tokens so far
// (among those with room), so every XCD's list is in decreasing size.
hipError_t syrk_bf16_grouped(const uint16_t* rows, int64_t k, K4Grouped& g, int nexp, float* H, hipStream_t s) {
  if (nexp <= 0) return hipSuccess;
  if (nexp > K4G_EXP || !syrk_k4_grouped_applies(k)) return hipErrorInvalidValue;
  int order[K4G_EXP];
  for (int j = 0; j < nexp; ++j) order[j] = j;
  std::sort(order, order + nexp, [&](int a, int b) { return g.cnt[a] != g.cnt[b] ? g.cnt[a] > g.cnt[b] : a < b; });
  int64_t load[kXcds] = {};
  for (int x = 0; x < kXcds; ++x) g.nx[x] = 0;
  for (int q = 0; q < nexp; ++q) {
    int best = -1;
    for (int x = 0; x < kXcds; ++x)
      if (g.nx[x] < K4G_PER_XCD && (best < 0 || load[x] < load[best])) best = x;
    g.xe[best][g.nx[best]++] = (uint8_t)order[q];
    load[best] += g.cnt[order[q]];
  }
  int most = 0;
  for (int x = 0; x < kXcds; ++x) most = std::max<int>(most, g.nx[x]);
  static bool attr = false;
  const size_t lds = (size_t)NS * K4_STAGE;
  if (!attr) {
    (void)hipFuncSetAttribute((const void*)syrk_k4_grouped_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds);
    attr = true;
  }
  hipLaunchKernelGGL(syrk_k4_grouped_kernel, dim3((unsigned)(kXcds * most * K4_ALL)), dim3(256), lds, s, rows, k, H,
                     g);
  const int64_t nt = k / 64;
  hipLaunchKernelGGL(k4_mirror_kernel, dim3((unsigned)(nt * (nt + 1) / 2), (unsigned)nexp), dim3(256), 0, s, H, k, g);
  return hipGetLastError();
}

// Row gather for grouped Hessians: out[t][0:k] = X[clamp(idx[t])][0:k],
// in 16-byte pieces (rows of k * esize bytes, a multiple of 16).
__global__ __launch_bounds__(256) void gather_rows_kernel(const char* __restrict__ X, int64_t row_bytes_src,
                                                          const int32_t* __restrict__ idx, int64_t nsrc, int64_t n,
                                                          int64_t pieces, char* __restrict__ out) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n * pieces) return;
  const int64_t t = e / pieces, c = e % pieces;
  int64_t r = idx[t];
  r = r < 0 ? 0 : (r >= nsrc ? nsrc - 1 : r);
  *(u32x4*)(out + (t * pieces + c) * 16) = *(const u32x4*)(X + r * row_bytes_src + c * 16);
}

hipError_t gather_rows(const void* X, int esize, int64_t ldx, const int32_t* idx, int64_t nsrc, int64_t n,
                       int64_t k, void* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t pieces = k * esize / 16;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)((n * pieces + 255) / 256)), dim3(256), 0, s,
                     (const char*)X, ldx * esize, idx, nsrc, n, pieces, (char*)out);
  return hipGetLastError();
}

hipError_t symmetrize_from_upper(float* H, int64_t k, hipStream_t s) {
  hipLaunchKernelGGL(symmetrize_kernel, dim3((unsigned)((k + 255) / 256), (unsigned)k), dim3(256), 0, s, H, k);
  return hipGetLastError();
}

}  // namespace nvq
