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

// Launch 1: G = qsplit * per_range items; logical item L covers token range
// L / per_range and item L % per_range of the order above (a strip pair only
// the head of the range when there are tail pieces).  With qsplit > 1 the
// item's partial sums go to slot L (a strip pair's two 128x256 strips fill
// the two halves of the slot).
__global__ __launch_bounds__(256) void syrk_main_kernel(const uint16_t* __restrict__ X, int64_t n, int64_t k,
                                                        int64_t ldx, float* __restrict__ H,
                                                        float* __restrict__ partial, int per_range, int qsplit,
                                                        int64_t qtokens, TailArgs tail) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int nb2 = (int)((k + QUAD - 1) / QUAD);
  const int L = xcd_logical(blockIdx.x, gridDim.x);
  const int sp = L / per_range;
  int kind, a, b;
  item_coords(L % per_range, nb2, kind, a, b);
  const int64_t t0 = (int64_t)sp * qtokens, t1 = min(n, t0 + qtokens);
  float* P = qsplit > 1 ? partial + (size_t)L * kSlotFloats : nullptr;
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

__global__ void symmetrize_kernel(float* H, int64_t k) {
  int64_t i = blockIdx.y, j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j < k && j < i) H[i * k + j] = H[j * k + i];
}

struct SyrkPlan {
  int nb2, per_range, qsplit, nsingle, ssplit;
  int64_t qtokens, stokens;
  TailArgs tail;
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
  p.per_range = items_per_range(p.nb2);
  p.nsingle = 0;
  for (int a = 0; a < p.nb2; ++a)
    if ((int64_t)a * QUAD + HALF < k) ++p.nsingle;
  int64_t nstages = (n + ST - 1) / ST;
  if (nstages < 1) nstages = 1;
  // Split the first launch's items over token ranges while they would not
  // give every CU an item.
  p.qsplit = 1;
  if (p.per_range < cus) {
    int64_t s = (cus + p.per_range - 1) / p.per_range;
    if (s > nstages) s = nstages;
    p.qsplit = (int)(s < 1 ? 1 : s);
  }
  p.qtokens = ((nstages + p.qsplit - 1) / p.qsplit) * ST;
  // Strip-pair tails (only with token splits, whose partial sums the tails
  // join): the pairs keep HEAD16/16 of each range, whole stages, when the
  // pieces leave at least half the device to the singles.
  p.tail = TailArgs{0, 1, 0, 0, 0};
  if (p.qsplit > 1) {
    const int npairs = pairs_per_range(p.nb2);
    const int64_t head = p.qtokens * HEAD16 / 16 / ST * ST;
    if (npairs > 0 && head > 0 && head < p.qtokens && (int64_t)npairs * p.qsplit * TSPLIT <= cus / 2) {
      const int64_t per = (p.qtokens - head + TSPLIT - 1) / TSPLIT;
      p.tail = TailArgs{npairs, TSPLIT, head, (per + ST - 1) / ST * ST, (int64_t)p.per_range * p.qsplit};
    }
  }
  const int tail_items = p.tail.npairs * p.qsplit * p.tail.tsplit;
  p.ssplit = 1;
  if (p.nsingle > 0 && p.nsingle < cus - tail_items) {
    int64_t s = (cus - tail_items) / p.nsingle;
    if (s > nstages) s = nstages;
    p.ssplit = (int)(s < 1 ? 1 : s);
  }
  p.stokens = ((nstages + p.ssplit - 1) / p.ssplit) * ST;
  // Slots: first-launch items, then the singles' splits, then the tail pieces.
  p.slots = (p.qsplit > 1 ? (size_t)p.per_range * p.qsplit : 0) + (p.ssplit > 1 ? (size_t)p.nsingle * p.ssplit : 0) +
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
  size_t slots = 0;
  if (p.qsplit > 1) slots += ((size_t)p.per_range + (size_t)pairs_per_range(p.nb2) * TSPLIT) * p.qsplit;
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
  const size_t lds_main = (size_t)NS * main_stage;
  const size_t lds_single = (size_t)NS * (Tile<HALF, QUAD>::STAGE_BYTES > Tile<HALF, HALF>::STAGE_BYTES
                                              ? Tile<HALF, QUAD>::STAGE_BYTES
                                              : Tile<HALF, HALF>::STAGE_BYTES);
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute((const void*)syrk_main_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds_main);
    (void)hipFuncSetAttribute((const void*)syrk_single_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds_single);
    attr = true;
  }
  // Order: first launch, second launch (singles and tail pieces), then the
  // reductions, since a strip pair's tiles sum the tail pieces too.
  const int items = p.per_range * p.qsplit;
  hipLaunchKernelGGL(syrk_main_kernel, dim3(items), dim3(256), lds_main, s, X, n, k, ldx, H, partial, p.per_range,
                     p.qsplit, p.qtokens, p.tail);
  const size_t single_base = p.qsplit > 1 ? (size_t)p.per_range * p.qsplit : 0;
  const int second = p.nsingle * p.ssplit + p.tail.npairs * p.qsplit * p.tail.tsplit;
  if (second > 0)
    hipLaunchKernelGGL(syrk_single_kernel, dim3(second), dim3(256), lds_single, s, X, n, k, ldx, H, partial,
                       p.nsingle, p.ssplit, p.stokens, single_base, p.qtokens, p.tail);
  if (p.qsplit > 1)
    hipLaunchKernelGGL(syrk_reduce_kernel, dim3(p.per_range, 16), dim3(256), 0, s, k, H, partial, 0, p.qsplit,
                       p.per_range, (size_t)0, p.tail);
  if (p.nsingle > 0 && p.ssplit > 1)
    hipLaunchKernelGGL(syrk_reduce_kernel, dim3(p.nsingle, 4), dim3(256), 0, s, k, H, partial, 1, p.ssplit, 0,
                       single_base, p.tail);
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
