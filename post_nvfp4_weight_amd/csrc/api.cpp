// C ABI of the NVFP4 GPTQ / Schur Replay quantizer: argument validation,
// workspace carving and kernel sequencing.  See include/nvq.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "../../include/nvq.h"
#include "common.h"
#include "kernels.h"

using namespace nvq;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return NVQ_OK;
  return fail(NVQ_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

struct QuantWs {
  size_t wp, w0, eslab, invd, mb, part, total;
};

// chol: the Cholesky-factor form also keeps the input weights in the working
// precision (w0) and the diagonal blocks' M - I (mb, k * 16 floats).
QuantWs quant_ws(int64_t m, int64_t k, bool f64, bool chol = false) {
  QuantWs w;
  const size_t es = f64 ? sizeof(double) : sizeof(float);
  size_t off = 0;
  w.wp = off;   off += align_up((size_t)m * k * es);
  w.w0 = off;   if (chol) off += align_up((size_t)m * k * es);
  w.eslab = off; off += align_up((size_t)m * kSuperBatch * es);
  w.invd = off;  off += align_up((size_t)k * sizeof(float));
  w.mb = off;    if (chol) off += align_up((size_t)k * kBlock * sizeof(float));
  w.part = off;  off += align_up((size_t)m * ((k + kGemmTile - 1) / kGemmTile) * sizeof(float));
  w.total = off;
  return w;
}

bool dtype_ok(int d) { return d == NVQ_DTYPE_F32 || d == NVQ_DTYPE_BF16; }

hipError_t hessian_run(const void* X, int x_dtype, int64_t n, int64_t k, int64_t ldx, float* H, void* ws,
                       hipStream_t s) {
  if (x_dtype == NVQ_DTYPE_BF16) return syrk_bf16((const uint16_t*)X, n, k, ldx, H, ws, s);
  hipError_t e = symmetrize_from_upper(H, k, s);
  if (e == hipSuccess) {
    GemmArgs a{};
    a.A = (const float*)X; a.lda = ldx;   // stored [n x k] = op(A)^T
    a.B = (const float*)X; a.ldb = ldx;
    a.C = H; a.ldc = k;
    a.M = k; a.N = k; a.K = n; a.batch = 1; a.alpha = 1.0f; a.beta = 1.0f;
    e = gemm_f32(a, true, false, false, kEpiAxpby, s);
  }
  if (e == hipSuccess) e = symmetrize_from_upper(H, k, s);
  return e;
}

// fail() with the entry point's name in front of the message.
int failp(int code, const char* fn, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = std::string(fn) + ": " + buf;
  return code;
}

int quant_check(const char* fn, const void* W, int w_dtype, int64_t m, int64_t k, int64_t ldw, const float* U,
                const float* H, const float* g, int n_cand, unsigned flags, const uint8_t* codes,
                const uint8_t* scales, const float* row_err, const void* ws, size_t ws_bytes) {
  const bool rtn = flags & NVQ_FLAG_RTN;
  const bool want_err = !(flags & NVQ_FLAG_NO_ERR);
  if (flags & ~(NVQ_FLAG_RTN | NVQ_FLAG_NO_ERR | NVQ_FLAG_FP64 | NVQ_FLAG_INDEP | NVQ_FLAG_CHECK_FINITE |
                NVQ_FLAG_CHOL_FACTOR))
    return failp(NVQ_ERR_VALUE, fn, "unknown flags 0x%x", flags);
  if (!W || !g || !codes || !scales) return failp(NVQ_ERR_NULL, fn, "W, g, codes and scales are required");
  if (!rtn && !U) return failp(NVQ_ERR_NULL, fn, "U is required without NVQ_FLAG_RTN");
  if (want_err && (!H || !row_err)) return failp(NVQ_ERR_NULL, fn, "H and row_err are required unless NVQ_FLAG_NO_ERR");
  if (!dtype_ok(w_dtype)) return failp(NVQ_ERR_DTYPE, fn, "w_dtype %d", w_dtype);
  if (m <= 0 || k <= 0 || k % 16 != 0 || ldw < k || ldw % 4 != 0)
    return failp(NVQ_ERR_SHAPE, fn, "m=%lld k=%lld ldw=%lld (need m>0, k>0, k%%16==0, ldw>=k, ldw%%4==0)",
                 (long long)m, (long long)k, (long long)ldw);
  if (n_cand < 1 || n_cand > 16) return failp(NVQ_ERR_NCAND, fn, "n_cand=%d", n_cand);
  if (!aligned(codes, 8)) return failp(NVQ_ERR_ALIGN, fn, "codes must be 8-byte aligned");
  if ((U && !aligned(U, 16)) || (H && !aligned(H, 16))) return failp(NVQ_ERR_ALIGN, fn, "U and H must be 16-byte aligned");
  QuantWs L = quant_ws(m, k, (flags & NVQ_FLAG_FP64) && !rtn, (flags & NVQ_FLAG_CHOL_FACTOR) && !rtn);
  if (!ws || ws_bytes < L.total || !aligned(ws, kAlign))
    return failp(NVQ_ERR_WORKSPACE, fn, "workspace needs %zu bytes (256-aligned), got %zu", L.total, ws_bytes);
  return NVQ_OK;
}

// A batch of nb equal-shape matrices for the quantizer: matrix e reads W + e
// * stride_w (elements of its dtype), U + e * stride_u, H + e * stride_h,
// g[e], writes codes + e*m*k/2, scales + e*m*k/16, row_err + e*m,
// row_loss + e*m, and uses its own workspace block at base + e * ws_stride
// bytes (the QuantWs layout).  Every launch covers all nb matrices.
struct QBatch {
  int64_t nb = 1, stride_w = 0, stride_u = 0, stride_h = 0;
  size_t ws_stride = 0;
};

// Weighted error dW H' dW^T, H' = 2 triu(H, 1) + diag(H), into the
// per-column-tile partial sums, then summed per row.
hipError_t weighted_error_all(const void* W, int bf, int64_t m, int64_t k, int64_t ldw, const float* H,
                              const float* g, const uint8_t* codes, const uint8_t* scales, float* row_err, float* dW,
                              float* part, const QBatch& qb, hipStream_t s) {
  const int64_t wsf = (int64_t)(qb.ws_stride / sizeof(float));
  const int64_t np = (k + kGemmTile - 1) / kGemmTile;
  hipError_t e = delta_w_launch(W, bf, m, k, ldw, codes, scales, g, dW, s, 0, -1, qb.nb, qb.stride_w, wsf);
  if (e == hipSuccess) {
    GemmArgs a{};
    a.A = dW; a.lda = k;
    a.B = H; a.ldb = k;
    a.D = dW; a.ldd = k;
    a.P = part; a.ldp = np;
    a.M = m; a.N = k; a.K = k; a.batch = (int)qb.nb; a.bi = 1; a.alpha = 1.0f; a.beta = 0.0f;
    a.sA2 = wsf; a.sB2 = qb.stride_h; a.sD2 = wsf; a.sP2 = wsf;
    a.kmode = kGemmKSymUpperB; a.noff = 0;
    e = gemm_f32(a, false, false, false, kEpiRowDot, s);
  }
  if (e == hipSuccess) e = row_sum_launch(part, m, np, row_err, s, qb.nb, wsf);
  return e;
}

// The fp32 sweep with two-level lazy updates (the same sums as eager GPTQ
// updates, in another order): a batch's errors update the rest of its
// 512-column block at once, and a finished block's error slab updates every
// later column.
hipError_t sweep_f32(int64_t m, int64_t k, const float* U, const float* g, int n_cand, bool indep, uint8_t* codes,
                     uint8_t* scales, float* row_loss, float* Wp, float* Eslab, const float* invd, const QBatch& qb,
                     hipStream_t s, const float* W0, const float* Mb) {
  const int64_t wsf = (int64_t)(qb.ws_stride / sizeof(float));
  SweepStrides bs;
  bs.wp = wsf; bs.u = qb.stride_u; bs.invd = wsf; bs.e = wsf; bs.mb = wsf;
  auto rank_update = [&](const float* Eb, int64_t r0, int64_t c0, int64_t kk, int64_t ncol) {
    GemmArgs a{};
    a.A = Eb; a.lda = kSuperBatch;
    a.B = U + r0 * k + c0; a.ldb = k;
    a.C = Wp + c0; a.ldc = k;
    a.M = m; a.N = ncol; a.K = kk; a.batch = (int)qb.nb; a.bi = 1; a.alpha = -1.0f; a.beta = 1.0f;
    a.sA2 = wsf; a.sB2 = qb.stride_u; a.sC2 = wsf;
    return gemm_f32(a, false, false, false, kEpiAxpby, s);
  };
  // With larger candidate groups the sweep launch itself applies the earlier
  // batches' errors of the block to its rows (pre columns); else a GEMM after
  // each batch updates the rest of the block.
  const bool inblock = sweep_applies_inblock(n_cand);
  hipError_t e = hipSuccess;
  for (int64_t s0 = 0; e == hipSuccess && s0 < k; s0 += kSuperBatch) {
    const int64_t s1 = std::min<int64_t>(k, s0 + kSuperBatch);
    for (int64_t i1 = s0; e == hipSuccess && i1 < s1; i1 += kBatch) {
      const int ncols = (int)std::min<int64_t>(kBatch, s1 - i1);
      e = sweep_batch_launch(Wp, U, invd, g, m, k, (int)i1, ncols, n_cand, indep, codes, scales, Eslab + (i1 - s0),
                             kSuperBatch, row_loss, s, qb.nb, bs, inblock ? (int)(i1 - s0) : 0, W0, Mb);
      const int64_t i2 = i1 + ncols;
      if (e == hipSuccess && !inblock && i2 < s1) e = rank_update(Eslab + (i1 - s0), i1, i2, ncols, s1 - i2);
    }
    if (e == hipSuccess && s1 < k) e = rank_update(Eslab, s0, s1, s1 - s0, k - s1);
  }
  return e;
}

// The quantization of nb matrices (arguments already checked).
hipError_t quant_run(const void* W, int w_dtype, int64_t m, int64_t k, int64_t ldw, const float* U, const float* H,
                     const float* g, int n_cand, unsigned flags, uint8_t* codes, uint8_t* scales, float* row_err,
                     float* row_loss, char* base, hipStream_t s, QBatch qb = QBatch()) {
  const bool rtn = flags & NVQ_FLAG_RTN;
  const bool want_err = !(flags & NVQ_FLAG_NO_ERR);
  const bool f64 = (flags & NVQ_FLAG_FP64) && !rtn;
  const bool indep = flags & NVQ_FLAG_INDEP;
  const bool chol = (flags & NVQ_FLAG_CHOL_FACTOR) && !rtn;
  QuantWs L = quant_ws(m, k, f64, chol);
  if (qb.ws_stride == 0) qb.ws_stride = L.total;
  float* Wp = (float*)(base + L.wp);
  float* Eslab = (float*)(base + L.eslab);
  float* invd = (float*)(base + L.invd);
  float* Mb = chol ? (float*)(base + L.mb) : nullptr;
  float* part = (float*)(base + L.part);
  const int bf = w_dtype == NVQ_DTYPE_BF16;
  hipError_t e = hipSuccess;

  if (rtn) {
    e = rtn_launch(W, bf, m, k, ldw, g, n_cand, codes, scales, row_loss, s, qb.nb, qb.stride_w);
  } else if (f64) {
    // The same sweep and two-level lazy updates with fp64 working weights and errors.
    double* Wd = (double*)(base + L.wp);
    double* W0d = chol ? (double*)(base + L.w0) : nullptr;
    double* Ed = (double*)(base + L.eslab);
    const int64_t wsd = (int64_t)(qb.ws_stride / sizeof(double));
    SweepStrides bs;
    bs.wp = wsd; bs.u = qb.stride_u; bs.e = wsd; bs.mb = (int64_t)(qb.ws_stride / sizeof(float));
    e = load_working_copy_f64(W, bf, m, k, ldw, Wd, s, qb.nb, qb.stride_w, wsd);
    if (e == hipSuccess && chol) e = chol_block_m_launch(U, k, Mb, s, qb.nb, qb.stride_u, bs.mb);
    if (e == hipSuccess && chol) e = load_working_copy_f64(W, bf, m, k, ldw, W0d, s, qb.nb, qb.stride_w, wsd);
    if (e == hipSuccess && row_loss) e = fill_f32(row_loss, qb.nb * m, 0.0f, s);
    for (int64_t s0 = 0; e == hipSuccess && s0 < k; s0 += kSuperBatch) {
      const int64_t s1 = std::min<int64_t>(k, s0 + kSuperBatch);
      for (int64_t i1 = s0; e == hipSuccess && i1 < s1; i1 += kBatch) {
        const int ncols = (int)std::min<int64_t>(kBatch, s1 - i1);
        e = sweep_batch_launch_f64(Wd, U, g, m, k, (int)i1, ncols, n_cand, indep, codes, scales, Ed + (i1 - s0),
                                   kSuperBatch, row_loss, s, qb.nb, bs, W0d, Mb);
        const int64_t i2 = i1 + ncols;
        if (e == hipSuccess && i2 < s1)
          e = rank_update_f64(Ed + (i1 - s0), kSuperBatch, U + i1 * k + i2, k, Wd + i2, k, m, s1 - i2, ncols, s,
                              qb.nb, wsd, qb.stride_u, wsd);
      }
      if (e == hipSuccess && s1 < k)
        e = rank_update_f64(Ed, kSuperBatch, U + s0 * k + s1, k, Wd + s1, k, m, k - s1, s1 - s0, s, qb.nb, wsd,
                            qb.stride_u, wsd);
    }
  } else {
    const int64_t wsf = (int64_t)(qb.ws_stride / sizeof(float));
    float* W0 = chol ? (float*)(base + L.w0) : nullptr;
    e = inv_diag_launch(U, k, invd, s, qb.nb, qb.stride_u, wsf, chol);
    if (e == hipSuccess && chol) e = chol_block_m_launch(U, k, Mb, s, qb.nb, qb.stride_u, wsf);
    if (e == hipSuccess) e = load_working_copy(W, bf, m, k, ldw, Wp, s, qb.nb, qb.stride_w, wsf);
    if (e == hipSuccess && chol) e = load_working_copy(W, bf, m, k, ldw, W0, s, qb.nb, qb.stride_w, wsf);
    if (e == hipSuccess && row_loss) e = fill_f32(row_loss, qb.nb * m, 0.0f, s);
    if (e == hipSuccess)
      e = sweep_f32(m, k, U, g, n_cand, indep, codes, scales, row_loss, Wp, Eslab, invd, qb, s, W0, Mb);
  }
  if (e == hipSuccess && want_err)
    e = weighted_error_all(W, bf, m, k, ldw, H, g, codes, scales, row_err, Wp, part, qb, s);
  if (e == hipSuccess && (flags & NVQ_FLAG_CHECK_FINITE))
    e = reject_nonfinite_rows_launch(W, bf, m, k, ldw, g, codes, scales, want_err ? row_err : nullptr, row_loss, s,
                                     qb.nb, qb.stride_w);
  return e;
}

}  // namespace

extern "C" {

const char* nvq_status_string(int status) {
  switch (status) {
    case NVQ_OK: return "ok";
    case NVQ_ERR_NULL: return "null pointer";
    case NVQ_ERR_SHAPE: return "invalid shape";
    case NVQ_ERR_DTYPE: return "unsupported dtype";
    case NVQ_ERR_NCAND: return "candidate count outside [1, 16]";
    case NVQ_ERR_WORKSPACE: return "workspace too small or misaligned";
    case NVQ_ERR_VALUE: return "invalid scalar argument";
    case NVQ_ERR_HIP: return "HIP runtime error";
    case NVQ_ERR_ALIGN: return "misaligned pointer";
    default: return "unknown status";
  }
}

const char* nvq_last_error(void) { return g_last_error.c_str(); }

// ---------------------------------------------------------------------------
size_t hessian_workspace_size(int64_t n, int64_t k, int x_dtype) {
  if (n <= 0 || k <= 0) return 0;
  if (x_dtype == NVQ_DTYPE_BF16) return align_up(syrk_bf16_workspace(n, k));
  return 0;
}

int hessian_accumulate(const void* X, int x_dtype, int64_t n, int64_t k, int64_t ldx, float* H, void* ws,
                       size_t ws_bytes, void* stream) {
  if (!H) return fail(NVQ_ERR_NULL, "hessian_accumulate: H is NULL");
  if (!dtype_ok(x_dtype)) return fail(NVQ_ERR_DTYPE, "hessian_accumulate: x_dtype %d", x_dtype);
  if (n < 0 || k <= 0 || k % 16 != 0 || ldx < k || ldx % 4 != 0)
    return fail(NVQ_ERR_SHAPE, "hessian_accumulate: n=%lld k=%lld ldx=%lld (need n>=0, k>0, k%%16==0, ldx>=k, ldx%%4==0)",
                (long long)n, (long long)k, (long long)ldx);
  if (n == 0) return NVQ_OK;
  if (!X) return fail(NVQ_ERR_NULL, "hessian_accumulate: X is NULL");
  if (!aligned(H, 16)) return fail(NVQ_ERR_ALIGN, "hessian_accumulate: H must be 16-byte aligned");
  if (!aligned(X, 16)) return fail(NVQ_ERR_ALIGN, "hessian_accumulate: X must be 16-byte aligned");
  if (x_dtype == NVQ_DTYPE_BF16 && ldx % 8 != 0)
    return fail(NVQ_ERR_SHAPE, "hessian_accumulate: bf16 rows must be 16-byte aligned (ldx %% 8 == 0)");
  size_t need = hessian_workspace_size(n, k, x_dtype);
  if (need && (!ws || ws_bytes < need || !aligned(ws, kAlign)))
    return fail(NVQ_ERR_WORKSPACE, "hessian_accumulate: workspace needs %zu bytes (256-aligned), got %zu", need,
                ws_bytes);
  return hip_status(hessian_run(X, x_dtype, n, k, ldx, H, ws, (hipStream_t)stream), "hessian_accumulate");
}

// ---- Hessian over host-resident activations ---------------------------------
namespace {
size_t host_chunk_bytes(int64_t chunk, int64_t k, int x_dtype) {
  return align_up((size_t)chunk * k * (x_dtype == NVQ_DTYPE_BF16 ? 2 : 4));
}
// Rows [r0, r0 + rows) of a host matrix with row stride ld into a dense buffer.
void copy_rows_host(char* dst, const char* src, int64_t rows, int64_t row_bytes, int64_t ld_bytes) {
  auto part = [&](int64_t a, int64_t b) {
    if (ld_bytes == row_bytes) {
      std::memcpy(dst + a * row_bytes, src + a * ld_bytes, (size_t)((b - a) * row_bytes));
    } else {
      for (int64_t r = a; r < b; ++r) std::memcpy(dst + r * row_bytes, src + r * ld_bytes, (size_t)row_bytes);
    }
  };
  const int64_t bytes = rows * row_bytes;
  const int nt = bytes >= (64ll << 20) ? 8 : (bytes >= (8ll << 20) ? 4 : 1);
  if (nt == 1) { part(0, rows); return; }
  std::vector<std::thread> th;
  for (int t = 0; t < nt; ++t) th.emplace_back(part, rows * t / nt, rows * (t + 1) / nt);
  for (auto& x : th) x.join();
}
}  // namespace

size_t hessian_host_workspace_size(int64_t chunk, int64_t k, int x_dtype) {
  if (chunk <= 0 || k <= 0 || !dtype_ok(x_dtype)) return 0;
  return 2 * host_chunk_bytes(chunk, k, x_dtype) + hessian_workspace_size(chunk, k, x_dtype);
}
size_t hessian_host_staging_size(int64_t chunk, int64_t k, int x_dtype) {
  if (chunk <= 0 || k <= 0 || !dtype_ok(x_dtype)) return 0;
  return 2 * host_chunk_bytes(chunk, k, x_dtype);
}

int hessian_accumulate_host(const void* X_host, int x_dtype, int64_t n, int64_t k, int64_t ldx, float* H,
                            int64_t chunk, void* ws, size_t ws_bytes, void* staging, size_t staging_bytes,
                            void* stream, void* copy_stream) {
  const char* fn = "hessian_accumulate_host";
  if (!H) return failp(NVQ_ERR_NULL, fn, "H is NULL");
  if (!dtype_ok(x_dtype)) return failp(NVQ_ERR_DTYPE, fn, "x_dtype %d", x_dtype);
  if (n < 0 || k <= 0 || k % 16 != 0 || ldx < k)
    return failp(NVQ_ERR_SHAPE, fn, "n=%lld k=%lld ldx=%lld (need n>=0, k>0, k%%16==0, ldx>=k)", (long long)n,
                 (long long)k, (long long)ldx);
  if (chunk <= 0) return failp(NVQ_ERR_SHAPE, fn, "chunk=%lld (need > 0)", (long long)chunk);
  if (n == 0) return NVQ_OK;
  if (!X_host) return failp(NVQ_ERR_NULL, fn, "X_host is NULL");
  if (!aligned(H, 16)) return failp(NVQ_ERR_ALIGN, fn, "H must be 16-byte aligned");
  const size_t need = hessian_host_workspace_size(chunk, k, x_dtype);
  if (!ws || ws_bytes < need || !aligned(ws, kAlign))
    return failp(NVQ_ERR_WORKSPACE, fn, "workspace needs %zu bytes (256-aligned), got %zu", need, ws_bytes);
  const size_t sneed = hessian_host_staging_size(chunk, k, x_dtype);
  if (staging && staging_bytes < sneed)
    return failp(NVQ_ERR_WORKSPACE, fn, "staging needs %zu bytes, got %zu", sneed, staging_bytes);

  const int64_t es = x_dtype == NVQ_DTYPE_BF16 ? 2 : 4;
  const size_t cb = host_chunk_bytes(chunk, k, x_dtype);
  char* dev[2] = {(char*)ws, (char*)ws + cb};
  void* hws = (char*)ws + 2 * cb;
  char* stg[2] = {(char*)staging, staging ? (char*)staging + cb : nullptr};
  hipStream_t s = (hipStream_t)stream, cs = copy_stream ? (hipStream_t)copy_stream : s;
  hipEvent_t copied[2] = {nullptr, nullptr}, used[2] = {nullptr, nullptr};
  hipError_t e = hipSuccess;
  for (int b = 0; b < 2 && e == hipSuccess; ++b) {
    e = hipEventCreateWithFlags(&copied[b], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&used[b], hipEventDisableTiming);
  }
  const char* src = (const char*)X_host;
  for (int64_t t0 = 0, i = 0; e == hipSuccess && t0 < n; t0 += chunk, ++i) {
    const int b = (int)(i & 1);
    const int64_t rows = std::min<int64_t>(chunk, n - t0);
    const char* from = src + t0 * ldx * es;
    int64_t from_ld = ldx * es;
    if (stg[0]) {
      // The copy out of this staging buffer two chunks ago must be done.
      if (i >= 2) e = hipEventSynchronize(copied[b]);
      if (e != hipSuccess) break;
      copy_rows_host(stg[b], from, rows, k * es, ldx * es);
      from = stg[b];
      from_ld = k * es;
    }
    // The device buffer's previous chunk must have been consumed.
    if (i >= 2) e = hipStreamWaitEvent(cs, used[b], 0);
    if (e == hipSuccess)
      e = hipMemcpy2DAsync(dev[b], (size_t)(k * es), from, (size_t)from_ld, (size_t)(k * es), (size_t)rows,
                           hipMemcpyHostToDevice, cs);
    if (e == hipSuccess) e = hipEventRecord(copied[b], cs);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, copied[b], 0);
    if (e == hipSuccess) e = hessian_run(dev[b], x_dtype, rows, k, k, H, hws, s);
    if (e == hipSuccess) e = hipEventRecord(used[b], s);
  }
  // With staging, return only once the staging buffers have been read, so the
  // caller may reuse them at once.
  for (int b = 0; b < 2 && stg[0] && e == hipSuccess; ++b) e = hipEventSynchronize(copied[b]);
  for (int b = 0; b < 2; ++b) {
    if (copied[b]) (void)hipEventDestroy(copied[b]);
    if (used[b]) (void)hipEventDestroy(used[b]);
  }
  return hip_status(e, fn);
}

// ---- consumer: NVFP4 weight-only GEMM ------------------------------------------
size_t nvfp4_gemm_workspace_size(int64_t T, int64_t k, int64_t m) { return align_up(nvfp4_gemm_workspace(T, k, m)); }

namespace {
// Arguments of nvfp4_gemm and its no-allocation variant; *empty is set when
// there is nothing to compute.
int gemm_check(const char* fn, const void* X, int x_dtype, int64_t T, int64_t k, int64_t ldx, const uint8_t* codes,
               const uint8_t* scales, const float* g, int64_t m, const void* Y, int y_dtype, int64_t ldy, bool* empty) {
  *empty = false;
  if (x_dtype != NVQ_DTYPE_BF16) return failp(NVQ_ERR_DTYPE, fn, "x_dtype %d (activations must be bf16)", x_dtype);
  if (!dtype_ok(y_dtype)) return failp(NVQ_ERR_DTYPE, fn, "y_dtype %d", y_dtype);
  if (T < 0 || m < 0 || k <= 0 || k % 16 != 0 || ldx < k || ldx % 8 != 0 || ldy < m)
    return failp(NVQ_ERR_SHAPE, fn, "T=%lld m=%lld k=%lld ldx=%lld ldy=%lld (need k%%16==0, ldx>=k, ldx%%8==0, ldy>=m)",
                 (long long)T, (long long)m, (long long)k, (long long)ldx, (long long)ldy);
  if (T == 0 || m == 0) {
    *empty = true;
    return NVQ_OK;
  }
  if (!X || !codes || !scales || !g || !Y) return failp(NVQ_ERR_NULL, fn, "X, codes, scales, g and Y are required");
  if (!aligned(X, 16)) return failp(NVQ_ERR_ALIGN, fn, "X must be 16-byte aligned");
  if (!aligned(codes, 8)) return failp(NVQ_ERR_ALIGN, fn, "codes must be 8-byte aligned");
  return NVQ_OK;
}
}  // namespace

int nvfp4_gemm(const void* X, int x_dtype, int64_t T, int64_t k, int64_t ldx, const uint8_t* codes,
               const uint8_t* scales, const float* g, int64_t m, void* Y, int y_dtype, int64_t ldy, void* ws,
               size_t ws_bytes, void* stream) {
  const char* fn = "nvfp4_gemm";
  bool empty = false;
  const int rc = gemm_check(fn, X, x_dtype, T, k, ldx, codes, scales, g, m, Y, y_dtype, ldy, &empty);
  if (rc != NVQ_OK || empty) return rc;
  const size_t need = nvfp4_gemm_workspace(T, k, m);
  if (need && (!ws || ws_bytes < need || !aligned(ws, kAlign)))
    return failp(NVQ_ERR_WORKSPACE, fn, "workspace needs %zu bytes (256-aligned), got %zu", need, ws_bytes);
  return hip_status(nvfp4_gemm_launch((const uint16_t*)X, T, k, ldx, codes, scales, g, m, Y,
                                      y_dtype == NVQ_DTYPE_BF16, ldy, (float*)ws, (hipStream_t)stream), fn);
}

int nvfp4_gemm_noalloc(const void* X, int x_dtype, int64_t T, int64_t k, int64_t ldx, const uint8_t* codes,
                       const uint8_t* scales, const float* g, int64_t m, void* Y, int y_dtype, int64_t ldy,
                       void* stream) {
  const char* fn = "nvfp4_gemm_noalloc";
  bool empty = false;
  const int rc = gemm_check(fn, X, x_dtype, T, k, ldx, codes, scales, g, m, Y, y_dtype, ldy, &empty);
  if (rc != NVQ_OK || empty) return rc;
  const size_t need = nvfp4_gemm_workspace(T, k, m);
  if (need > kNoAllocScratchBytes)
    return failp(NVQ_ERR_WORKSPACE, fn,
                 "T=%lld k=%lld m=%lld needs %zu bytes of partial sums; this variant holds at most %zu "
                 "(use nvfp4_gemm with a workspace)",
                 (long long)T, (long long)k, (long long)m, need, kNoAllocScratchBytes);
  float* scr = nullptr;
  hipError_t e = noalloc_scratch(&scr);
  if (e != hipSuccess) return hip_status(e, fn);
  return hip_status(nvfp4_gemm_launch((const uint16_t*)X, T, k, ldx, codes, scales, g, m, Y,
                                      y_dtype == NVQ_DTYPE_BF16, ldy, scr, (hipStream_t)stream), fn);
}

// Grouped Hessians: experts of at least kGroupedLarge tokens (or every expert
// when the grouped k = 4096 launch does not apply) are gathered and
// accumulated one at a time; the others are gathered one after another into
// the same row buffer and accumulated K4G_EXP at a time by one grouped launch
// each (a launch also ends when the buffer is full).  The buffer holds the
// largest expert's rows, and at least min(the small experts' rows, 2 GiB).
constexpr int64_t kGroupedLarge = 16384;
constexpr size_t kGroupedRowBytes = (size_t)2 << 30;

static bool grouped_launch_applies(int64_t k, int x_dtype) {
  return x_dtype == NVQ_DTYPE_BF16 && syrk_k4_grouped_applies(k);
}

static int64_t grouped_rows_cap(const int64_t* grp_off, int64_t G, int64_t k, int x_dtype, int64_t* nmax_out) {
  int64_t nmax = 0, small = 0;
  const bool grouped = grouped_launch_applies(k, x_dtype);
  for (int64_t e = 0; e < G; ++e) {
    const int64_t ne = grp_off[e + 1] - grp_off[e];
    nmax = std::max<int64_t>(nmax, ne);
    if (grouped && ne < kGroupedLarge) small += ne;
  }
  *nmax_out = nmax;
  const size_t esize = x_dtype == NVQ_DTYPE_BF16 ? 2 : 4;
  const int64_t cap = (int64_t)(kGroupedRowBytes / ((size_t)k * esize));
  return std::max<int64_t>(nmax, std::min<int64_t>(small, cap));
}

size_t hessian_grouped_workspace_size(const int64_t* grp_off, int64_t G, int64_t k, int x_dtype) {
  if (!grp_off || G <= 0 || k <= 0 || !dtype_ok(x_dtype)) return 0;
  int64_t nmax = 0;
  const int64_t rows = grouped_rows_cap(grp_off, G, k, x_dtype, &nmax);
  if (nmax <= 0) return 0;
  const size_t esize = x_dtype == NVQ_DTYPE_BF16 ? 2 : 4;
  return align_up((size_t)rows * k * esize) + hessian_workspace_size(nmax, k, x_dtype);
}

int hessian_accumulate_grouped(const void* X, int x_dtype, int64_t n, int64_t k, int64_t ldx, const int32_t* tok_idx,
                               const int64_t* grp_off, int64_t G, float* H, void* ws, size_t ws_bytes, void* stream) {
  if (!H || !grp_off) return fail(NVQ_ERR_NULL, "hessian_accumulate_grouped: H and grp_off are required");
  if (!dtype_ok(x_dtype)) return fail(NVQ_ERR_DTYPE, "hessian_accumulate_grouped: x_dtype %d", x_dtype);
  if (G <= 0 || n < 0 || k <= 0 || k % 16 != 0 || ldx < k || ldx % (x_dtype == NVQ_DTYPE_BF16 ? 8 : 4) != 0)
    return fail(NVQ_ERR_SHAPE, "hessian_accumulate_grouped: G=%lld n=%lld k=%lld ldx=%lld", (long long)G,
                (long long)n, (long long)k, (long long)ldx);
  if (grp_off[0] != 0) return fail(NVQ_ERR_VALUE, "hessian_accumulate_grouped: grp_off[0] must be 0");
  for (int64_t e = 0; e < G; ++e)
    if (grp_off[e + 1] < grp_off[e])
      return fail(NVQ_ERR_VALUE, "hessian_accumulate_grouped: grp_off must be non-decreasing (group %lld)", (long long)e);
  if (grp_off[G] == 0) return NVQ_OK;
  if (n == 0) return fail(NVQ_ERR_SHAPE, "hessian_accumulate_grouped: assignments given but n = 0");
  if (!X || !tok_idx) return fail(NVQ_ERR_NULL, "hessian_accumulate_grouped: X and tok_idx are required");
  if (!aligned(H, 16) || !aligned(X, 16)) return fail(NVQ_ERR_ALIGN, "hessian_accumulate_grouped: X and H must be 16-byte aligned");
  const size_t need = hessian_grouped_workspace_size(grp_off, G, k, x_dtype);
  if (!ws || ws_bytes < need || !aligned(ws, kAlign))
    return fail(NVQ_ERR_WORKSPACE, "hessian_accumulate_grouped: workspace needs %zu bytes (256-aligned), got %zu", need,
                ws_bytes);
  hipStream_t s = (hipStream_t)stream;
  const int esize = x_dtype == NVQ_DTYPE_BF16 ? 2 : 4;
  int64_t nmax = 0;
  const int64_t cap = grouped_rows_cap(grp_off, G, k, x_dtype, &nmax);
  const bool grouped = grouped_launch_applies(k, x_dtype);
  char* rows = (char*)ws;
  void* hws = rows + align_up((size_t)cap * k * esize);
  hipError_t err = hipSuccess;
  for (int64_t e = 0; err == hipSuccess && e < G; ++e) {
    const int64_t ne = grp_off[e + 1] - grp_off[e];
    if (ne == 0 || (grouped && ne < kGroupedLarge)) continue;
    err = gather_rows(X, esize, ldx, tok_idx + grp_off[e], n, ne, k, rows, s);
    if (err == hipSuccess) err = hessian_run(rows, x_dtype, ne, k, k, H + (size_t)e * k * k, hws, s);
  }
  if (grouped) {
    K4Grouped g{};
    int nexp = 0;
    int64_t used = 0;
    for (int64_t e = 0; err == hipSuccess && e <= G; ++e) {
      const int64_t ne = e < G ? grp_off[e + 1] - grp_off[e] : 0;
      if (e < G && (ne == 0 || ne >= kGroupedLarge)) continue;
      if (nexp > 0 && (e == G || nexp == K4G_EXP || used + ne > cap)) {
        err = syrk_bf16_grouped((const uint16_t*)rows, k, g, nexp, H, s);
        nexp = 0;
        used = 0;
      }
      if (e == G || err != hipSuccess) break;
      err = gather_rows(X, esize, ldx, tok_idx + grp_off[e], n, ne, k, rows + (size_t)used * k * esize, s);
      g.beg[nexp] = (int32_t)used;
      g.cnt[nexp] = (int32_t)ne;
      g.hexp[nexp] = (int32_t)e;
      ++nexp;
      used += ne;
    }
  }
  return hip_status(err, "hessian_accumulate_grouped");
}

// ---------------------------------------------------------------------------
size_t factor_hinv_workspace_size(int64_t k) { return k > 0 ? align_up(factor_workspace(k)) : 0; }

int factor_hinv(const float* H, int64_t k, float damp_rel, float* U, float* lambda_out, int32_t* info, void* ws,
                size_t ws_bytes, void* stream) {
  if (!H || !U || !lambda_out || !info) return fail(NVQ_ERR_NULL, "factor_hinv: H, U, lambda_out and info are required");
  if (k <= 0 || k % 16 != 0) return fail(NVQ_ERR_SHAPE, "factor_hinv: k=%lld (need k>0, k%%16==0)", (long long)k);
  if (!(damp_rel >= 0.0f) || !std::isfinite(damp_rel))
    return fail(NVQ_ERR_VALUE, "factor_hinv: damp_rel must be finite and >= 0");
  if (H == U) return fail(NVQ_ERR_VALUE, "factor_hinv: U must not overlap H");
  if (!aligned(H, 16) || !aligned(U, 16)) return fail(NVQ_ERR_ALIGN, "factor_hinv: H and U must be 16-byte aligned");
  size_t need = factor_hinv_workspace_size(k);
  if (!ws || ws_bytes < need || !aligned(ws, kAlign))
    return fail(NVQ_ERR_WORKSPACE, "factor_hinv: workspace needs %zu bytes (256-aligned), got %zu", need, ws_bytes);
  return hip_status(factor_hinv_launch(H, k, 1, k * k, damp_rel, U, k * k, lambda_out, info, ws, 1,
                                       (hipStream_t)stream), "factor_hinv");
}

// factor_hinv_batched and factor_chol_batched: the same checks, the U form or
// the Cholesky-factor form over passes of as many matrices as the workspace
// holds.
static int factor_batched(const char* fn, bool chol, const float* H, int64_t k, int64_t batch, int64_t stride_h,
                          float damp_rel, float* U, int64_t stride_u, float* lambda_out, int32_t* info, void* ws,
                          size_t ws_bytes, void* stream) {
  if (batch < 0) return failp(NVQ_ERR_SHAPE, fn, "batch=%lld", (long long)batch);
  if (batch == 0) return NVQ_OK;
  if (!H || !U || !lambda_out || !info) return failp(NVQ_ERR_NULL, fn, "H, the output, lambda_out and info are required");
  if (k <= 0 || k % 16 != 0) return failp(NVQ_ERR_SHAPE, fn, "k=%lld (need k>0, k%%16==0)", (long long)k);
  if (stride_h < k * k || stride_u < k * k || stride_h % 4 != 0 || stride_u % 4 != 0)
    return failp(NVQ_ERR_SHAPE, fn, "strides must be >= k*k and multiples of 4");
  if (!(damp_rel >= 0.0f) || !std::isfinite(damp_rel)) return failp(NVQ_ERR_VALUE, fn, "damp_rel must be finite and >= 0");
  if ((const float*)U < H + (size_t)stride_h * batch && H < (const float*)U + (size_t)stride_u * batch)
    return failp(NVQ_ERR_VALUE, fn, "the output must not overlap H");
  if (!aligned(H, 16) || !aligned(U, 16)) return failp(NVQ_ERR_ALIGN, fn, "H and the output must be 16-byte aligned");
  const size_t one = factor_hinv_workspace_size(k);
  if (!ws || ws_bytes < one || !aligned(ws, kAlign))
    return failp(NVQ_ERR_WORKSPACE, fn, "workspace needs at least %zu bytes (256-aligned), got %zu", one, ws_bytes);
  const int64_t chunk = std::min<int64_t>((int64_t)(ws_bytes / one), batch);
  return hip_status(factor_hinv_launch(H, k, batch, stride_h, damp_rel, U, stride_u, lambda_out, info, ws, chunk,
                                       (hipStream_t)stream, chol), fn);
}

int factor_hinv_batched(const float* H, int64_t k, int64_t batch, int64_t stride_h, float damp_rel, float* U,
                        int64_t stride_u, float* lambda_out, int32_t* info, void* ws, size_t ws_bytes, void* stream) {
  return factor_batched("factor_hinv_batched", false, H, k, batch, stride_h, damp_rel, U, stride_u, lambda_out, info,
                        ws, ws_bytes, stream);
}

int factor_chol_batched(const float* H, int64_t k, int64_t batch, int64_t stride_h, float damp_rel, float* V,
                        int64_t stride_v, float* lambda_out, int32_t* info, void* ws, size_t ws_bytes, void* stream) {
  return factor_batched("factor_chol_batched", true, H, k, batch, stride_h, damp_rel, V, stride_v, lambda_out, info,
                        ws, ws_bytes, stream);
}

size_t factor_chol_workspace_size(int64_t k) { return factor_hinv_workspace_size(k); }

int factor_chol(const float* H, int64_t k, float damp_rel, float* V, float* lambda_out, int32_t* info, void* ws,
                size_t ws_bytes, void* stream) {
  const char* fn = "factor_chol";
  if (!H || !V || !lambda_out || !info) return failp(NVQ_ERR_NULL, fn, "H, V, lambda_out and info are required");
  if (k <= 0 || k % 16 != 0) return failp(NVQ_ERR_SHAPE, fn, "k=%lld (need k>0, k%%16==0)", (long long)k);
  if (!(damp_rel >= 0.0f) || !std::isfinite(damp_rel)) return failp(NVQ_ERR_VALUE, fn, "damp_rel must be finite and >= 0");
  if (H == V) return failp(NVQ_ERR_VALUE, fn, "V must not overlap H");
  if (!aligned(H, 16) || !aligned(V, 16)) return failp(NVQ_ERR_ALIGN, fn, "H and V must be 16-byte aligned");
  const size_t need = factor_chol_workspace_size(k);
  if (!ws || ws_bytes < need || !aligned(ws, kAlign))
    return failp(NVQ_ERR_WORKSPACE, fn, "workspace needs %zu bytes (256-aligned), got %zu", need, ws_bytes);
  return hip_status(factor_hinv_launch(H, k, 1, k * k, damp_rel, V, k * k, lambda_out, info, ws, 1,
                                       (hipStream_t)stream, true), fn);
}

// ---------------------------------------------------------------------------
size_t nvfp4_global_scale_workspace_size(int64_t m, int64_t k) {
  return (m > 0 && k > 0) ? align_up((size_t)global_scale_parts(m, k) * sizeof(float)) : 0;
}

int nvfp4_global_scale(const void* W, int w_dtype, int64_t m, int64_t k, int64_t ldw, float* g_out, void* ws,
                       size_t ws_bytes, void* stream) {
  if (!W || !g_out) return fail(NVQ_ERR_NULL, "nvfp4_global_scale: W and g_out are required");
  if (!dtype_ok(w_dtype)) return fail(NVQ_ERR_DTYPE, "nvfp4_global_scale: w_dtype %d", w_dtype);
  if (m <= 0 || k <= 0 || ldw < k) return fail(NVQ_ERR_SHAPE, "nvfp4_global_scale: m=%lld k=%lld ldw=%lld",
                                               (long long)m, (long long)k, (long long)ldw);
  size_t need = nvfp4_global_scale_workspace_size(m, k);
  if (!ws || ws_bytes < need || !aligned(ws, kAlign))
    return fail(NVQ_ERR_WORKSPACE, "nvfp4_global_scale: workspace needs %zu bytes, got %zu", need, ws_bytes);
  return hip_status(global_scale_launch(W, w_dtype == NVQ_DTYPE_BF16, m, k, ldw, g_out, (float*)ws,
                                        global_scale_parts(m, k), (hipStream_t)stream),
                    "nvfp4_global_scale");
}

// ---------------------------------------------------------------------------
size_t gptq_nvfp4_workspace_size(int64_t m, int64_t k, unsigned flags) {
  if (m <= 0 || k <= 0) return 0;
  const bool rtn = flags & NVQ_FLAG_RTN;
  return quant_ws(m, k, (flags & NVQ_FLAG_FP64) && !rtn, (flags & NVQ_FLAG_CHOL_FACTOR) && !rtn).total;
}

int gptq_nvfp4_quantize(const void* W, int w_dtype, int64_t m, int64_t k, int64_t ldw, const float* U,
                        const float* H, const float* g, int n_cand, unsigned flags, uint8_t* codes, uint8_t* scales,
                        float* row_err, float* row_loss, void* ws, size_t ws_bytes, void* stream) {
  const int rc = quant_check("gptq_nvfp4_quantize", W, w_dtype, m, k, ldw, U, H, g, n_cand, flags, codes, scales,
                             row_err, ws, ws_bytes);
  if (rc != NVQ_OK) return rc;
  return hip_status(quant_run(W, w_dtype, m, k, ldw, U, H, g, n_cand, flags, codes, scales, row_err, row_loss,
                              (char*)ws, (hipStream_t)stream),
                    "gptq_nvfp4_quantize");
}

int gptq_nvfp4_quantize_batched(const void* W, int w_dtype, int64_t batch, int64_t m, int64_t k, int64_t ldw,
                                int64_t stride_w, const float* U, int64_t stride_u, const float* H, int64_t stride_h,
                                const float* g, int n_cand, unsigned flags, uint8_t* codes, uint8_t* scales,
                                float* row_err, float* row_loss, void* ws, size_t ws_bytes, void* stream) {
  if (batch < 0) return fail(NVQ_ERR_SHAPE, "gptq_nvfp4_quantize_batched: batch=%lld", (long long)batch);
  if (batch == 0) return NVQ_OK;
  const int rc = quant_check("gptq_nvfp4_quantize_batched", W, w_dtype, m, k, ldw, U, H, g, n_cand, flags, codes,
                             scales, row_err, ws, ws_bytes);
  if (rc != NVQ_OK) return rc;
  const bool rtn = flags & NVQ_FLAG_RTN, want_err = !(flags & NVQ_FLAG_NO_ERR);
  if (stride_w < m * ldw || (!rtn && (stride_u < k * k || stride_u % 4 != 0)) ||
      (want_err && (stride_h < k * k || stride_h % 4 != 0)))
    return fail(NVQ_ERR_SHAPE, "gptq_nvfp4_quantize_batched: strides must cover one element (W: m*ldw, U and H: k*k, "
                               "multiples of 4)");
  // As many matrices per pass as the workspace holds (each launch covers all of them).
  const QuantWs L = quant_ws(m, k, (flags & NVQ_FLAG_FP64) && !rtn, (flags & NVQ_FLAG_CHOL_FACTOR) && !rtn);
  const int64_t chunk = std::max<int64_t>(1, std::min<int64_t>({batch, (int64_t)(ws_bytes / L.total), 65535}));
  const size_t es = w_dtype == NVQ_DTYPE_BF16 ? 2 : 4;
  QBatch qb;
  qb.stride_w = stride_w; qb.stride_u = stride_u; qb.stride_h = stride_h; qb.ws_stride = L.total;
  hipError_t err = hipSuccess;
  for (int64_t e = 0; err == hipSuccess && e < batch; e += chunk) {
    qb.nb = std::min<int64_t>(chunk, batch - e);
    err = quant_run((const char*)W + (size_t)e * stride_w * es, w_dtype, m, k, ldw,
                    U ? U + (size_t)e * stride_u : nullptr, H ? H + (size_t)e * stride_h : nullptr, g + e, n_cand,
                    flags, codes + (size_t)e * m * (k / 2), scales + (size_t)e * m * (k / kBlock),
                    row_err ? row_err + (size_t)e * m : nullptr, row_loss ? row_loss + (size_t)e * m : nullptr,
                    (char*)ws, (hipStream_t)stream, qb);
  }
  return hip_status(err, "gptq_nvfp4_quantize_batched");
}

// ---------------------------------------------------------------------------
int nvq_check_finite(const void* A, int dtype, int64_t rows, int64_t cols, int64_t ld, int32_t* status,
                     void* stream) {
  const char* fn = "nvq_check_finite";
  if (!status) return failp(NVQ_ERR_NULL, fn, "status is NULL");
  if (!dtype_ok(dtype)) return failp(NVQ_ERR_DTYPE, fn, "dtype %d", dtype);
  if (rows < 0 || cols <= 0 || ld < cols || rows > 0x7FFFFFFE)
    return failp(NVQ_ERR_SHAPE, fn, "rows=%lld cols=%lld ld=%lld (need 0<=rows<2^31-1, cols>0, ld>=cols)",
                 (long long)rows, (long long)cols, (long long)ld);
  if (rows > 0 && !A) return failp(NVQ_ERR_NULL, fn, "A is NULL");
  if (!aligned(status, 4)) return failp(NVQ_ERR_ALIGN, fn, "status must be 4-byte aligned");
  return hip_status(nonfinite_scan_launch(A, dtype == NVQ_DTYPE_BF16, rows, cols, ld, status, (hipStream_t)stream), fn);
}

// ---------------------------------------------------------------------------
int nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* g, int64_t m, int64_t k, void* out,
                     int out_dtype, void* stream) {
  if (m < 0 || k <= 0 || k % 16 != 0) return fail(NVQ_ERR_SHAPE, "nvfp4_dequantize: m=%lld k=%lld", (long long)m,
                                                  (long long)k);
  if (!dtype_ok(out_dtype)) return fail(NVQ_ERR_DTYPE, "nvfp4_dequantize: out_dtype %d", out_dtype);
  if (m == 0) return NVQ_OK;
  if (!codes || !scales || !g || !out) return fail(NVQ_ERR_NULL, "nvfp4_dequantize: null argument");
  if (!aligned(codes, 8) || !aligned(out, 16)) return fail(NVQ_ERR_ALIGN, "nvfp4_dequantize: codes need 8-byte and out 16-byte alignment");
  return hip_status(dequant_launch(codes, scales, g, m, k, out, out_dtype == NVQ_DTYPE_BF16, (hipStream_t)stream),
                    "nvfp4_dequantize");
}

}  // extern "C"
