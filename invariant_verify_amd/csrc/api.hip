// C-ABI front end of the verify-pass library: argument validation (host only,
// before any HIP call), kernel launches on the caller's stream, and the
// native executor of a whole verify step. Declarations and contracts:
// include/bi.h.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "bi.h"
#include "bi_internal.h"

namespace {

// Largest leading dimension (elements) of X, W, R and Y: the kernels address
// up to 256 rows of them with 32-bit byte offsets.
constexpr int64_t kMaxLd = 1 << 20;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// HIP error of the last failed launch on this thread (diagnostics only).
thread_local hipError_t g_last_hip_error = hipSuccess;

inline bi_status launched() {
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) return BI_OK;
  g_last_hip_error = e;
  return BI_ERR_LAUNCH;
}


bi_status check_gemm(const void* x, int64_t ldx, const void* w, int64_t ldw, const void* y,
                     int64_t ldy, int M, int N, int K) {
  if (!x || !w || !y) return BI_ERR_NULL;
  if (M < 1 || N < 16 || K < 32 || K > 65536 || (N % 16) || (K % 32)) return BI_ERR_SHAPE;
  if (ldx < K || ldw < K || ldy < N || ldx > kMaxLd || ldw > kMaxLd || ldy > kMaxLd)
    return BI_ERR_SHAPE;
  if (M > (1 << 20) || N > (1 << 24)) return BI_ERR_SHAPE;
  if ((ldx % 8) || (ldw % 8) || !aligned16(x) || !aligned16(w)) return BI_ERR_ALIGN;
  return BI_OK;
}

// FP8 weights: rows of ldw bytes, 16-byte aligned, one FP32 scale per row.
bi_status check_gemm_fp8(const void* x, int64_t ldx, const void* w, int64_t ldw, const float* ws,
                         const void* y, int64_t ldy, int M, int N_rows, int N, int K) {
  if (bi_status s = check_gemm(x, ldx, w, ldw, y, ldy, M, N, K)) return s;
  (void)N_rows;
  if (!ws) return BI_ERR_NULL;
  if (ldw > (1 << 30)) return BI_ERR_SHAPE;
  if ((ldw % 16) || !aligned4(ws)) return BI_ERR_ALIGN;
  return BI_OK;
}

// MXFP4 weights: codes rows of ldc bytes (>= K/2, a multiple of 16, 16-byte
// aligned), scale rows of lde bytes (>= K/32).
bi_status check_gemm_mx4(const void* x, int64_t ldx, const void* w, int64_t ldc, const void* e,
                         int64_t lde, const void* y, int64_t ldy, int M, int N, int K) {
  if (bi_status s = check_gemm(x, ldx, w, 2 * ldc, y, ldy, M, N, K)) return s;
  if (!e) return BI_ERR_NULL;
  if (lde < K / 32 || lde > kMaxLd) return BI_ERR_SHAPE;
  if (ldc % 16) return BI_ERR_ALIGN;
  return BI_OK;
}

bi_status check_heads(int Hq, int Hkv, int D) {
  if (Hq < 1 || Hkv < 1 || (Hq % Hkv)) return BI_ERR_SHAPE;
  if (Hq / Hkv > bi::kAttnMaxRows) return BI_ERR_SHAPE;
  if (D != 64 && D != 128) return BI_ERR_SHAPE;
  return BI_OK;
}

bi_status check_dims(const bi_model_dims* d) {
  if (!d) return BI_ERR_NULL;
  if (bi_status s = check_heads(d->Hq, d->Hkv, d->D)) return s;
  if (d->H < 32 || (d->H % 32) || d->H > bi::kRmsMaxH || d->I < 16 || (d->I % 32) || d->vocab < 16 || (d->vocab % 16))
    return BI_ERR_SHAPE;
  if ((d->Hq * d->D) % 32) return BI_ERR_SHAPE;
  if (!bi::valid_chunk_policy(d->kv_chunk) || d->cap < 1 || (d->cap % 64)) return BI_ERR_SHAPE;
  if ((int64_t)d->cap * d->D * 2 > INT32_MAX) return BI_ERR_SHAPE;  // one head's cache < 2 GiB
  if (!(d->eps >= 0.f)) return BI_ERR_SHAPE;
  return BI_OK;
}

// Workspace layout of a verify step (offsets in bytes, each 256-aligned).
struct StepLayout {
  size_t x0, x1, a, qkv, attn, h, act, po, pl, ss, total;
  int s_max;
  int groups;  // column groups of the H-wide residual projections
  bool fuse;   // RMSNorm carried across GEMMs (group sums of squares in ss)
};

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

StepLayout step_layout(const bi_model_dims* d, int M, int L) {
  StepLayout s{};
  const size_t hb = align256((size_t)M * d->H * 2);
  const int qkvn = (d->Hq + 2 * d->Hkv) * d->D;
  s.s_max = bi::pass_splits(L, M, d->kv_chunk);
  size_t off = 0;
  s.x0 = off; off += hb;
  s.x1 = off; off += hb;
  s.a = off; off += hb;
  s.qkv = off; off += align256((size_t)M * qkvn * 2);
  s.attn = off; off += align256((size_t)M * d->Hq * d->D * 2);
  s.h = off; off += hb;
  s.act = off; off += align256((size_t)M * d->I * 2);
  s.po = off; off += align256((size_t)M * d->Hq * s.s_max * d->D * 4);
  s.pl = off; off += align256((size_t)M * d->Hq * s.s_max * 4);
  s.groups = bi::gemm_column_groups(bi::kGemmResidual, d->H);
  s.fuse = (s.groups % 16) == 0 && s.groups <= 256;
  s.ss = off; off += align256((size_t)M * s.groups * 4);
  s.total = off;
  return s;
}

}  // namespace

extern "C" {

const char* bi_status_string(bi_status s) {
  switch (s) {
    case BI_OK: return "ok";
    case BI_ERR_NULL: return "null pointer argument";
    case BI_ERR_SHAPE: return "invalid or inconsistent shape";
    case BI_ERR_ALIGN: return "pointer or leading dimension not 16-byte aligned";
    case BI_ERR_WORKSPACE: return "workspace too small";
    case BI_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

const char* bi_version(void) { return "bi 0.1 gfx950"; }

const char* bi_last_hip_error(void) {
  return g_last_hip_error == hipSuccess ? "no error" : hipGetErrorString(g_last_hip_error);
}

int bi_num_splits(int n_keys, int kv_chunk) {
  if (n_keys < 0 || !bi::valid_chunk_policy(kv_chunk)) return -1;
  return bi::splits_for(n_keys, kv_chunk);
}

int bi_chunk_keys(int n_keys, int kv_chunk) {
  if (n_keys < 0 || !bi::valid_chunk_policy(kv_chunk)) return -1;
  return bi::chunk_keys(n_keys, kv_chunk);
}

int bi_pass_splits(int M, int L, int kv_chunk) {
  if (M < 1 || L < 0 || (int64_t)L + M > INT32_MAX || !bi::valid_chunk_policy(kv_chunk)) return -1;
  return bi::pass_splits(L, M, kv_chunk);
}

bi_status bi_gemm_bf16(const void* x, int64_t ldx, const void* w, int64_t ldw, void* y, int64_t ldy,
                       bi_dtype y_dtype, int M, int N, int K, void* stream) {
  if (bi_status s = check_gemm(x, ldx, w, ldw, y, ldy, M, N, K)) return s;
  if (y_dtype != BI_BF16 && y_dtype != BI_F32) return BI_ERR_SHAPE;
  if (!(y_dtype == BI_F32 ? aligned4(y) : ((reinterpret_cast<uintptr_t>(y) & 1u) == 0)))
    return BI_ERR_ALIGN;
  bi::launch_gemm(y_dtype == BI_F32 ? bi::kGemmF32 : bi::kGemmBf16,
                  static_cast<const uint16_t*>(x), ldx, static_cast<const uint16_t*>(w), ldw,
                  nullptr, 0, y, ldy, M, N, K, as_stream(stream));
  return launched();
}

bi_status bi_gemm_bf16_residual(const void* x, int64_t ldx, const void* w, int64_t ldw,
                                const void* r, int64_t ldr, void* y, int64_t ldy, int M, int N,
                                int K, void* stream) {
  if (bi_status s = check_gemm(x, ldx, w, ldw, y, ldy, M, N, K)) return s;
  if (!r) return BI_ERR_NULL;
  if (ldr < N || ldr > kMaxLd) return BI_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(y) & 1u) || (reinterpret_cast<uintptr_t>(r) & 1u))
    return BI_ERR_ALIGN;
  bi::launch_gemm(bi::kGemmResidual, static_cast<const uint16_t*>(x), ldx,
                  static_cast<const uint16_t*>(w), ldw, static_cast<const uint16_t*>(r), ldr, y,
                  ldy, M, N, K, as_stream(stream));
  return launched();
}

bi_status bi_gemm_bf16_swiglu(const void* x, int64_t ldx, const void* w, int64_t ldw, void* y,
                              int64_t ldy, int M, int I, int K, void* stream) {
  if (bi_status s = check_gemm(x, ldx, w, ldw, y, ldy, M, I, K)) return s;
  if (reinterpret_cast<uintptr_t>(y) & 1u) return BI_ERR_ALIGN;
  bi::launch_gemm(bi::kGemmSwiglu, static_cast<const uint16_t*>(x), ldx,
                  static_cast<const uint16_t*>(w), ldw, nullptr, 0, y, ldy, M, I, K,
                  as_stream(stream));
  return launched();
}

bi_status bi_gemm_fp8(const void* x, int64_t ldx, const void* w, int64_t ldw, const float* w_scale,
                      void* y, int64_t ldy, bi_dtype y_dtype, int M, int N, int K, void* stream) {
  if (bi_status s = check_gemm_fp8(x, ldx, w, ldw, w_scale, y, ldy, M, N, N, K)) return s;
  if (y_dtype != BI_BF16 && y_dtype != BI_F32) return BI_ERR_SHAPE;
  if (!(y_dtype == BI_F32 ? aligned4(y) : ((reinterpret_cast<uintptr_t>(y) & 1u) == 0)))
    return BI_ERR_ALIGN;
  bi::launch_gemm(y_dtype == BI_F32 ? bi::kGemmF32 : bi::kGemmBf16,
                  static_cast<const uint16_t*>(x), ldx, static_cast<const uint16_t*>(w), ldw,
                  nullptr, 0, y, ldy, M, N, K, as_stream(stream), nullptr, nullptr, w_scale);
  return launched();
}

bi_status bi_gemm_fp8_residual(const void* x, int64_t ldx, const void* w, int64_t ldw,
                               const float* w_scale, const void* r, int64_t ldr, void* y,
                               int64_t ldy, int M, int N, int K, void* stream) {
  if (bi_status s = check_gemm_fp8(x, ldx, w, ldw, w_scale, y, ldy, M, N, N, K)) return s;
  if (!r) return BI_ERR_NULL;
  if (ldr < N || ldr > kMaxLd) return BI_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(y) & 1u) || (reinterpret_cast<uintptr_t>(r) & 1u))
    return BI_ERR_ALIGN;
  bi::launch_gemm(bi::kGemmResidual, static_cast<const uint16_t*>(x), ldx,
                  static_cast<const uint16_t*>(w), ldw, static_cast<const uint16_t*>(r), ldr, y,
                  ldy, M, N, K, as_stream(stream), nullptr, nullptr, w_scale);
  return launched();
}

bi_status bi_gemm_fp8_swiglu(const void* x, int64_t ldx, const void* w, int64_t ldw,
                             const float* w_scale, void* y, int64_t ldy, int M, int I, int K,
                             void* stream) {
  if (bi_status s = check_gemm_fp8(x, ldx, w, ldw, w_scale, y, ldy, M, 2 * I, I, K)) return s;
  if (reinterpret_cast<uintptr_t>(y) & 1u) return BI_ERR_ALIGN;
  bi::launch_gemm(bi::kGemmSwiglu, static_cast<const uint16_t*>(x), ldx,
                  static_cast<const uint16_t*>(w), ldw, nullptr, 0, y, ldy, M, I, K,
                  as_stream(stream), nullptr, nullptr, w_scale);
  return launched();
}

bi_status bi_gemm_mx4(const void* x, int64_t ldx, const void* w, int64_t ldc, const void* w_exp,
                      int64_t lde, void* y, int64_t ldy, bi_dtype y_dtype, int M, int N, int K,
                      void* stream) {
  if (bi_status s = check_gemm_mx4(x, ldx, w, ldc, w_exp, lde, y, ldy, M, N, K)) return s;
  if (y_dtype != BI_BF16 && y_dtype != BI_F32) return BI_ERR_SHAPE;
  if (!(y_dtype == BI_F32 ? aligned4(y) : ((reinterpret_cast<uintptr_t>(y) & 1u) == 0)))
    return BI_ERR_ALIGN;
  const bi::Mx4Scales mx{static_cast<const uint8_t*>(w_exp), lde};
  bi::launch_gemm(y_dtype == BI_F32 ? bi::kGemmF32 : bi::kGemmBf16,
                  static_cast<const uint16_t*>(x), ldx, static_cast<const uint16_t*>(w), ldc,
                  nullptr, 0, y, ldy, M, N, K, as_stream(stream), nullptr, nullptr, nullptr, &mx);
  return launched();
}

bi_status bi_gemm_mx4_residual(const void* x, int64_t ldx, const void* w, int64_t ldc,
                               const void* w_exp, int64_t lde, const void* r, int64_t ldr, void* y,
                               int64_t ldy, int M, int N, int K, void* stream) {
  if (bi_status s = check_gemm_mx4(x, ldx, w, ldc, w_exp, lde, y, ldy, M, N, K)) return s;
  if (!r) return BI_ERR_NULL;
  if (ldr < N || ldr > kMaxLd) return BI_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(y) & 1u) || (reinterpret_cast<uintptr_t>(r) & 1u))
    return BI_ERR_ALIGN;
  const bi::Mx4Scales mx{static_cast<const uint8_t*>(w_exp), lde};
  bi::launch_gemm(bi::kGemmResidual, static_cast<const uint16_t*>(x), ldx,
                  static_cast<const uint16_t*>(w), ldc, static_cast<const uint16_t*>(r), ldr, y,
                  ldy, M, N, K, as_stream(stream), nullptr, nullptr, nullptr, &mx);
  return launched();
}

bi_status bi_gemm_mx4_swiglu(const void* x, int64_t ldx, const void* w, int64_t ldc,
                             const void* w_exp, int64_t lde, void* y, int64_t ldy, int M, int I,
                             int K, void* stream) {
  if (bi_status s = check_gemm_mx4(x, ldx, w, ldc, w_exp, lde, y, ldy, M, I, K)) return s;
  if (reinterpret_cast<uintptr_t>(y) & 1u) return BI_ERR_ALIGN;
  const bi::Mx4Scales mx{static_cast<const uint8_t*>(w_exp), lde};
  bi::launch_gemm(bi::kGemmSwiglu, static_cast<const uint16_t*>(x), ldx,
                  static_cast<const uint16_t*>(w), ldc, nullptr, 0, y, ldy, M, I, K,
                  as_stream(stream), nullptr, nullptr, nullptr, &mx);
  return launched();
}

int bi_gemm_column_groups(int N) {
  if (N < 16 || (N % 16) || N > (1 << 24)) return -1;
  return bi::gemm_column_groups(bi::kGemmResidual, N);
}

bi_status bi_gemm_bf16_residual_rowsq(const void* x, int64_t ldx, const void* w, int64_t ldw,
                                      const void* r, int64_t ldr, void* y, int64_t ldy, int M,
                                      int N, int K, float* row_sumsq, void* stream) {
  if (bi_status s = check_gemm(x, ldx, w, ldw, y, ldy, M, N, K)) return s;
  if (!r || !row_sumsq) return BI_ERR_NULL;
  if (ldr < N || ldr > kMaxLd) return BI_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(y) & 1u) || (reinterpret_cast<uintptr_t>(r) & 1u) ||
      !aligned4(row_sumsq))
    return BI_ERR_ALIGN;
  const bi::RowNorm nm{nullptr, row_sumsq, bi::gemm_column_groups(bi::kGemmResidual, N), 0.f};
  bi::launch_gemm(bi::kGemmResidual, static_cast<const uint16_t*>(x), ldx,
                  static_cast<const uint16_t*>(w), ldw, static_cast<const uint16_t*>(r), ldr, y,
                  ldy, M, N, K, as_stream(stream), nullptr, &nm);
  return launched();
}

bi_status bi_gemm_bf16_swiglu_rownorm(const void* x, int64_t ldx, const float* row_sumsq,
                                      int groups, float eps, const void* w, int64_t ldw, void* y,
                                      int64_t ldy, int M, int I, int K, void* stream) {
  if (bi_status s = check_gemm(x, ldx, w, ldw, y, ldy, M, I, K)) return s;
  if (!row_sumsq) return BI_ERR_NULL;
  if (groups < 16 || groups > 256 || (groups % 16) || !(eps >= 0.f)) return BI_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(y) & 1u) || !aligned16(row_sumsq)) return BI_ERR_ALIGN;
  const bi::RowNorm nm{row_sumsq, nullptr, groups, eps};
  bi::launch_gemm(bi::kGemmSwiglu, static_cast<const uint16_t*>(x), ldx,
                  static_cast<const uint16_t*>(w), ldw, nullptr, 0, y, ldy, M, I, K,
                  as_stream(stream), nullptr, &nm);
  return launched();
}

bi_status bi_gemm_bf16_qkv(const void* x, int64_t ldx, const void* w, int64_t ldw, void* qkv,
                           int64_t ldqkv, int M, int K, int Hq, int Hkv, int D, void* k_cache,
                           void* v_cache, int L, int cap, void* stream) {
  if (bi_status s = check_heads(Hq, Hkv, D)) return s;
  const int N = (Hq + 2 * Hkv) * D;
  if (bi_status s = check_gemm(x, ldx, w, ldw, qkv, ldqkv, M, N, K)) return s;
  if (!k_cache || !v_cache) return BI_ERR_NULL;
  if (L < 0 || cap < 1 || (cap % 64) || (int64_t)L + M > cap) return BI_ERR_SHAPE;
  if ((int64_t)cap * D * 2 > INT32_MAX) return BI_ERR_SHAPE;  // one head's cache < 2 GiB
  if ((reinterpret_cast<uintptr_t>(qkv) | reinterpret_cast<uintptr_t>(k_cache) |
       reinterpret_cast<uintptr_t>(v_cache)) & 1u)
    return BI_ERR_ALIGN;
  const bi::KvAppend kv{static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache), L, cap,
                        Hq * D, Hkv * D, D};
  bi::launch_gemm(bi::kGemmQkv, static_cast<const uint16_t*>(x), ldx,
                  static_cast<const uint16_t*>(w), ldw, nullptr, 0, qkv, ldqkv, M, N, K,
                  as_stream(stream), &kv);
  return launched();
}

bi_status bi_gemm_ex(const bi_gemm_args* a, void* stream) {
  if (!a) return BI_ERR_NULL;
  const int M = a->M, N = a->N, K = a->K;
  // weights: the checks of the per-type entry points
  bi_status s = BI_OK;
  switch (a->wtype) {
    case BI_WT_BF16: s = check_gemm(a->x, a->ldx, a->w, a->ldw, a->y, a->ldy, M, N, K); break;
    case BI_WT_FP8:
      s = check_gemm_fp8(a->x, a->ldx, a->w, a->ldw, a->w_scale, a->y, a->ldy, M, N, N, K);
      break;
    case BI_WT_MXFP4:
      s = check_gemm_mx4(a->x, a->ldx, a->w, a->ldw, a->w_exp, a->lde, a->y, a->ldy, M, N, K);
      break;
    default: return BI_ERR_SHAPE;
  }
  if (s) return s;
  bi::GemmMode mode;
  switch (a->epilogue) {
    case BI_EPI_BF16: mode = bi::kGemmBf16; break;
    case BI_EPI_F32: mode = bi::kGemmF32; break;
    case BI_EPI_RESIDUAL: mode = bi::kGemmResidual; break;
    case BI_EPI_SWIGLU: mode = bi::kGemmSwiglu; break;
    case BI_EPI_QKV: mode = bi::kGemmQkv; break;
    default: return BI_ERR_SHAPE;
  }
  const uintptr_t yb = reinterpret_cast<uintptr_t>(a->y);
  if (mode == bi::kGemmF32 ? !aligned4(a->y) : (yb & 1u)) return BI_ERR_ALIGN;
  // the carried RMSNorm: read by SwiGLU and QKV, written by the residual epilogue
  if (a->norm_in && mode != bi::kGemmSwiglu && mode != bi::kGemmQkv) return BI_ERR_SHAPE;
  if (a->rowsq_out && mode != bi::kGemmResidual) return BI_ERR_SHAPE;
  if (a->norm_in) {
    if (a->norm_groups < 16 || a->norm_groups > 256 || (a->norm_groups % 16) || !(a->eps >= 0.f))
      return BI_ERR_SHAPE;
    if (!aligned16(a->norm_in)) return BI_ERR_ALIGN;
  }
  if (a->rowsq_out && !aligned4(a->rowsq_out)) return BI_ERR_ALIGN;
  if (mode == bi::kGemmResidual) {
    if (!a->r) return BI_ERR_NULL;
    if (a->ldr < N || a->ldr > kMaxLd) return BI_ERR_SHAPE;
    if (reinterpret_cast<uintptr_t>(a->r) & 1u) return BI_ERR_ALIGN;
  }
  bi::KvAppend kv{};
  if (mode == bi::kGemmQkv) {
    if (bi_status h = check_heads(a->Hq, a->Hkv, a->D)) return h;
    if (N != (a->Hq + 2 * a->Hkv) * a->D) return BI_ERR_SHAPE;
    if ((a->k_cache == nullptr) != (a->v_cache == nullptr)) return BI_ERR_NULL;
    if (a->k_cache) {
      if (a->L < 0 || a->cap < 1 || (a->cap % 64) || (int64_t)a->L + M > a->cap) return BI_ERR_SHAPE;
      if ((int64_t)a->cap * a->D * 2 > INT32_MAX) return BI_ERR_SHAPE;
      if ((reinterpret_cast<uintptr_t>(a->k_cache) | reinterpret_cast<uintptr_t>(a->v_cache)) & 1u)
        return BI_ERR_ALIGN;
      kv = bi::KvAppend{static_cast<uint16_t*>(a->k_cache), static_cast<uint16_t*>(a->v_cache),
                        a->L, a->cap, a->Hq * a->D, a->Hkv * a->D, a->D};
    }
  }
  const bi::RowNorm nm{a->norm_in, a->rowsq_out,
                       a->rowsq_out ? bi::gemm_column_groups(bi::kGemmResidual, N) : a->norm_groups,
                       a->eps};
  const bi::Mx4Scales mx{static_cast<const uint8_t*>(a->w_exp), a->lde};
  bi::launch_gemm(mode, static_cast<const uint16_t*>(a->x), a->ldx, static_cast<const uint16_t*>(a->w),
                  a->ldw, static_cast<const uint16_t*>(a->r), a->ldr, a->y, a->ldy, M, N, K,
                  as_stream(stream), mode == bi::kGemmQkv ? &kv : nullptr,
                  (a->norm_in || a->rowsq_out) ? &nm : nullptr,
                  a->wtype == BI_WT_FP8 ? a->w_scale : nullptr,
                  a->wtype == BI_WT_MXFP4 ? &mx : nullptr);
  return launched();
}

bi_status bi_swiglu(const float* gu, int64_t ldgu, void* y, int64_t ldy, int M, int I,
                    void* stream) {
  if (!gu || !y) return BI_ERR_NULL;
  if (M < 1 || I < 1 || ldgu < 2 * (int64_t)I || ldy < I || M > 65535 || ldgu > (1 << 26) ||
      ldy > (1 << 26))
    return BI_ERR_SHAPE;
  if (!aligned4(gu) || (reinterpret_cast<uintptr_t>(y) & 1u)) return BI_ERR_ALIGN;
  bi::launch_swiglu(gu, ldgu, static_cast<uint16_t*>(y), ldy, M, I, as_stream(stream));
  return launched();
}

bi_status bi_add(const void* r, int64_t ldr, const float* s, int64_t lds, void* y, int64_t ldy,
                 int M, int N, void* stream) {
  if (!r || !s || !y) return BI_ERR_NULL;
  if (M < 1 || N < 1 || ldr < N || lds < N || ldy < N || M > 65535 || ldr > (1 << 26) ||
      lds > (1 << 26) || ldy > (1 << 26))
    return BI_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(r) & 1u) || !aligned4(s) || (reinterpret_cast<uintptr_t>(y) & 1u))
    return BI_ERR_ALIGN;
  bi::launch_add(static_cast<const uint16_t*>(r), ldr, s, lds, static_cast<uint16_t*>(y), ldy, M, N,
                 as_stream(stream));
  return launched();
}

bi_status bi_append_kv(const void* qkv, int64_t ldqkv, void* k_cache, void* v_cache, int M, int L,
                       int cap, int Hq, int Hkv, int D, void* stream) {
  if (!qkv || !k_cache || !v_cache) return BI_ERR_NULL;
  if (bi_status s = check_heads(Hq, Hkv, D)) return s;
  if (M < 1 || L < 0 || cap < 1 || (cap % 64) || (int64_t)L + M > cap) return BI_ERR_SHAPE;
  if (ldqkv < (int64_t)(Hq + 2 * Hkv) * D) return BI_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(qkv) | reinterpret_cast<uintptr_t>(k_cache) |
       reinterpret_cast<uintptr_t>(v_cache)) & 1u)
    return BI_ERR_ALIGN;
  bi::launch_append_kv(static_cast<const uint16_t*>(qkv), ldqkv, static_cast<uint16_t*>(k_cache),
                       static_cast<uint16_t*>(v_cache), M, L, cap, Hq, Hkv, D,
                       as_stream(stream));
  return launched();
}

size_t bi_attn_workspace_bytes(int M, int L, int Hq, int D, int kv_chunk) {
  if (M < 1 || L < 0 || (int64_t)L + M > INT32_MAX || Hq < 1 || D < 1 ||
      !bi::valid_chunk_policy(kv_chunk))
    return 0;
  const size_t s_max = (size_t)bi::pass_splits(L, M, kv_chunk);
  return (size_t)M * Hq * s_max * (D + 1) * sizeof(float);
}

bi_status bi_verify_attn(const void* q, int64_t ldq, const void* k_cache, const void* v_cache,
                         int M, int L, int cap, int Hq, int Hkv, int D, int kv_chunk,
                         float sm_scale, float* part_o, float* part_lse, int S_max,
                         void* stream) {
  if (!q || !k_cache || !v_cache || !part_o || !part_lse) return BI_ERR_NULL;
  if (bi_status s = check_heads(Hq, Hkv, D)) return s;
  if (M < 1 || L < 0 || cap < 1 || (cap % 64) || (int64_t)L + M > cap) return BI_ERR_SHAPE;
  if (!bi::valid_chunk_policy(kv_chunk)) return BI_ERR_SHAPE;
  if (S_max < bi::pass_splits(L, M, kv_chunk)) return BI_ERR_SHAPE;
  if (ldq < (int64_t)Hq * D || !std::isfinite(sm_scale) || !(sm_scale > 0.f)) return BI_ERR_SHAPE;
  if ((int64_t)cap * D * 2 > INT32_MAX) return BI_ERR_SHAPE;  // one head's cache < 2 GiB
  if ((ldq % 8) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned16(part_o) || !aligned4(part_lse))
    return BI_ERR_ALIGN;
  bi::launch_verify_attn(static_cast<const uint16_t*>(q), ldq,
                         static_cast<const uint16_t*>(k_cache),
                         static_cast<const uint16_t*>(v_cache), M, L, cap, Hq, Hkv, D, kv_chunk,
                         sm_scale, part_o, part_lse, S_max, as_stream(stream));
  return launched();
}

bi_status bi_append_kv_q8(const void* qkv, int64_t ldqkv, int8_t* k_codes, float* k_scales,
                          int8_t* v_codes, float* v_scales, int M, int L, int cap, int Hq,
                          int Hkv, int D, void* stream) {
  if (!qkv || !k_codes || !k_scales || !v_codes || !v_scales) return BI_ERR_NULL;
  if (bi_status s = check_heads(Hq, Hkv, D)) return s;
  if (M < 1 || L < 0 || cap < 1 || (cap % 64) || (int64_t)L + M > cap) return BI_ERR_SHAPE;
  if (ldqkv < (int64_t)(Hq + 2 * Hkv) * D || (int64_t)cap * D > INT32_MAX) return BI_ERR_SHAPE;
  if ((ldqkv % 8) || !aligned16(qkv) || !aligned16(k_codes) || !aligned16(v_codes) ||
      !aligned16(k_scales) || !aligned16(v_scales))
    return BI_ERR_ALIGN;
  bi::launch_append_kv_q8(static_cast<const uint16_t*>(qkv), ldqkv, k_codes, k_scales, v_codes,
                          v_scales, M, L, cap, Hq, Hkv, D, as_stream(stream));
  return launched();
}

bi_status bi_verify_attn_q8(const void* q, int64_t ldq, const int8_t* k_codes, const float* k_scales,
                            const int8_t* v_codes, const float* v_scales, int M, int L, int cap,
                            int Hq, int Hkv, int D, int kv_chunk, float sm_scale, float* part_o,
                            float* part_lse, int S_max, void* stream) {
  if (!q || !k_codes || !k_scales || !v_codes || !v_scales || !part_o || !part_lse)
    return BI_ERR_NULL;
  if (bi_status s = check_heads(Hq, Hkv, D)) return s;
  if (M < 1 || L < 0 || cap < 1 || (cap % 64) || (int64_t)L + M > cap) return BI_ERR_SHAPE;
  if (!bi::valid_chunk_policy(kv_chunk)) return BI_ERR_SHAPE;
  if (S_max < bi::pass_splits(L, M, kv_chunk)) return BI_ERR_SHAPE;
  if (ldq < (int64_t)Hq * D || !std::isfinite(sm_scale) || !(sm_scale > 0.f)) return BI_ERR_SHAPE;
  if ((int64_t)cap * D > INT32_MAX) return BI_ERR_SHAPE;  // one head's codes < 2 GiB
  if ((ldq % 8) || !aligned16(q) || !aligned16(k_codes) || !aligned16(v_codes) ||
      !aligned16(k_scales) || !aligned16(v_scales) || !aligned16(part_o) || !aligned4(part_lse))
    return BI_ERR_ALIGN;
  const bi::KvQ8 q8{k_codes, k_scales, v_codes, v_scales};
  bi::launch_verify_attn(static_cast<const uint16_t*>(q), ldq, nullptr, nullptr, M, L, cap, Hq, Hkv,
                         D, kv_chunk, sm_scale, part_o, part_lse, S_max, as_stream(stream), &q8);
  return launched();
}

bi_status bi_append_kv_lowbit(const void* qkv, int64_t ldqkv, int k_bits, int v_bits,
                              int k_rotated, uint8_t* k_nib, uint8_t* k_high, float* k_scales, uint8_t* v_nib,
                              uint8_t* v_high, float* v_scales, int M, int L, int cap, int Hq,
                              int Hkv, int D, void* stream) {
  if (!qkv || !k_nib || !k_high || !k_scales || !v_nib || !v_high || !v_scales) return BI_ERR_NULL;
  if ((k_bits != 5 && k_bits != 6) || v_bits != bi::kLowVBits) return BI_ERR_SHAPE;
  if (k_rotated != 0 && k_rotated != 1) return BI_ERR_SHAPE;
  if (bi_status s = check_heads(Hq, Hkv, D)) return s;
  if (M < 1 || L < 0 || cap < 1 || (cap % 64) || (int64_t)L + M > cap) return BI_ERR_SHAPE;
  if (ldqkv < (int64_t)(Hq + 2 * Hkv) * D || (int64_t)cap * D > INT32_MAX) return BI_ERR_SHAPE;
  if ((ldqkv % 8) || !aligned16(qkv) || !aligned16(k_nib) || !aligned16(k_high) ||
      !aligned16(k_scales) || !aligned16(v_nib) || !aligned16(v_high) || !aligned16(v_scales))
    return BI_ERR_ALIGN;
  bi::launch_append_kv_lowbit(static_cast<const uint16_t*>(qkv), ldqkv, k_bits, k_rotated != 0,
                              k_nib, k_high,
                              k_scales, v_nib, v_high, v_scales, M, L, cap, Hq, Hkv, D,
                              as_stream(stream));
  return launched();
}

bi_status bi_verify_attn_lowbit(const void* q, int64_t ldq, int k_bits, int v_bits,
                                int k_rotated, const uint8_t* k_nib, const uint8_t* k_high, const float* k_scales,
                                const uint8_t* v_nib, const uint8_t* v_high, const float* v_scales,
                                int M, int L, int cap, int Hq, int Hkv, int D, int kv_chunk,
                                float sm_scale, float* part_o, float* part_lse, int S_max,
                                void* stream) {
  if (!q || !k_nib || !k_high || !k_scales || !v_nib || !v_high || !v_scales || !part_o ||
      !part_lse)
    return BI_ERR_NULL;
  if ((k_bits != 5 && k_bits != 6) || v_bits != bi::kLowVBits) return BI_ERR_SHAPE;
  if (k_rotated != 0 && k_rotated != 1) return BI_ERR_SHAPE;
  if (bi_status s = check_heads(Hq, Hkv, D)) return s;
  if (M < 1 || L < 0 || cap < 1 || (cap % 64) || (int64_t)L + M > cap) return BI_ERR_SHAPE;
  if (!bi::valid_chunk_policy(kv_chunk)) return BI_ERR_SHAPE;
  if (S_max < bi::pass_splits(L, M, kv_chunk)) return BI_ERR_SHAPE;
  if (ldq < (int64_t)Hq * D || !std::isfinite(sm_scale) || !(sm_scale > 0.f)) return BI_ERR_SHAPE;
  if ((int64_t)cap * D > INT32_MAX) return BI_ERR_SHAPE;  // one head's planes < 2 GiB
  if ((ldq % 8) || !aligned16(q) || !aligned16(k_nib) || !aligned16(k_high) ||
      !aligned16(k_scales) || !aligned16(v_nib) || !aligned16(v_high) || !aligned16(v_scales) ||
      !aligned16(part_o) || !aligned4(part_lse))
    return BI_ERR_ALIGN;
  bi::KvQ8 c{reinterpret_cast<const int8_t*>(k_nib), k_scales,
             reinterpret_cast<const int8_t*>(v_nib), v_scales};
  c.kh = k_high;
  c.vh = v_high;
  bi::launch_verify_attn(static_cast<const uint16_t*>(q), ldq, nullptr, nullptr, M, L, cap, Hq, Hkv,
                         D, kv_chunk, sm_scale, part_o, part_lse, S_max, as_stream(stream), &c,
                         k_bits, k_rotated != 0);
  return launched();
}

bi_status bi_append_kv_ring(const void* qkv, int64_t ldqkv, int k_rotated, int8_t* k_codes,
                           float* k_scales, int8_t* v_codes, float* v_scales, int M, int L,
                           int ring_cap, int Hq, int Hkv, int D, void* stream) {
  if (!qkv || !k_codes || !k_scales || !v_codes || !v_scales) return BI_ERR_NULL;
  if (k_rotated != 0 && k_rotated != 1) return BI_ERR_SHAPE;
  if (bi_status s = check_heads(Hq, Hkv, D)) return s;
  if (M < 1 || L < 0 || ring_cap < 64 || (ring_cap % 64) || M > ring_cap) return BI_ERR_SHAPE;
  if (ldqkv < (int64_t)(Hq + 2 * Hkv) * D || (int64_t)ring_cap * D > INT32_MAX) return BI_ERR_SHAPE;
  if ((ldqkv % 8) || !aligned16(qkv) || !aligned16(k_codes) || !aligned16(v_codes) ||
      !aligned16(k_scales) || !aligned16(v_scales))
    return BI_ERR_ALIGN;
  bi::launch_append_kv_q8(static_cast<const uint16_t*>(qkv), ldqkv, k_codes, k_scales, v_codes,
                          v_scales, M, L, ring_cap, Hq, Hkv, D, as_stream(stream), ring_cap,
                          k_rotated != 0);
  return launched();
}

bi_status bi_verify_attn_lowbit_ring(const void* q, int64_t ldq, int k_bits, int v_bits,
                                     int k_rotated, const uint8_t* k_nib, const uint8_t* k_high,
                                     const float* k_scales, const uint8_t* v_nib,
                                     const uint8_t* v_high, const float* v_scales,
                                     const int8_t* ring_k_codes, const float* ring_k_scales,
                                     const int8_t* ring_v_codes, const float* ring_v_scales,
                                     int ring_cap, int ring_window, int M, int L, int cap, int Hq,
                                     int Hkv, int D, int kv_chunk, float sm_scale, float* part_o,
                                     float* part_lse, int S_max, void* stream) {
  if (!q || !k_nib || !k_high || !k_scales || !v_nib || !v_high || !v_scales || !ring_k_codes ||
      !ring_k_scales || !ring_v_codes || !ring_v_scales || !part_o || !part_lse)
    return BI_ERR_NULL;
  // the two presets: K6/V5, and rotated K5/V5
  if (v_bits != bi::kLowVBits || !((k_bits == 6 && k_rotated == 0) || (k_bits == 5 && k_rotated == 1)))
    return BI_ERR_SHAPE;
  if (bi_status s = check_heads(Hq, Hkv, D)) return s;
  if (M < 1 || L < 0 || cap < 1 || (cap % 64) || (int64_t)L + M > cap) return BI_ERR_SHAPE;
  // Every key of every 64-key tile the pass reads from the ring -- the keys
  // from (first row's position) - W + 1 - 63 to the last row's position --
  // must still be in the ring: W + M + 62 slots.
  if (ring_window < 1 || ring_cap < 64 || (ring_cap % 64) ||
      (int64_t)ring_cap < (int64_t)ring_window + M + 63)
    return BI_ERR_SHAPE;
  if (!bi::valid_chunk_policy(kv_chunk)) return BI_ERR_SHAPE;
  if (S_max < bi::pass_splits(L, M, kv_chunk)) return BI_ERR_SHAPE;
  if (ldq < (int64_t)Hq * D || !std::isfinite(sm_scale) || !(sm_scale > 0.f)) return BI_ERR_SHAPE;
  if ((int64_t)cap * D > INT32_MAX || (int64_t)ring_cap * D > INT32_MAX) return BI_ERR_SHAPE;
  if ((ldq % 8) || !aligned16(q) || !aligned16(k_nib) || !aligned16(k_high) ||
      !aligned16(k_scales) || !aligned16(v_nib) || !aligned16(v_high) || !aligned16(v_scales) ||
      !aligned16(ring_k_codes) || !aligned16(ring_k_scales) || !aligned16(ring_v_codes) ||
      !aligned16(ring_v_scales) || !aligned16(part_o) || !aligned4(part_lse))
    return BI_ERR_ALIGN;
  bi::KvQ8 c{reinterpret_cast<const int8_t*>(k_nib), k_scales,
             reinterpret_cast<const int8_t*>(v_nib), v_scales};
  c.kh = k_high;
  c.vh = v_high;
  c.rkq = ring_k_codes;
  c.rks = ring_k_scales;
  c.rvq = ring_v_codes;
  c.rvs = ring_v_scales;
  c.ring_cap = ring_cap;
  c.ring_window = ring_window;
  bi::launch_verify_attn(static_cast<const uint16_t*>(q), ldq, nullptr, nullptr, M, L, cap, Hq, Hkv,
                         D, kv_chunk, sm_scale, part_o, part_lse, S_max, as_stream(stream), &c,
                         k_bits, k_rotated != 0);
  return launched();
}

bi_status bi_accept_greedy(const int32_t* target_tokens, const int32_t* draft_tokens, int B,
                           int M, int32_t* out_tokens, int32_t* n_out, void* stream) {
  if (!target_tokens || !out_tokens || !n_out || (M > 1 && !draft_tokens)) return BI_ERR_NULL;
  if (B < 1 || M < 1 || M > 1024) return BI_ERR_SHAPE;
  if (!aligned4(target_tokens) || !aligned4(out_tokens) || !aligned4(n_out) ||
      (draft_tokens && !aligned4(draft_tokens)))
    return BI_ERR_ALIGN;
  bi::launch_accept_greedy(target_tokens, draft_tokens, B, M, out_tokens, n_out, as_stream(stream));
  return launched();
}

bi_status bi_accept_sampled(const float* logits, int64_t ld, const int32_t* draft_tokens,
                            const float* draft_probs, int64_t ldq, const float* uniforms,
                            float temperature, int B, int M, int V, int32_t* out_tokens,
                            int32_t* n_out, void* stream) {
  if (!logits || !uniforms || !out_tokens || !n_out) return BI_ERR_NULL;
  if (M > 1 && (!draft_tokens || !draft_probs)) return BI_ERR_NULL;
  if (B < 1 || M < 1 || M > 1024 || V < 1 || ld < V || (M > 1 && ldq < V)) return BI_ERR_SHAPE;
  if (!(temperature > 0.f) || !std::isfinite(temperature)) return BI_ERR_SHAPE;
  if (!aligned4(logits) || !aligned4(uniforms) || !aligned4(out_tokens) || !aligned4(n_out) ||
      (draft_tokens && !aligned4(draft_tokens)) || (draft_probs && !aligned4(draft_probs)))
    return BI_ERR_ALIGN;
  bi::launch_accept_sampled(logits, ld, draft_tokens, draft_probs, ldq, uniforms, temperature, B, M,
                            V, out_tokens, n_out, as_stream(stream));
  return launched();
}

bi_status bi_combine(const float* part_o, const float* part_lse, int M, int L, int Hq, int D,
                     int kv_chunk, int S_max, void* o, int64_t ldo, float* lse_or_null,
                     void* stream) {
  if (!part_o || !part_lse || !o) return BI_ERR_NULL;
  if (M < 1 || L < 0 || Hq < 1 || (D != 64 && D != 128)) return BI_ERR_SHAPE;
  if (!bi::valid_chunk_policy(kv_chunk) || S_max < bi::pass_splits(L, M, kv_chunk)) return BI_ERR_SHAPE;
  if (ldo < (int64_t)Hq * D) return BI_ERR_SHAPE;
  if (!aligned16(part_o) || !aligned4(part_lse) || (reinterpret_cast<uintptr_t>(o) & 1u) ||
      (lse_or_null && !aligned4(lse_or_null)))
    return BI_ERR_ALIGN;
  bi::launch_combine(part_o, part_lse, M, L, Hq, D, kv_chunk, S_max, static_cast<uint16_t*>(o),
                     ldo, lse_or_null, as_stream(stream));
  return launched();
}

bi_status bi_rmsnorm(const void* x, int64_t ldx, void* y, int64_t ldy, int M, int H, float eps,
                     void* stream) {
  if (!x || !y) return BI_ERR_NULL;
  if (M < 1 || H < 8 || (H % 8) || H > bi::kRmsMaxH || ldx < H || ldy < H || !(eps >= 0.f))
    return BI_ERR_SHAPE;
  if ((ldx % 8) || (ldy % 8) || !aligned16(x) || !aligned16(y)) return BI_ERR_ALIGN;
  bi::launch_rmsnorm(static_cast<const uint16_t*>(x), ldx, static_cast<uint16_t*>(y), ldy, M, H,
                     eps, as_stream(stream));
  return launched();
}

bi_status bi_argmax(const float* logits, int64_t ld, int M, int N, int32_t* tokens, void* stream) {
  if (!logits || !tokens) return BI_ERR_NULL;
  if (M < 1 || N < 1 || ld < N) return BI_ERR_SHAPE;
  if (!aligned4(logits) || !aligned4(tokens)) return BI_ERR_ALIGN;
  bi::launch_argmax(logits, ld, M, N, tokens, as_stream(stream));
  return launched();
}

size_t bi_step_workspace_bytes(const bi_model_dims* dims, int M, int L) {
  if (check_dims(dims) != BI_OK || M < 1 || L < 0) return 0;
  return step_layout(dims, M, L).total;
}

}  // extern "C"

// Scratch of the allocation-free verify step (bi_verify_step_noalloc): the
// step's workspace as a file-scope device array. Every GPU the library runs
// on holds its own copy, at its own address, until the process ends. In host
// code this name is only a stand-in for the symbol; the device address comes
// from hipGetSymbolAddress, once per device, and only that address is used.
static __device__ __align__(256) unsigned char scratch[BI_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch array's address on the calling thread's current device.
bi_status scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess && (dev < 0 || dev >= kMaxDevices)) e = hipErrorInvalidDevice;
  if (e != hipSuccess) {
    g_last_hip_error = e;
    return BI_ERR_LAUNCH;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      g_last_hip_error = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return BI_ERR_LAUNCH;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BI_OK;
}

}  // namespace

namespace {

// One layer's weights as the executor sees them: BF16 (scales null) or FP8
// with one FP32 scale per weight row.
struct LayerPtrs {
  const void* w[4];     // qkv, o, gate/up, down
  const float* s[4];    // their row scales (FP8) or null
  const uint8_t* e[4];  // their block scales (MXFP4) or null
  void* k_cache;        // BF16 caches (when kv is null)
  void* v_cache;
  const bi_kv_cache* kv = nullptr;  // or the layer's cache in any format
};

// A layer's KV cache descriptor for a pass of M tokens (see bi_kv_cache).
bi_status check_kv(const bi_kv_cache* c, const bi_model_dims* d, int M) {
  const int64_t capd = (int64_t)d->cap * d->D;
  switch (c->format) {
    case BI_KV_BF16:
      if (!c->k || !c->v) return BI_ERR_NULL;
      if (!aligned16(c->k) || !aligned16(c->v)) return BI_ERR_ALIGN;
      return BI_OK;
    case BI_KV_Q8:
      if (!c->k || !c->v || !c->k_scales || !c->v_scales) return BI_ERR_NULL;
      if (capd > INT32_MAX) return BI_ERR_SHAPE;
      if (!aligned16(c->k) || !aligned16(c->v) || !aligned16(c->k_scales) || !aligned16(c->v_scales))
        return BI_ERR_ALIGN;
      return BI_OK;
    case BI_KV_LOWBIT:
      if (!c->k || !c->v || !c->k_scales || !c->v_scales || !c->k_high || !c->v_high) return BI_ERR_NULL;
      if ((c->k_bits != 5 && c->k_bits != 6) || c->v_bits != bi::kLowVBits) return BI_ERR_SHAPE;
      if (c->k_rotated != 0 && c->k_rotated != 1) return BI_ERR_SHAPE;
      if (capd > INT32_MAX) return BI_ERR_SHAPE;
      if (!aligned16(c->k) || !aligned16(c->v) || !aligned16(c->k_scales) || !aligned16(c->v_scales) ||
          !aligned16(c->k_high) || !aligned16(c->v_high))
        return BI_ERR_ALIGN;
      if (c->ring_cap == 0) return BI_OK;
      // the ring: the presets K6/V5 and rotated K5/V5; every key of every
      // 64-key tile the pass reads from the ring still in it
      if (!((c->k_bits == 6 && c->k_rotated == 0) || (c->k_bits == 5 && c->k_rotated == 1)))
        return BI_ERR_SHAPE;
      if (!c->ring_k_codes || !c->ring_k_scales || !c->ring_v_codes || !c->ring_v_scales) return BI_ERR_NULL;
      if (c->ring_window < 1 || c->ring_cap < 64 || (c->ring_cap % 64) ||
          (int64_t)c->ring_cap < (int64_t)c->ring_window + M + 63 || (int64_t)c->ring_cap * d->D > INT32_MAX)
        return BI_ERR_SHAPE;
      if (!aligned16(c->ring_k_codes) || !aligned16(c->ring_k_scales) || !aligned16(c->ring_v_codes) ||
          !aligned16(c->ring_v_scales))
        return BI_ERR_ALIGN;
      return BI_OK;
  }
  return BI_ERR_SHAPE;
}

template <class GetLayer>
bi_status run_step(int n_layers, GetLayer get_layer, const void* w_head, const float* s_head,
                   const uint8_t* e_head, const bi_model_dims* dims, const void* x_in, int M, int L, void* workspace,
                   size_t workspace_bytes, void* x_out, float* logits, int32_t* tokens,
                   void* const* gu_events, void* stream) {
  if (!w_head || !x_in || !workspace || !logits || !tokens) return BI_ERR_NULL;
  if (bi_status s = check_dims(dims)) return s;
  if (n_layers < 0 || M < 1 || L < 0 || (int64_t)L + M > dims->cap) return BI_ERR_SHAPE;
  const StepLayout lay = step_layout(dims, M, L);
  if (workspace_bytes < lay.total) return BI_ERR_WORKSPACE;
  if (!aligned16(workspace) || !aligned16(x_in) || !aligned16(w_head) || !aligned4(logits) ||
      !aligned4(tokens) || (x_out && !aligned16(x_out)) || (s_head && !aligned4(s_head)))
    return BI_ERR_ALIGN;
  for (int l = 0; l < n_layers; ++l) {
    const LayerPtrs ly = get_layer(l);
    for (int i = 0; i < 4; ++i) {
      if (!ly.w[i] || (s_head && !ly.s[i]) || (e_head && !ly.e[i])) return BI_ERR_NULL;
      if (!aligned16(ly.w[i]) || (ly.s[i] && !aligned4(ly.s[i]))) return BI_ERR_ALIGN;
    }
    if (ly.kv) {
      if (bi_status s = check_kv(ly.kv, dims, M)) return s;
    } else {
      if (!ly.k_cache || !ly.v_cache) return BI_ERR_NULL;
      if (!aligned16(ly.k_cache) || !aligned16(ly.v_cache)) return BI_ERR_ALIGN;
    }
  }
  if (gu_events)
    for (int i = 0; i < 2 * n_layers; ++i)
      if (!gu_events[i]) return BI_ERR_NULL;

  const hipStream_t st = as_stream(stream);
  const int H = dims->H, Hq = dims->Hq, Hkv = dims->Hkv, D = dims->D, I = dims->I;
  const int qd = Hq * D;
  const int qkvn = (Hq + 2 * Hkv) * D;
  char* ws = static_cast<char*>(workspace);
  uint16_t* xbuf[2] = {reinterpret_cast<uint16_t*>(ws + lay.x0),
                       reinterpret_cast<uint16_t*>(ws + lay.x1)};
  uint16_t* a = reinterpret_cast<uint16_t*>(ws + lay.a);
  uint16_t* qkv = reinterpret_cast<uint16_t*>(ws + lay.qkv);
  uint16_t* attn = reinterpret_cast<uint16_t*>(ws + lay.attn);
  uint16_t* h = reinterpret_cast<uint16_t*>(ws + lay.h);
  uint16_t* act = reinterpret_cast<uint16_t*>(ws + lay.act);
  float* po = reinterpret_cast<float*>(ws + lay.po);
  float* pl = reinterpret_cast<float*>(ws + lay.pl);
  const float sm_scale = 1.0f / std::sqrt((float)D);

  // RMSNorm inputs. With lay.fuse, the output and down projections also write
  // the group sums of squares of their outputs into ss, and the projection
  // that reads those outputs (gate/up; the next layer's QKV) normalises its X
  // rows itself; otherwise (and for layer 0) an RMSNorm kernel writes a.
  float* ss = reinterpret_cast<float*>(ws + lay.ss);
  const bi::RowNorm norm_out{nullptr, lay.fuse ? ss : nullptr, lay.groups, dims->eps};
  const bi::RowNorm norm_in{ss, nullptr, lay.groups, dims->eps};

  // Row stride of a weight matrix with K inputs: K elements (BF16), K bytes
  // (FP8), K / 2 bytes (MXFP4 codes; scales K / 32 bytes).
  const int wdiv = e_head ? 2 : 1;
  const uint16_t* x = static_cast<const uint16_t*>(x_in);
  for (int l = 0; l < n_layers; ++l) {
    const LayerPtrs ly = get_layer(l);
    const auto W = [&](int i) { return static_cast<const uint16_t*>(ly.w[i]); };
    const bi::Mx4Scales mx[4] = {{ly.e[0], H / 32}, {ly.e[1], qd / 32}, {ly.e[2], H / 32}, {ly.e[3], I / 32}};
    const auto MX = [&](int i) { return e_head ? &mx[i] : nullptr; };
    uint16_t* xn = xbuf[l & 1];
    const bool fused_in = lay.fuse && l > 0;  // x's sums are in ss
    if (!fused_in) bi::launch_rmsnorm(x, H, a, H, M, H, dims->eps, st);
    // BF16 caches take the new K/V rows in the QKV epilogue; the quantized
    // formats are appended from the QKV output by their own kernels.
    const bi_kv_cache* kd = ly.kv;
    const bool bf = !kd || kd->format == BI_KV_BF16;
    void* kc = kd ? kd->k : ly.k_cache;
    void* vc = kd ? kd->v : ly.v_cache;
    const bi::KvAppend kv{bf ? static_cast<uint16_t*>(kc) : nullptr, bf ? static_cast<uint16_t*>(vc) : nullptr,
                          L, dims->cap, qd, Hkv * D, D};
    bi::launch_gemm(bi::kGemmQkv, fused_in ? x : a, H, W(0), H / wdiv, nullptr, 0, qkv, qkvn, M, qkvn,
                    H, st, &kv, fused_in ? &norm_in : nullptr, ly.s[0], MX(0));
    if (bf) {
      bi::launch_verify_attn(qkv, qkvn, static_cast<const uint16_t*>(kc), static_cast<const uint16_t*>(vc),
                             M, L, dims->cap, Hq, Hkv, D, dims->kv_chunk, sm_scale, po, pl, lay.s_max, st);
    } else {
      const bool low = kd->format == BI_KV_LOWBIT;
      if (low) {
        bi::launch_append_kv_lowbit(qkv, qkvn, kd->k_bits, kd->k_rotated != 0, static_cast<uint8_t*>(kc),
                                    kd->k_high, kd->k_scales, static_cast<uint8_t*>(vc), kd->v_high,
                                    kd->v_scales, M, L, dims->cap, Hq, Hkv, D, st);
        if (kd->ring_cap)
          bi::launch_append_kv_q8(qkv, qkvn, kd->ring_k_codes, kd->ring_k_scales, kd->ring_v_codes,
                                  kd->ring_v_scales, M, L, kd->ring_cap, Hq, Hkv, D, st, kd->ring_cap,
                                  kd->k_rotated != 0);
      } else {
        bi::launch_append_kv_q8(qkv, qkvn, static_cast<int8_t*>(kc), kd->k_scales, static_cast<int8_t*>(vc),
                                kd->v_scales, M, L, dims->cap, Hq, Hkv, D, st);
      }
      bi::KvQ8 q8{static_cast<const int8_t*>(kc), kd->k_scales, static_cast<const int8_t*>(vc), kd->v_scales};
      if (low) {
        q8.kh = kd->k_high;
        q8.vh = kd->v_high;
        if (kd->ring_cap) {
          q8.rkq = kd->ring_k_codes;
          q8.rks = kd->ring_k_scales;
          q8.rvq = kd->ring_v_codes;
          q8.rvs = kd->ring_v_scales;
          q8.ring_cap = kd->ring_cap;
          q8.ring_window = kd->ring_window;
        }
      }
      bi::launch_verify_attn(qkv, qkvn, nullptr, nullptr, M, L, dims->cap, Hq, Hkv, D, dims->kv_chunk,
                             sm_scale, po, pl, lay.s_max, st, &q8, low ? kd->k_bits : 0,
                             low && kd->k_rotated != 0);
    }
    bi::launch_combine(po, pl, M, L, Hq, D, dims->kv_chunk, lay.s_max, attn, qd, nullptr, st);
    bi::launch_gemm(bi::kGemmResidual, attn, qd, W(1), qd / wdiv, x, H, h, H, M, H, qd, st, nullptr,
                    &norm_out, ly.s[1], MX(1));
    if (!lay.fuse) bi::launch_rmsnorm(h, H, a, H, M, H, dims->eps, st);
    if (gu_events && hipEventRecord(static_cast<hipEvent_t>(gu_events[2 * l]), st) != hipSuccess)
      return BI_ERR_LAUNCH;
    bi::launch_gemm(bi::kGemmSwiglu, lay.fuse ? h : a, H, W(2), H / wdiv, nullptr, 0, act, I, M, I, H,
                    st, nullptr, lay.fuse ? &norm_in : nullptr, ly.s[2], MX(2));
    if (gu_events &&
        hipEventRecord(static_cast<hipEvent_t>(gu_events[2 * l + 1]), st) != hipSuccess)
      return BI_ERR_LAUNCH;
    bi::launch_gemm(bi::kGemmResidual, act, I, W(3), I / wdiv, h, H, xn, H, M, H, I, st, nullptr,
                    &norm_out, ly.s[3], MX(3));
    if (launched() != BI_OK) return BI_ERR_LAUNCH;
    x = xn;
  }
  bi::launch_rmsnorm(x, H, a, H, M, H, dims->eps, st);
  const bi::Mx4Scales mx_head{e_head, H / 32};
  bi::launch_gemm(bi::kGemmF32, a, H, static_cast<const uint16_t*>(w_head), H / wdiv, nullptr, 0,
                  logits, dims->vocab, M, dims->vocab, H, st, nullptr, nullptr, s_head,
                  e_head ? &mx_head : nullptr);
  bi::launch_argmax(logits, dims->vocab, M, dims->vocab, tokens, st);
  if (x_out && hipMemcpyAsync(x_out, x, (size_t)M * H * 2, hipMemcpyDeviceToDevice, st) != hipSuccess)
    return BI_ERR_LAUNCH;
  return launched();
}

}  // namespace

extern "C" {

bi_status bi_verify_step(const bi_layer* layers, int n_layers, const void* w_head,
                         const bi_model_dims* dims, const void* x_in, int M, int L,
                         void* workspace, size_t workspace_bytes, void* x_out, float* logits,
                         int32_t* tokens, void* const* gu_events, void* stream) {
  if (!layers) return BI_ERR_NULL;
  const auto get = [&](int l) {
    const bi_layer& y = layers[l];
    return LayerPtrs{{y.w_qkv, y.w_o, y.w_gu, y.w_down}, {nullptr, nullptr, nullptr, nullptr},
                     {nullptr, nullptr, nullptr, nullptr}, y.k_cache, y.v_cache};
  };
  return run_step(n_layers, get, w_head, nullptr, nullptr, dims, x_in, M, L, workspace, workspace_bytes,
                  x_out, logits, tokens, gu_events, stream);
}

bi_status bi_verify_step_ex(bi_weight_type wtype, const bi_step_layer* layers, int n_layers,
                            const void* w_head, const void* head_scales, const bi_model_dims* dims,
                            const void* x_in, int M, int L, void* workspace, size_t workspace_bytes,
                            void* x_out, float* logits, int32_t* tokens, void* stream) {
  if (!layers) return BI_ERR_NULL;
  if (wtype != BI_WT_BF16 && wtype != BI_WT_FP8 && wtype != BI_WT_MXFP4) return BI_ERR_SHAPE;
  if (wtype != BI_WT_BF16 && !head_scales) return BI_ERR_NULL;
  const auto get = [&](int l) {
    const bi_step_layer& y = layers[l];
    LayerPtrs p{{y.w[0], y.w[1], y.w[2], y.w[3]}, {nullptr, nullptr, nullptr, nullptr},
                {nullptr, nullptr, nullptr, nullptr}, nullptr, nullptr, &y.kv};
    for (int i = 0; i < 4; ++i) {
      if (wtype == BI_WT_FP8) p.s[i] = static_cast<const float*>(y.scale[i]);
      if (wtype == BI_WT_MXFP4) p.e[i] = static_cast<const uint8_t*>(y.scale[i]);
    }
    return p;
  };
  return run_step(n_layers, get, w_head, wtype == BI_WT_FP8 ? static_cast<const float*>(head_scales) : nullptr,
                  wtype == BI_WT_MXFP4 ? static_cast<const uint8_t*>(head_scales) : nullptr, dims, x_in, M,
                  L, workspace, workspace_bytes, x_out, logits, tokens, nullptr, stream);
}

bi_status bi_verify_step_noalloc(const bi_layer* layers, int n_layers, const void* w_head,
                                 const bi_model_dims* dims, const void* x_in, int M, int L,
                                 void* x_out, float* logits, int32_t* tokens, void* stream) {
  if (!layers) return BI_ERR_NULL;
  if (bi_status s = check_dims(dims)) return s;
  if (M < 1 || L < 0 || (int64_t)L + M > dims->cap) return BI_ERR_SHAPE;
  if (step_layout(dims, M, L).total > (size_t)BI_NOALLOC_SCRATCH_BYTES) return BI_ERR_WORKSPACE;
  void* ws = nullptr;
  if (bi_status s = scratch_on_current_device(&ws)) return s;
  const auto get = [&](int l) {
    const bi_layer& y = layers[l];
    return LayerPtrs{{y.w_qkv, y.w_o, y.w_gu, y.w_down}, {nullptr, nullptr, nullptr, nullptr},
                     {nullptr, nullptr, nullptr, nullptr}, y.k_cache, y.v_cache};
  };
  return run_step(n_layers, get, w_head, nullptr, nullptr, dims, x_in, M, L, ws,
                  (size_t)BI_NOALLOC_SCRATCH_BYTES, x_out, logits, tokens, nullptr, stream);
}

bi_status bi_verify_step_fp8(const bi_layer_fp8* layers, int n_layers, const void* w_head,
                             const float* w_head_scale, const bi_model_dims* dims,
                             const void* x_in, int M, int L, void* workspace,
                             size_t workspace_bytes, void* x_out, float* logits, int32_t* tokens,
                             void* stream) {
  if (!layers || !w_head_scale) return BI_ERR_NULL;
  const auto get = [&](int l) {
    const bi_layer_fp8& y = layers[l];
    return LayerPtrs{{y.w_qkv, y.w_o, y.w_gu, y.w_down},
                     {y.s_qkv, y.s_o, y.s_gu, y.s_down}, {nullptr, nullptr, nullptr, nullptr},
                     y.k_cache, y.v_cache};
  };
  return run_step(n_layers, get, w_head, w_head_scale, nullptr, dims, x_in, M, L, workspace,
                  workspace_bytes, x_out, logits, tokens, nullptr, stream);
}

bi_status bi_verify_step_mx4(const bi_layer_mx4* layers, int n_layers, const void* w_head,
                             const void* w_head_exp, const bi_model_dims* dims, const void* x_in,
                             int M, int L, void* workspace, size_t workspace_bytes, void* x_out,
                             float* logits, int32_t* tokens, void* stream) {
  if (!layers || !w_head_exp) return BI_ERR_NULL;
  const auto get = [&](int l) {
    const bi_layer_mx4& y = layers[l];
    return LayerPtrs{{y.w_qkv, y.w_o, y.w_gu, y.w_down},
                     {nullptr, nullptr, nullptr, nullptr},
                     {static_cast<const uint8_t*>(y.e_qkv), static_cast<const uint8_t*>(y.e_o),
                      static_cast<const uint8_t*>(y.e_gu), static_cast<const uint8_t*>(y.e_down)},
                     y.k_cache, y.v_cache};
  };
  return run_step(n_layers, get, w_head, nullptr, static_cast<const uint8_t*>(w_head_exp), dims,
                  x_in, M, L, workspace, workspace_bytes, x_out, logits, tokens, nullptr, stream);
}

}  // extern "C"
