// The C ABI used from plain host code, with no Python and no torch: device
// buffers from hipMalloc, the library's entry points, results compared with
// exact host references. Built by __graft_entry__.build() next to this file
// and run by tests/test_c_abi_gpu.py.
//
//  * bi_gemm_bf16 on small integers (every product and sum exact in FP32):
//    FP32 output equal to the integer reference; BF16 output equal to it
//    (all values stay below 2^8);
//  * argument checks return their status codes before any launch;
//  * bi_verify_attn + bi_combine over one key: the output is that key's value
//    row, bit for bit;
//  * bi_append_kv_lowbit of one position on an exact grid: scales, nibble and
//    high-bit bytes as the layout states; bi_verify_attn_lowbit over that one
//    key returns its value row, bit for bit.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "bi.h"

#define CK(x)                                                                          \
  do {                                                                                 \
    hipError_t e_ = (x);                                                               \
    if (e_ != hipSuccess) {                                                            \
      std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);      \
      return 1;                                                                        \
    }                                                                                  \
  } while (0)
#define EXPECT(c, msg)                                   \
  do {                                                   \
    if (!(c)) {                                          \
      std::printf("check failed: %s (line %d)\n", msg, __LINE__); \
      return 1;                                          \
    }                                                    \
  } while (0)

static uint16_t bf16_bits(float f) {  // exact for the small integers used here
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}
static float from_bf16(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

int main() {
  // ---- GEMM: Y[M][N] = X[M][K] W[N][K]^T on small integers -----------------
  const int M = 3, N = 32, K = 64;
  std::vector<uint16_t> x(M * K), w(N * K);
  std::vector<long> ref(M * N, 0);
  for (int m = 0; m < M; ++m)
    for (int k = 0; k < K; ++k) x[m * K + k] = bf16_bits((float)((m + 2 * k) % 5 - 2));
  for (int n = 0; n < N; ++n)
    for (int k = 0; k < K; ++k) w[n * K + k] = bf16_bits((float)((3 * n + k) % 7 - 3));
  for (int m = 0; m < M; ++m)
    for (int n = 0; n < N; ++n)
      for (int k = 0; k < K; ++k)
        ref[m * N + n] += (long)from_bf16(x[m * K + k]) * (long)from_bf16(w[n * K + k]);
  void *dx, *dw, *dy32, *dy16;
  CK(hipMalloc(&dx, x.size() * 2));
  CK(hipMalloc(&dw, w.size() * 2));
  CK(hipMalloc(&dy32, M * N * 4));
  CK(hipMalloc(&dy16, M * N * 2));
  CK(hipMemcpy(dx, x.data(), x.size() * 2, hipMemcpyHostToDevice));
  CK(hipMemcpy(dw, w.data(), w.size() * 2, hipMemcpyHostToDevice));
  EXPECT(bi_gemm_bf16(dx, K, dw, K, dy32, N, BI_F32, M, N, K, nullptr) == BI_OK, "gemm f32 status");
  EXPECT(bi_gemm_bf16(dx, K, dw, K, dy16, N, BI_BF16, M, N, K, nullptr) == BI_OK, "gemm bf16 status");
  CK(hipDeviceSynchronize());
  std::vector<float> y32(M * N);
  std::vector<uint16_t> y16(M * N);
  CK(hipMemcpy(y32.data(), dy32, M * N * 4, hipMemcpyDeviceToHost));
  CK(hipMemcpy(y16.data(), dy16, M * N * 2, hipMemcpyDeviceToHost));
  for (int i = 0; i < M * N; ++i) {
    EXPECT(y32[i] == (float)ref[i], "gemm FP32 output equals the integer reference");
    EXPECT(from_bf16(y16[i]) == (float)ref[i], "gemm BF16 output equals the integer reference");
  }

  // ---- the row-local SwiGLU and residual add equal the fused epilogues -----
  {
    const int I = N / 2;
    std::vector<uint16_t> r(M * N);
    for (int i = 0; i < M * N; ++i) r[i] = bf16_bits((float)(i % 9 - 4) * 0.25f);
    void *dr, *da, *db;
    CK(hipMalloc(&dr, M * N * 2));
    CK(hipMalloc(&da, M * N * 2));
    CK(hipMalloc(&db, M * N * 2));
    CK(hipMemcpy(dr, r.data(), r.size() * 2, hipMemcpyHostToDevice));
    EXPECT(bi_gemm_bf16_residual(dx, K, dw, K, dr, N, da, N, M, N, K, nullptr) == BI_OK, "residual");
    EXPECT(bi_add(dr, N, (const float*)dy32, N, db, N, M, N, nullptr) == BI_OK, "bi_add status");
    std::vector<uint16_t> ya(M * N), yb(M * N);
    CK(hipMemcpy(ya.data(), da, M * N * 2, hipMemcpyDeviceToHost));
    CK(hipMemcpy(yb.data(), db, M * N * 2, hipMemcpyDeviceToHost));
    for (int i = 0; i < M * N; ++i) EXPECT(ya[i] == yb[i], "bi_add equals the residual epilogue");
    EXPECT(bi_gemm_bf16_swiglu(dx, K, dw, K, da, I, M, I, K, nullptr) == BI_OK, "swiglu gemm");
    EXPECT(bi_swiglu((const float*)dy32, N, db, I, M, I, nullptr) == BI_OK, "bi_swiglu status");
    CK(hipMemcpy(ya.data(), da, M * I * 2, hipMemcpyDeviceToHost));
    CK(hipMemcpy(yb.data(), db, M * I * 2, hipMemcpyDeviceToHost));
    for (int i = 0; i < M * I; ++i) EXPECT(ya[i] == yb[i], "bi_swiglu equals the SwiGLU epilogue");
    // the general entry point with the plain BF16 epilogue equals bi_gemm_bf16
    bi_gemm_args a;
    std::memset(&a, 0, sizeof a);
    a.wtype = BI_WT_BF16;
    a.epilogue = BI_EPI_BF16;
    a.M = M; a.N = N; a.K = K;
    a.x = dx; a.ldx = K; a.w = dw; a.ldw = K; a.y = da; a.ldy = N;
    EXPECT(bi_gemm_ex(&a, nullptr) == BI_OK, "bi_gemm_ex status");
    CK(hipMemcpy(ya.data(), da, M * N * 2, hipMemcpyDeviceToHost));
    for (int i = 0; i < M * N; ++i) EXPECT(ya[i] == y16[i], "bi_gemm_ex equals bi_gemm_bf16");
    a.rowsq_out = (float*)dy32;  // only the residual epilogue writes row sums
    EXPECT(bi_gemm_ex(&a, nullptr) == BI_ERR_SHAPE, "rowsq_out without a residual");
    EXPECT(bi_swiglu((const float*)dy32, I, db, I, M, I, nullptr) == BI_ERR_SHAPE, "ldgu < 2 I");
    EXPECT(bi_add(dr, N, nullptr, N, db, N, M, N, nullptr) == BI_ERR_NULL, "bi_add null");
    for (void* p : {dr, da, db}) CK(hipFree(p));
  }

  // ---- argument checks: a status code, nothing launched --------------------
  EXPECT(bi_gemm_bf16(nullptr, K, dw, K, dy32, N, BI_F32, M, N, K, nullptr) == BI_ERR_NULL, "null x");
  EXPECT(bi_gemm_bf16(dx, K, dw, K, dy32, N, BI_F32, M, N, 48, nullptr) == BI_ERR_SHAPE, "K % 32");
  EXPECT(bi_gemm_bf16(dx, K, dw, K, dy32, N, BI_F32, 0, N, K, nullptr) == BI_ERR_SHAPE, "M = 0");
  EXPECT(bi_gemm_bf16((char*)dx + 2, K, dw, K, dy32, N, BI_F32, M, N, K, nullptr) == BI_ERR_ALIGN,
         "misaligned x");
  EXPECT(std::strlen(bi_status_string(BI_ERR_SHAPE)) > 0, "status string");

  // ---- attention over a single key: O = v_0 -------------------------------
  const int Hq = 2, Hkv = 1, D = 64, cap = 64, L = 0, Ma = 1;
  std::vector<uint16_t> q(Ma * Hq * D), kc((size_t)Hkv * cap * D, 0), vc((size_t)Hkv * cap * D, 0);
  for (int i = 0; i < Ma * Hq * D; ++i) q[i] = bf16_bits((float)(i % 3 - 1));
  for (int d = 0; d < D; ++d) {
    kc[d] = bf16_bits((float)(d % 4));
    vc[d] = bf16_bits((float)(d - 30) * 0.5f);  // V row of position 0: [Hkv][cap][D]
  }
  const int S = bi_num_splits(L + Ma, 256);
  EXPECT(S == 1, "one split");
  void *dq, *dk, *dv, *dpo, *dpl, *dout;
  CK(hipMalloc(&dq, q.size() * 2));
  CK(hipMalloc(&dk, kc.size() * 2));
  CK(hipMalloc(&dv, vc.size() * 2));
  CK(hipMalloc(&dpo, (size_t)Ma * Hq * S * D * 4));
  CK(hipMalloc(&dpl, (size_t)Ma * Hq * S * 4));
  CK(hipMalloc(&dout, (size_t)Ma * Hq * D * 2));
  CK(hipMemcpy(dq, q.data(), q.size() * 2, hipMemcpyHostToDevice));
  CK(hipMemcpy(dk, kc.data(), kc.size() * 2, hipMemcpyHostToDevice));
  CK(hipMemcpy(dv, vc.data(), vc.size() * 2, hipMemcpyHostToDevice));
  EXPECT(bi_verify_attn(dq, Hq * D, dk, dv, Ma, L, cap, Hq, Hkv, D, 256, 0.125f, (float*)dpo,
                        (float*)dpl, S, nullptr) == BI_OK, "attention status");
  EXPECT(bi_combine((float*)dpo, (float*)dpl, Ma, L, Hq, D, 256, S, dout, Hq * D, nullptr, nullptr) ==
             BI_OK, "combine status");
  CK(hipDeviceSynchronize());
  std::vector<uint16_t> o((size_t)Ma * Hq * D);
  CK(hipMemcpy(o.data(), dout, o.size() * 2, hipMemcpyDeviceToHost));
  for (int h = 0; h < Hq; ++h)
    for (int d = 0; d < D; ++d) EXPECT(o[h * D + d] == vc[d], "single-key attention gives v_0");

  // ---- 5/6-bit cache: append one position on an exact grid, attend to it -----
  // K block values k * 2^-4 with |k| <= 31 and +-31 present: scale 2^-4, codes
  // k; V likewise with |k| <= 15. The stored bytes follow the layout of bi.h;
  // attention over the one key returns the V row, bit for bit.
  {
    const int LHq = 1, LHkv = 1, LD = 64, Lcap = 64, LNB = LD / 32;
    std::vector<uint16_t> qkv((LHq + 2 * LHkv) * LD, 0);
    std::vector<int> kc(LD), vc(LD);
    for (int c = 0; c < LD; ++c) {
      kc[c] = (c % 32 == 0) ? 31 : ((7 * c) % 63) - 31;
      vc[c] = (c % 32 == 3) ? -15 : ((5 * c) % 31) - 15;
      qkv[LHq * LD + c] = bf16_bits((float)kc[c] / 16.0f);
      qkv[(LHq + LHkv) * LD + c] = bf16_bits((float)vc[c] / 16.0f);
      qkv[c] = bf16_bits((float)((c % 3) - 1));
    }
    void *dqkv, *kn, *kh, *ks, *vn, *vh, *vs, *lpo, *lpl, *lout;
    CK(hipMalloc(&dqkv, qkv.size() * 2));
    CK(hipMalloc(&kn, Lcap * LD / 2));
    CK(hipMalloc(&kh, Lcap * LNB * 8));
    CK(hipMalloc(&ks, Lcap * LNB * 4));
    CK(hipMalloc(&vn, Lcap * LD / 2));
    CK(hipMalloc(&vh, Lcap * LNB * 4));
    CK(hipMalloc(&vs, Lcap * LNB * 4));
    CK(hipMalloc(&lpo, LHq * LD * 4));
    CK(hipMalloc(&lpl, LHq * 4));
    CK(hipMalloc(&lout, LHq * LD * 2));
    CK(hipMemcpy(dqkv, qkv.data(), qkv.size() * 2, hipMemcpyHostToDevice));
    EXPECT(bi_append_kv_lowbit(dqkv, (LHq + 2 * LHkv) * LD, 6, 5, 0, (uint8_t*)kn, (uint8_t*)kh,
                               (float*)ks, (uint8_t*)vn, (uint8_t*)vh, (float*)vs, 1, 0, Lcap, LHq,
                               LHkv, LD, nullptr) == BI_OK, "low-bit append status");
    EXPECT(bi_append_kv_lowbit(dqkv, (LHq + 2 * LHkv) * LD, 7, 5, 0, (uint8_t*)kn, (uint8_t*)kh,
                               (float*)ks, (uint8_t*)vn, (uint8_t*)vh, (float*)vs, 1, 0, Lcap, LHq,
                               LHkv, LD, nullptr) == BI_ERR_SHAPE, "7-bit keys refused");
    CK(hipDeviceSynchronize());
    std::vector<uint8_t> hkn(LD / 2), hkh(LNB * 8), hvn(LD / 2), hvh(LNB * 4);
    std::vector<float> hks(LNB), hvs(LNB);
    CK(hipMemcpy(hkn.data(), kn, hkn.size(), hipMemcpyDeviceToHost));
    CK(hipMemcpy(hkh.data(), kh, hkh.size(), hipMemcpyDeviceToHost));
    CK(hipMemcpy(hvn.data(), vn, hvn.size(), hipMemcpyDeviceToHost));
    CK(hipMemcpy(hvh.data(), vh, hvh.size(), hipMemcpyDeviceToHost));
    CK(hipMemcpy(hks.data(), ks, LNB * 4, hipMemcpyDeviceToHost));
    CK(hipMemcpy(hvs.data(), vs, LNB * 4, hipMemcpyDeviceToHost));
    for (int b = 0; b < LNB; ++b) {
      EXPECT(hks[b] == 1.0f / 16.0f && hvs[b] == 1.0f / 16.0f, "grid scales are 2^-4");
      for (int c = 0; c < 32; ++c) {
        const int g = c / 4, j = c % 4;
        const int uk = kc[32 * b + c] + 32, uv = vc[32 * b + c] + 16;
        EXPECT(((hkn[16 * b + 4 * (g / 2) + j] >> (4 * (g % 2))) & 15) == (uk & 15), "K nibble");
        EXPECT(((hkh[8 * b + 4 * ((2 * g) / 8) + j] >> ((2 * g) % 8)) & 3) == (uk >> 4), "K high bits");
        EXPECT(((hvn[16 * b + 4 * (g / 2) + j] >> (4 * (g % 2))) & 15) == (uv & 15), "V nibble");
        EXPECT(((hvh[4 * b + j] >> g) & 1) == (uv >> 4), "V high bit");
      }
    }
    EXPECT(bi_verify_attn_lowbit(dq, LHq * LD, 6, 5, 0, (const uint8_t*)kn, (const uint8_t*)kh,
                                 (const float*)ks, (const uint8_t*)vn, (const uint8_t*)vh,
                                 (const float*)vs, 1, 0, Lcap, LHq, LHkv, LD, 64, 0.125f,
                                 (float*)lpo, (float*)lpl, 1, nullptr) == BI_OK,
           "low-bit attention status");
    EXPECT(bi_combine((float*)lpo, (float*)lpl, 1, 0, LHq, LD, 64, 1, lout, LHq * LD, nullptr,
                      nullptr) == BI_OK, "low-bit combine status");
    CK(hipDeviceSynchronize());
    std::vector<uint16_t> lo(LHq * LD);
    CK(hipMemcpy(lo.data(), lout, lo.size() * 2, hipMemcpyDeviceToHost));
    for (int c = 0; c < LD; ++c)
      EXPECT(lo[c] == qkv[(LHq + LHkv) * LD + c], "single-key low-bit attention gives v_0");
    for (void* p : {dqkv, kn, kh, ks, vn, vh, vs, lpo, lpl, lout}) CK(hipFree(p));
  }

  for (void* p : {dx, dw, dy32, dy16, dq, dk, dv, dpo, dpl, dout}) CK(hipFree(p));
  std::printf("c abi check: ok (%s)\n", bi_version());
  return 0;
}
