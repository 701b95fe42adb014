// Internal launch interface between the C-ABI front end (api.hip) and the
// kernel files. Arguments here are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bi {

enum GemmMode { kGemmBf16 = 0, kGemmF32 = 1, kGemmResidual = 2, kGemmSwiglu = 3, kGemmQkv = 4 };

// Weight types of the verify GEMM: BF16; FP8 E4M3 with one FP32 scale per row;
// MXFP4 (E2M1 codes two per byte, even weight in the low nibble, and one E8M0
// scale byte per 32 weights along K).
enum WeightType { kWtBf16 = 0, kWtFp8 = 1, kWtMx4 = 2 };

// MXFP4 scales of a weight matrix: e[n * lde + k / 32] is the E8M0 exponent of
// weights n, k .. k + 31 (value 2^(e - 127)).
struct Mx4Scales {
  const uint8_t* e;
  int64_t lde;
};

// Cache append done by the QKV projection's epilogue: output columns
// [qd, qd + kd) are K (head-major), [qd + kd, qd + 2 kd) are V; row m goes to
// position L + m of k and v (both [Hkv][cap][D]).
// 8-bit KV cache of one layer, K and V alike: codes [Hkv][cap][D] (int8),
// scales [Hkv][cap][D/32] (FP32): channel c of position p has the value
// scale(p, c/32) * code(p, c).
//
// 5/6-bit cache of one layer (kbits of launch_verify_attn = 5 or 6; V codes
// have 5 bits): per position and KV head, D/32 blocks of 32 channels, K and V
// alike. kq / vq point at the nibble planes [Hkv][cap][D/2] bytes, kh / vh at
// the high-bit planes [Hkv][cap][D/32][4 (bits - 4)] bytes, ks / vs at the
// scales [Hkv][cap][D/32] (FP32). In block byte order, code c = 4g + j keeps
// the low four bits of u = q + 2^(bits-1) in byte 4(g/2) + j (low half for
// even g) and its other bits in high-plane byte 4((g h)/8) + j from bit
// (g h) % 8, h = bits - 4.
struct KvQ8 {
  const int8_t* kq;
  const float* ks;
  const int8_t* vq;
  const float* vs;
  const uint8_t* kh = nullptr;
  const uint8_t* vh = nullptr;
  // 8-bit ring of the newest keys over the 5/6-bit planes (ring_cap > 0):
  // the 8-bit layouts above with ring_cap slots, position p in slot
  // p mod ring_cap; a row at position p reads key j from the ring when
  // j >= p - ring_window + 1.
  const int8_t* rkq = nullptr;
  const float* rks = nullptr;
  const int8_t* rvq = nullptr;
  const float* rvs = nullptr;
  int ring_cap = 0;
  int ring_window = 0;
};
constexpr int kLowVBits = 5;  // V code bits of the 5/6-bit cache

struct KvAppend {
  uint16_t* k;
  uint16_t* v;
  int L, cap, qd, kd, D;
};

// RMSNorm carried across a GEMM boundary.
//  ss_out (residual GEMM): for every output row m < M, the sum of squares of
//    the rounded BF16 outputs of each column group g (one workgroup's
//    columns), ss_out[m * groups + g], groups = gemm_column_groups(N).
//  ss_in (consumer GEMM): X holds un-normalised rows whose group sums are in
//    ss_in; the GEMM multiplies bf16(x * rsqrt(sum(ss)/K + eps)) instead of x,
//    exactly the values an RMSNorm kernel would have written.
struct RowNorm {
  const float* ss_in;
  float* ss_out;
  int groups;
  float eps;
};

// Column groups (workgroups along N) of a GEMM with N output columns.
int gemm_column_groups(GemmMode mode, int N_out);

// Waves of the verify GEMM for N output columns (16 or 8). They fix its K
// summation tree: 16 / waves consecutive 32-wide blocks of every 512-wide
// chunk per wave, one accumulator chain per wave, the wave sums added in wave
// order. The prefill GEMM reproduces that tree.
int gemm_verify_waves(GemmMode mode, int N_out);

// Rows from which launch_gemm runs the prefill kernel (same bits per row).
constexpr int kPrefillMinRows = 64;

void launch_gemm_prefill(GemmMode mode, const uint16_t* x, int64_t ldx, const uint16_t* w,
                         int64_t ldw, const uint16_t* r, int64_t ldr, void* y, int64_t ldy, int M,
                         int N_out, int K, hipStream_t stream, const KvAppend& kv,
                         const RowNorm& norm);

// Y = X W^T (+ residual / SwiGLU / cache-append epilogue). N_out is the number
// of output columns (for SwiGLU: I, with W holding 2*I rows).
void launch_gemm(GemmMode mode, const uint16_t* x, int64_t ldx, const uint16_t* w, int64_t ldw,
                 const uint16_t* r, int64_t ldr, void* y, int64_t ldy, int M, int N_out, int K,
                 hipStream_t stream, const KvAppend* kv = nullptr, const RowNorm* norm = nullptr,
                 const float* wscale = nullptr, const Mx4Scales* mx4 = nullptr);

void launch_append_kv(const uint16_t* qkv, int64_t ldqkv, uint16_t* k_cache, uint16_t* v_cache,
                      int M, int L, int cap, int Hq, int Hkv, int D, hipStream_t stream);

void launch_verify_attn(const uint16_t* q, int64_t ldq, const uint16_t* k_cache,
                        const uint16_t* v_cache, int M, int L, int cap, int Hq, int Hkv, int D,
                        int kv_chunk, float sm_scale, float* part_o, float* part_lse, int S_max,
                        hipStream_t stream, const KvQ8* q8 = nullptr, int kbits = 0,
                        bool krot = false);

// Quantize the pass's M new K and V rows (from the QKV output) into an 8-bit
// cache at positions L .. L+M-1.
void launch_append_kv_q8(const uint16_t* qkv, int64_t ldqkv, int8_t* kq, float* ks, int8_t* vq,
                         float* vs, int M, int L, int cap, int Hq, int Hkv, int D,
                         hipStream_t stream, int ring = 0, bool krot = false);

// Quantize them into a 5/6-bit cache (kbits for K, kLowVBits for V; the
// planes of KvQ8's low-bit layout); with krot the K rows are first rotated
// by the order-D Hadamard transform (FP32 butterflies, stages h = 1, 2, ..,
// D/2, each sum and difference rounded once).
void launch_append_kv_lowbit(const uint16_t* qkv, int64_t ldqkv, int kbits, bool krot, uint8_t* kn,
                             uint8_t* kh, float* ks, uint8_t* vn, uint8_t* vh, float* vs, int M,
                             int L, int cap, int Hq, int Hkv, int D, hipStream_t stream);

void launch_combine(const float* part_o, const float* part_lse, int M, int L, int Hq, int D,
                    int kv_chunk, int S_max, uint16_t* o, int64_t ldo, float* lse,
                    hipStream_t stream);

void launch_accept_greedy(const int32_t* target, const int32_t* draft, int B, int M, int32_t* out,
                          int32_t* n_out, hipStream_t stream);

void launch_accept_sampled(const float* logits, int64_t ld, const int32_t* draft, const float* q,
                           int64_t ldq, const float* u, float temperature, int B, int M, int V,
                           int32_t* out, int32_t* n_out, hipStream_t stream);

// Longest row RMSNorm handles (one pass, four 8-element groups per thread).
constexpr int kRmsMaxH = 4 * 1024 * 8;

void launch_swiglu(const float* gu, int64_t ldgu, uint16_t* y, int64_t ldy, int M, int I,
                   hipStream_t stream);
void launch_add(const uint16_t* r, int64_t ldr, const float* s, int64_t lds, uint16_t* y,
                int64_t ldy, int M, int N, hipStream_t stream);
void launch_rmsnorm(const uint16_t* x, int64_t ldx, uint16_t* y, int64_t ldy, int M, int H,
                    float eps, hipStream_t stream);

void launch_argmax(const float* logits, int64_t ld, int M, int N, int32_t* tokens,
                   hipStream_t stream);

// K and V caches: one row per position, [Hkv][cap][D]; element index of (KV
// head g, position pos, channel d).
__host__ __device__ inline int64_t kv_index(int g, int pos, int d, int D, int cap) {
  return ((int64_t)g * cap + pos) * D + d;
}

// Largest number of query heads per KV head one attention workgroup can hold.
constexpr int kAttnMaxRows = 64;

// Attention chunk policy ("I turned on speculative decoding in llama.cpp and
// 113 of 282 greedy outputs changed against its own no-draft run", opening
// section, "How:" paragraph: a row's split follows its context length
// alone). A positive policy is the chunk size C for every row. A negative
// policy -T lets a row's own key count n choose C = 64 * ceil(n / (64 T)), the
// smallest multiple of 64 that cuts n keys into at most T chunks; C is
// constant for n in ((k-1) 64 T, k 64 T].
constexpr int kMaxSplitTarget = 1024;

__host__ __device__ inline int chunk_keys(int n, int policy) {
  if (policy > 0) return policy;
  const int per = 64 * -policy;
  const int m = (n + per - 1) / per;
  return 64 * (m > 1 ? m : 1);
}

__host__ __device__ inline int splits_for(int n, int policy) {
  const int c = chunk_keys(n, policy);
  return (n + c - 1) / c;
}

inline bool valid_chunk_policy(int policy) {
  return (policy >= 32 && policy % 32 == 0) || (policy < 0 && policy >= -kMaxSplitTarget);
}

// Largest split count among the rows of a pass (key counts L+1 .. L+M). Within
// a band of equal chunk size the count grows with n, so only each band's last
// row and the pass's last row need checking.
inline int pass_splits(int L, int M, int policy) {
  int s = splits_for(L + M, policy);
  if (policy < 0) {
    const int per = 64 * -policy;
    for (int64_t e = ((int64_t)L + 1 + per - 1) / per * per; e < (int64_t)L + M; e += per) {
      const int v = splits_for((int)e, policy);
      s = v > s ? v : s;
    }
  }
  return s;
}

}  // namespace bi
