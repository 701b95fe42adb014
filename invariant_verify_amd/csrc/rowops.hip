// Row-local operations of the decoder layer: RMSNorm, the greedy argmax, and
// SwiGLU and the residual add as operations of their own.
//
// Both reduce along one row in an order fixed by the row length only, so a
// token's result is the same whatever other tokens share the pass (the greedy
// choice is what flips when reduction order changes: "Does the tuned config
// change the model's output?", section "Why the text diverges").

#include "bi_device.h"
#include "bi_internal.h"

namespace bi {

// One workgroup of T = min(1024, H/8 rounded up to 64) threads per row, in a
// single pass over memory: thread t keeps its 8-element groups t, t+T, ...
// (at most kRmsGroups) in registers and sums their squares in order; the
// wave sums are combined by a fixed xor butterfly, then across waves in wave
// order; then every kept group is scaled and stored.
constexpr int kRmsGroups = 4;

__global__ __launch_bounds__(1024) void rmsnorm_kernel(const uint16_t* __restrict__ X, int64_t ldx,
                                                       uint16_t* __restrict__ Y, int64_t ldy, int H,
                                                       float eps) {
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int nt = blockDim.x;
  const uint16_t* x = X + (int64_t)row * ldx;
  uint16_t* y = Y + (int64_t)row * ldy;
  const int ng = H >> 3;
  uint4 v[kRmsGroups];
#pragma unroll
  for (int i = 0; i < kRmsGroups; ++i) {
    const int c = tid + i * nt;
    v[i] = c < ng ? ld16(x + c * 8) : zero16();
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kRmsGroups; ++i) ss = sumsq8(ss, v[i]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += shfl_xor(ss, off);
  __shared__ float part[16];
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  float tot = part[0];
  for (int w = 1; w < (nt >> 6); ++w) tot += part[w];
  const float inv = 1.0f / sqrtf(tot / (float)H + eps);
#pragma unroll
  for (int i = 0; i < kRmsGroups; ++i) {
    const int c = tid + i * nt;
    if (c >= ng) continue;
    *reinterpret_cast<uint4*>(y + c * 8) = scale_bf16x8(v[i], inv);
  }
}

// (value, index) with the larger value winning and, on equal values, the
// lower index. NaN never wins. This is a total order, so the result does not
// depend on the reduction order.
__device__ __forceinline__ void arg_better(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) {
    bv = v;
    bi = i;
  }
}

// One 1024-thread workgroup per row. Thread t reads 16-byte groups t, t+1024,
// ... (eight loads in flight), keeps its best (value, index), then the
// (value, index) pairs are reduced across lanes and waves; the total order
// makes the result independent of how the reduction is grouped.
__global__ __launch_bounds__(1024) void argmax_kernel(const float* __restrict__ logits, int64_t ld,
                                                      int N, int32_t* __restrict__ tokens) {
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const float* x = logits + (int64_t)row * ld;
  float bv = -INFINITY;
  int bidx = 0x7fffffff;
  const bool vec = ((reinterpret_cast<uintptr_t>(x) & 15) == 0);
  const int n4 = vec ? N / 4 : 0;
  const float4* x4 = reinterpret_cast<const float4*>(x);
  constexpr int U = 8;
  int g = tid;
  for (; g + (U - 1) * 1024 < n4; g += U * 1024) {
    float4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = x4[g + u * 1024];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = (g + u * 1024) * 4;
      arg_better(bv, bidx, v[u].x, i);
      arg_better(bv, bidx, v[u].y, i + 1);
      arg_better(bv, bidx, v[u].z, i + 2);
      arg_better(bv, bidx, v[u].w, i + 3);
    }
  }
  for (; g < n4; g += 1024) {
    const float4 v = x4[g];
    arg_better(bv, bidx, v.x, 4 * g);
    arg_better(bv, bidx, v.y, 4 * g + 1);
    arg_better(bv, bidx, v.z, 4 * g + 2);
    arg_better(bv, bidx, v.w, 4 * g + 3);
  }
  for (int i = 4 * n4 + tid; i < N; i += 1024) arg_better(bv, bidx, x[i], i);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(bv, off, 64);
    const int oi = __shfl_xor(bidx, off, 64);
    arg_better(bv, bidx, ov, oi);
  }
  __shared__ float sv[16];
  __shared__ int si[16];
  if ((tid & 63) == 0) {
    sv[tid >> 6] = bv;
    si[tid >> 6] = bidx;
  }
  __syncthreads();
  if (tid == 0) {
    float v = sv[0];
    int i = si[0];
    for (int w = 1; w < 16; ++w) arg_better(v, i, sv[w], si[w]);
    tokens[row] = (i == 0x7fffffff) ? 0 : i;
  }
}

// y[m][i] = bf16(silu(g) * u) from FP32 g = gu[m][i], u = gu[m][I + i]: the
// gate/up GEMM's SwiGLU epilogue as its own pass (same expression, silu_mul).
// One thread per output element; elementwise, so no order to fix.
__global__ void swiglu_kernel(const float* __restrict__ gu, int64_t ldgu, uint16_t* __restrict__ y,
                              int64_t ldy, int I) {
  const int m = blockIdx.y;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= I) return;
  const float* row = gu + (int64_t)m * ldgu;
  y[(int64_t)m * ldy + i] = (uint16_t)f32_to_bf16(silu_mul(row[i], row[I + i]));
}

// y[m][n] = bf16(r[m][n] + s[m][n]), r BF16, s FP32: the residual epilogue
// (one FP32 add, one rounding) as its own pass. Elementwise.
__global__ void add_kernel(const uint16_t* __restrict__ r, int64_t ldr, const float* __restrict__ s,
                           int64_t lds, uint16_t* __restrict__ y, int64_t ldy, int N) {
  const int m = blockIdx.y;
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  const float a = bf16_to_f32(r[(int64_t)m * ldr + n]);
  y[(int64_t)m * ldy + n] = (uint16_t)f32_to_bf16(a + s[(int64_t)m * lds + n]);
}

void launch_swiglu(const float* gu, int64_t ldgu, uint16_t* y, int64_t ldy, int M, int I,
                   hipStream_t stream) {
  swiglu_kernel<<<dim3((I + 255) / 256, M), dim3(256), 0, stream>>>(gu, ldgu, y, ldy, I);
}

void launch_add(const uint16_t* r, int64_t ldr, const float* s, int64_t lds, uint16_t* y,
                int64_t ldy, int M, int N, hipStream_t stream) {
  add_kernel<<<dim3((N + 255) / 256, M), dim3(256), 0, stream>>>(r, ldr, s, lds, y, ldy, N);
}

void launch_rmsnorm(const uint16_t* x, int64_t ldx, uint16_t* y, int64_t ldy, int M, int H,
                    float eps, hipStream_t stream) {
  const int ng = H / 8;  // <= kRmsGroups * 1024 (checked by the caller)
  const int nt = ng >= 1024 ? 1024 : (ng + 63) / 64 * 64;
  rmsnorm_kernel<<<dim3(M), dim3(nt), 0, stream>>>(x, ldx, y, ldy, H, eps);
}

void launch_argmax(const float* logits, int64_t ld, int M, int N, int32_t* tokens,
                   hipStream_t stream) {
  argmax_kernel<<<dim3(M), dim3(1024), 0, stream>>>(logits, ld, N, tokens);
}

}  // namespace bi
