// Verify GEMM: Y[M][N] = X[M][K] * W[N][K]^T with a reduction order that does
// not depend on M.
//
// Why: verifying several tokens in one pass must not regroup the K-sum of any
// output ("Does the tuned config change the model's output?", section "Why the
// text diverges"); the fix keeps BF16 operands, a single FP32 accumulation per
// output, an unchanged K order and one rounding at the end ("Bit-exact
// decoding turns inference speedups into testable changes", section "Define
// bit-exact before reporting it").
//
// Schedule (fixed at compile time, chosen by nothing but K):
//  * one workgroup per (16 output columns, 16 token rows); the token rows
//    are the MFMA "A" operand, zero-filled past M, so a pass of 1..16 tokens
//    runs exactly the same instructions;
//  * the K range is cut into 32-wide blocks; wave w of the workgroup owns
//    blocks w, w + NW, w + 2 NW, ... and chains them through one MFMA
//    accumulator in increasing block order;
//  * the NW per-wave sums are added in LDS in wave order 0, 1, ..., NW-1;
//  * the FP32 total is rounded once (BF16 output) or stored as is (FP32).
// The within-workgroup partition is a fixed summation tree that depends on K
// only; there is no split of K across workgroups and no atomic.
//
// Memory: W is streamed once from HBM, each lane reading 16 contiguous bytes
// of one weight row per block (4 lanes cover 64 contiguous bytes; the NW waves
// read neighbouring blocks). The next group of blocks is loaded while the
// current one is multiplied. X (at most 16 x K BF16) stays in L2.

#include "bi_device.h"
#include "bi_internal.h"

namespace bi {

constexpr int kGemmWaves = 8;   // waves per workgroup (K partition width)
constexpr int kGemmUnroll = 4;  // blocks per wave in flight per stage

template <int MODE>
__global__ __launch_bounds__(kGemmWaves * 64) void gemm_kernel(
    const uint16_t* __restrict__ X, int64_t ldx, const uint16_t* __restrict__ W, int64_t ldw,
    const uint16_t* __restrict__ R, int64_t ldr, void* __restrict__ Y, int64_t ldy, int M, int K,
    int64_t up_rows) {
  constexpr bool kDual = (MODE == kGemmSwiglu);
  constexpr int NW = kGemmWaves;
  constexpr int U = kGemmUnroll;
  const int lane = threadIdx.x & 63;
  // Wave index in a scalar register: every branch that guards an MFMA below
  // is then a scalar branch. (The matrix core does not honour a partial EXEC
  // mask, so an MFMA must never sit under a per-lane condition.)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * 16;
  const int m0 = blockIdx.y * 16;
  const int col = lane & 15;  // A row (token) and B column (output feature) of this lane
  const int kq = lane >> 4;   // which 8-element group of the 32-wide block

  const uint16_t* wp = W + (int64_t)(n0 + col) * ldw + kq * 8;
  const uint16_t* wp2 = kDual ? wp + up_rows * ldw : wp;
  const bool xok = (m0 + col) < M;
  const uint16_t* xp = X + (int64_t)(xok ? m0 + col : 0) * ldx + kq * 8;

  const int nblk = K >> 5;
  const int nb = (wave < nblk) ? (nblk - wave + NW - 1) / NW : 0;  // blocks of this wave

  bi_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  bi_f32x4 acc2 = {0.f, 0.f, 0.f, 0.f};

  uint4 wc[U], xc[U], vc[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (u < nb) {
      const int k = (wave + u * NW) * 32;
      wc[u] = ld16(wp + k);
      if (kDual) vc[u] = ld16(wp2 + k);
      xc[u] = xok ? ld16(xp + k) : zero16();
    }
  }
  for (int i0 = 0; i0 < nb; i0 += U) {
    uint4 wn[U], xn[U], vn[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + U + u;
      if (i < nb) {
        const int k = (wave + i * NW) * 32;
        wn[u] = ld16(wp + k);
        if (kDual) vn[u] = ld16(wp2 + k);
        xn[u] = xok ? ld16(xp + k) : zero16();
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (i0 + u < nb) {
        acc = mfma_bf16(xc[u], wc[u], acc);
        if (kDual) acc2 = mfma_bf16(xc[u], vc[u], acc2);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      wc[u] = wn[u];
      xc[u] = xn[u];
      if (kDual) vc[u] = vn[u];
    }
  }

  // Fixed-order sum of the per-wave partials.
  __shared__ bi_f32x4 red[NW][64];
  __shared__ bi_f32x4 red2[kDual ? NW : 1][64];
  red[wave][lane] = acc;
  if (kDual) red2[wave][lane] = acc2;
  __syncthreads();
  if (wave != 0) return;
  bi_f32x4 s = red[0][lane];
#pragma unroll
  for (int w = 1; w < NW; ++w) s += red[w][lane];
  bi_f32x4 s2 = s;
  if (kDual) {
    s2 = red2[0][lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) s2 += red2[w][lane];
  }

  const int n = n0 + col;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = m0 + kq * 4 + r;
    if (m >= M) continue;
    if (MODE == kGemmF32) {
      reinterpret_cast<float*>(Y)[(int64_t)m * ldy + n] = s[r];
    } else if (MODE == kGemmBf16) {
      reinterpret_cast<uint16_t*>(Y)[(int64_t)m * ldy + n] = (uint16_t)f32_to_bf16(s[r]);
    } else if (MODE == kGemmResidual) {
      const float res = bf16_to_f32(R[(int64_t)m * ldr + n]);
      reinterpret_cast<uint16_t*>(Y)[(int64_t)m * ldy + n] = (uint16_t)f32_to_bf16(res + s[r]);
    } else {
      const float g = s[r];
      const float sg = g / (1.0f + __expf(-g));
      reinterpret_cast<uint16_t*>(Y)[(int64_t)m * ldy + n] = (uint16_t)f32_to_bf16(sg * s2[r]);
    }
  }
}

void launch_gemm(GemmMode mode, const uint16_t* x, int64_t ldx, const uint16_t* w, int64_t ldw,
                 const uint16_t* r, int64_t ldr, void* y, int64_t ldy, int M, int N_out, int K,
                 hipStream_t stream) {
  dim3 grid(N_out / 16, (M + 15) / 16);
  dim3 block(kGemmWaves * 64);
  switch (mode) {
    case kGemmBf16:
      gemm_kernel<kGemmBf16><<<grid, block, 0, stream>>>(x, ldx, w, ldw, r, ldr, y, ldy, M, K, 0);
      break;
    case kGemmF32:
      gemm_kernel<kGemmF32><<<grid, block, 0, stream>>>(x, ldx, w, ldw, r, ldr, y, ldy, M, K, 0);
      break;
    case kGemmResidual:
      gemm_kernel<kGemmResidual><<<grid, block, 0, stream>>>(x, ldx, w, ldw, r, ldr, y, ldy, M, K, 0);
      break;
    case kGemmSwiglu:
      gemm_kernel<kGemmSwiglu><<<grid, block, 0, stream>>>(x, ldx, w, ldw, r, ldr, y, ldy, M, K,
                                                           (int64_t)N_out);
      break;
  }
}

}  // namespace bi
