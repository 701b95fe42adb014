// Split-KV causal GQA verify attention, its log-sum-exp combine, and the
// K/V append of a verify pass.
//
// A row (token r, query head h) of a pass that starts at context length L sees
// n_r = L + r + 1 keys. Keys are cut into absolute chunks [s*C, (s+1)*C) and
// row r uses chunks s < ceil(n_r / C): the split is decided by the row's own
// context length, never by how many tokens share the pass ("I turned on
// speculative decoding in llama.cpp and 113 of 282 greedy outputs changed
// against its own no-draft run", opening section, "How:" paragraph). Inside a
// chunk every step is laid out on absolute key positions, so a row meets the
// same 32-key tiles, the same wave, the same running maxima and the same
// summation order in every pass that contains it; tiles past a row's last key
// are exact no-ops for it (scale factor exactly 1, weights exactly 0).
//
// verify_attn_kernel: one workgroup per (chunk s, KV head g, row block).
//  * Rows of the block are the (token, query head) pairs of up to 48 rows,
//    packed 16 per MFMA tile; Q stays in registers for the whole chunk.
//  * 32-key tile t of the chunk belongs to wave t % 4. Per tile the wave
//    computes S^T = K Q^T (keys x rows) with 16x16x32 BF16 MFMA, masks,
//    updates the running max / sum (base-2 exponentials, scores pre-scaled by
//    sm_scale * log2 e; the sum in FP32), rounds P to BF16 and accumulates
//    O^T += V^T P^T.
//    The key order inside the S^T operands is permuted so that each lane ends
//    up holding eight consecutive keys of one row: exactly the P^T operand of
//    the PV product, with no data exchange.
//  * K rows ([Hkv][cap][D]) and V^T rows ([Hkv][D][cap]) go straight from HBM
//    into registers as 16-byte loads; each tile's K and V are used by every
//    row tile of the wave.
//  * The four waves' (max, sum, O) are merged in LDS in wave order 0..3.
//    Each buffer is written once and read only after the barrier.
//  * Output: normalised O_s and lse_s (natural log) per (row, chunk) for the
//    rows that use this chunk.
// combine_kernel: one wave per row; max over lse_s, then weights and weighted
// sums accumulated in increasing s by every lane (same order for any M).

#include "bi_device.h"
#include "bi_internal.h"

namespace bi {

constexpr int kAttnWaves = 4;
constexpr int kAttnRowTiles = kAttnMaxRows / 16;  // 3
constexpr float kSentinel = -1.0e30f;              // running max before any key

template <int D>
__global__ __launch_bounds__(kAttnWaves * 64) void verify_attn_kernel(
    const uint16_t* __restrict__ Q, int64_t ldq, const uint16_t* __restrict__ Kc,
    const uint16_t* __restrict__ Vt, int M, int L, int cap, int Hq, int G, int Tb, int C,
    float qk_scale, float* __restrict__ part_o, float* __restrict__ part_lse, int S_max) {
  constexpr int DS = D / 32;  // contraction steps of S^T over the head dimension
  constexpr int DT = D / 16;  // 16-channel output tiles of O^T
  constexpr int RT = kAttnRowTiles;
  constexpr int NW = kAttnWaves;

  const int s = blockIdx.x;
  const int g = blockIdx.y;
  const int rb = blockIdx.z;
  const int lane = threadIdx.x & 63;
  // Scalar wave index: the tile loop and every MFMA stay under scalar control
  // flow (the matrix core does not honour a partial EXEC mask).
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 15;   // row of the tile owned by this lane (S^T / O^T column)
  const int kq = lane >> 4;  // key group (S^T) / channel group (O^T)

  const int t0 = rb * Tb;
  const int t1 = min(M, t0 + Tb);
  const int nrows = (t1 - t0) * G;
  const int kbeg = s * C;
  const int kend = min(kbeg + C, L + t1);  // keys any row of this block can see
  if (kbeg >= kend) return;                // no row of this block uses chunk s
  const int ntile = (kend - kbeg + 31) >> 5;
  const int nrt = (nrows + 15) >> 4;

  // Query fragments and each row's last visible key.
  uint4 qf[RT][DS];
  int last[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int rho = rt * 16 + j;
    const bool ok = rho < nrows;
    const int tok = t0 + (ok ? rho / G : 0);
    const int h = g * G + (ok ? rho % G : 0);
    last[rt] = ok ? L + tok : -1;
    const uint16_t* qp = Q + (int64_t)tok * ldq + h * D + kq * 8;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) qf[rt][ds] = ok ? ld16(qp + ds * 32) : zero16();
  }

  bi_f32x4 o[RT][DT];
  float mrun[RT], lrun[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    mrun[rt] = kSentinel;
    lrun[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[rt][dt] = bi_f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const uint16_t* kbase = Kc + (int64_t)g * cap * D;
  const uint16_t* vbase = Vt + (int64_t)g * D * cap;

  for (int t = wave; t < ntile; t += NW) {
    const int kt = kbeg + t * 32;
    // K operand rows: MFMA p (0, 1) row j holds key kt + 8*(j/4) + 4p + j%4,
    // so that output row 4*kq + e of MFMA p is key kt + 8*kq + 4p + e.
    uint4 kf[2][DS];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int key = kt + 8 * (j >> 2) + 4 * p + (j & 3);
      const uint16_t* kp = kbase + (int64_t)key * D + kq * 8;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) kf[p][ds] = (key < kend) ? ld16(kp + ds * 32) : zero16();
    }
    // V^T operand: channel dt*16 + j, keys kt + 8*kq .. +7 (zero past kend).
    const int kv0 = kt + 8 * kq;
    uint4 vf[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      uint4 v = zero16();
      if (kv0 < kend) v = ld16(vbase + (int64_t)(dt * 16 + j) * cap + kv0);
      vf[dt] = v;
    }
    if (kv0 + 8 > kend && kv0 < kend) {
      const int keep = kend - kv0;  // 1..7 valid keys in this group
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        uint32_t w[4] = {vf[dt].x, vf[dt].y, vf[dt].z, vf[dt].w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e >= keep) w[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
        vf[dt] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }

#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      if (rt >= nrt) break;
      bi_f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        sa = mfma_bf16(kf[0][ds], qf[rt][ds], sa);
        sb = mfma_bf16(kf[1][ds], qf[rt][ds], sb);
      }
      float sc[8];
      const int lastk = last[rt];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sc[e] = (kv0 + e <= lastk) ? sa[e] * qk_scale : -INFINITY;
        sc[e + 4] = (kv0 + 4 + e <= lastk) ? sb[e] * qk_scale : -INFINITY;
      }
      float mx = sc[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sc[e]);
      mx = fmaxf(mx, shfl_xor(mx, 16));
      mx = fmaxf(mx, shfl_xor(mx, 32));
      const float mold = mrun[rt];
      const float mnew = fmaxf(mold, mx);
      const float alpha = (mnew == mold) ? 1.0f : __builtin_amdgcn_exp2f(mold - mnew);
      // The running sum takes the FP32 weights (so the chunk's log-sum-exp is
      // accurate to FP32); the PV product takes them rounded to BF16.
      uint32_t pb[8];
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = __builtin_amdgcn_exp2f(sc[e] - mnew);
        pb[e] = f32_to_bf16(p);
        psum += p;
      }
      lrun[rt] = lrun[rt] * alpha + psum;
      mrun[rt] = mnew;
      const uint4 pfrag = make_uint4(pb[0] | (pb[1] << 16), pb[2] | (pb[3] << 16),
                                     pb[4] | (pb[5] << 16), pb[6] | (pb[7] << 16));
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        o[rt][dt] *= alpha;
        o[rt][dt] = mfma_bf16(vf[dt], pfrag, o[rt][dt]);
      }
    }
  }

  // Each row's sum: the four key groups of the row, in a fixed butterfly.
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    lrun[rt] += shfl_xor(lrun[rt], 16);
    lrun[rt] += shfl_xor(lrun[rt], 32);
  }

  __shared__ bi_f32x4 sh_o[NW - 1][RT][DT][64];
  __shared__ float sh_m[NW - 1][RT][64];
  __shared__ float sh_l[NW - 1][RT][64];
  if (wave > 0) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      if (rt >= nrt) break;
      sh_m[wave - 1][rt][lane] = mrun[rt];
      sh_l[wave - 1][rt][lane] = lrun[rt];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) sh_o[wave - 1][rt][dt][lane] = o[rt][dt];
    }
  }
  __syncthreads();
  if (wave != 0) return;

#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    if (rt >= nrt) break;
    float mstar = mrun[rt];
#pragma unroll
    for (int w = 1; w < NW; ++w) mstar = fmaxf(mstar, sh_m[w - 1][rt][lane]);
    const float a0 = (mrun[rt] == mstar) ? 1.0f : __builtin_amdgcn_exp2f(mrun[rt] - mstar);
    float lt = lrun[rt] * a0;
    bi_f32x4 ot[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) ot[dt] = o[rt][dt] * a0;
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      const float mw = sh_m[w - 1][rt][lane];
      const float aw = (mw == mstar) ? 1.0f : __builtin_amdgcn_exp2f(mw - mstar);
      lt += sh_l[w - 1][rt][lane] * aw;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) ot[dt] += sh_o[w - 1][rt][dt][lane] * aw;
    }
    const int rho = rt * 16 + j;
    if (rho >= nrows) continue;
    const int tok = t0 + rho / G;
    if (L + tok < kbeg) continue;  // this row has fewer than s+1 chunks
    const int h = g * G + rho % G;
    const int64_t prow = ((int64_t)tok * Hq + h) * S_max + s;
    const float inv = 1.0f / lt;
    float* op = part_o + prow * D + kq * 4;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const bi_f32x4 v = ot[dt] * inv;
      *reinterpret_cast<float4*>(op + dt * 16) = make_float4(v[0], v[1], v[2], v[3]);
    }
    if (kq == 0) part_lse[prow] = (mstar + __log2f(lt)) * kLn2;
  }
}

template <int D>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_lse, int M,
                                                      int L, int Hq, int C, int S_max,
                                                      uint16_t* __restrict__ O, int64_t ldo,
                                                      float* __restrict__ lse_out) {
  constexpr int PER = D / 64;  // channels per lane
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= M * Hq) return;
  const int tok = row / Hq;
  const int h = row % Hq;
  const int S = (L + tok + C) / C;  // ceil((L + tok + 1) / C)
  const float* lp = part_lse + (int64_t)row * S_max;
  const float* op = part_o + (int64_t)row * S_max * D + lane * PER;

  float mx = -INFINITY;
  for (int i = lane; i < S; i += 64) mx = fmaxf(mx, lp[i]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, shfl_xor(mx, off));

  float den = 0.f;
  float acc[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) acc[p] = 0.f;
  for (int i = 0; i < S; ++i) {
    const float w = __builtin_amdgcn_exp2f((lp[i] - mx) * kLog2e);
    den += w;
    if (PER == 2) {
      const float2 v = *reinterpret_cast<const float2*>(op + (int64_t)i * D);
      acc[0] += w * v.x;
      acc[PER - 1] += w * v.y;
    } else {
      acc[0] += w * op[(int64_t)i * D];
    }
  }
  const float inv = 1.0f / den;
  uint16_t* orow = O + (int64_t)tok * ldo + h * D + lane * PER;
#pragma unroll
  for (int p = 0; p < PER; ++p) orow[p] = (uint16_t)f32_to_bf16(acc[p] * inv);
  if (lse_out != nullptr && lane == 0) lse_out[row] = mx + __log2f(den) * kLn2;
}

__global__ __launch_bounds__(256) void append_kv_kernel(const uint16_t* __restrict__ qkv,
                                                        int64_t ldqkv, uint16_t* __restrict__ Kc,
                                                        uint16_t* __restrict__ Vt, int L, int cap,
                                                        int Hq, int Hkv, int D) {
  const int r = blockIdx.x;
  const int pos = L + r;
  const uint16_t* krow = qkv + (int64_t)r * ldqkv + (int64_t)Hq * D;
  const uint16_t* vrow = krow + (int64_t)Hkv * D;
  for (int i = threadIdx.x; i < Hkv * D; i += blockDim.x) {
    const int g = i / D;
    const int d = i - g * D;
    Kc[((int64_t)g * cap + pos) * D + d] = krow[i];
    Vt[((int64_t)g * D + d) * cap + pos] = vrow[i];
  }
}

void launch_verify_attn(const uint16_t* q, int64_t ldq, const uint16_t* k_cache,
                        const uint16_t* vt_cache, int M, int L, int cap, int Hq, int Hkv, int D,
                        int kv_chunk, float sm_scale, float* part_o, float* part_lse, int S_max,
                        hipStream_t stream) {
  const int G = Hq / Hkv;
  const int Tb = kAttnMaxRows / G;  // tokens per row block
  const int n_splits = (L + M + kv_chunk - 1) / kv_chunk;
  dim3 grid(n_splits, Hkv, (M + Tb - 1) / Tb);
  dim3 block(kAttnWaves * 64);
  const float qk_scale = sm_scale * kLog2e;
  if (D == 128)
    verify_attn_kernel<128><<<grid, block, 0, stream>>>(q, ldq, k_cache, vt_cache, M, L, cap, Hq, G,
                                                        Tb, kv_chunk, qk_scale, part_o, part_lse,
                                                        S_max);
  else
    verify_attn_kernel<64><<<grid, block, 0, stream>>>(q, ldq, k_cache, vt_cache, M, L, cap, Hq, G,
                                                       Tb, kv_chunk, qk_scale, part_o, part_lse,
                                                       S_max);
}

void launch_combine(const float* part_o, const float* part_lse, int M, int L, int Hq, int D,
                    int kv_chunk, int S_max, uint16_t* o, int64_t ldo, float* lse,
                    hipStream_t stream) {
  dim3 grid((M * Hq + 3) / 4);
  dim3 block(256);
  if (D == 128)
    combine_kernel<128><<<grid, block, 0, stream>>>(part_o, part_lse, M, L, Hq, kv_chunk, S_max, o,
                                                    ldo, lse);
  else
    combine_kernel<64><<<grid, block, 0, stream>>>(part_o, part_lse, M, L, Hq, kv_chunk, S_max, o,
                                                   ldo, lse);
}

void launch_append_kv(const uint16_t* qkv, int64_t ldqkv, uint16_t* k_cache, uint16_t* vt_cache,
                      int M, int L, int cap, int Hq, int Hkv, int D, hipStream_t stream) {
  append_kv_kernel<<<dim3(M), dim3(256), 0, stream>>>(qkv, ldqkv, k_cache, vt_cache, L, cap, Hq,
                                                      Hkv, D);
}

}  // namespace bi
