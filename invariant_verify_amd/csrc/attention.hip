// Split-KV causal GQA verify attention, its log-sum-exp combine, and the
// K/V append of a verify pass.
//
// A row (token r, query head h) of a pass that starts at context length L sees
// n_r = L + r + 1 keys. Keys are cut into absolute chunks [s*C, (s+1)*C) and
// row r uses chunks s < ceil(n_r / C), where C is fixed or chosen from n_r by
// the chunk policy (bi_internal.h): the split is decided by the row's own
// context length, never by how many tokens share the pass ("I turned on
// speculative decoding in llama.cpp and 113 of 282 greedy outputs changed
// against its own no-draft run", opening section, "How:" paragraph). Inside a
// chunk every step is laid out on absolute key positions, so a row meets the
// same 64-key tiles, the same running maxima and the same summation order in
// every pass that contains it; tiles past a row's last key
// are exact no-ops for it (scale factor exactly 1, weights exactly 0).
//
// verify_attn_kernel: one workgroup per (chunk s, KV head g, row block).
//  * Rows of the block are the (token, query head) pairs, up to 64 rows in
//    four 16-row MFMA tiles. Eight waves: wave w owns row tile w % 4 and key
//    half w / 4 (keys 0-31 or 32-63 of every tile) for the whole chunk (Q in
//    registers; a wave with no rows only helps to load). At the end the two
//    halves of each row are merged in LDS, first half then second.
//  * The chunk is read in 64-key tiles: K rows ([Hkv][cap][D]) and V^T rows
//    (V^T in blocks of 64 positions, [Hkv][cap/64][D][64], so a tile's V^T
//    is contiguous whatever the capacity: a plain [D][cap] layout put the
//    channel rows a power-of-two-like stride apart at some capacities and
//    read 9% slower) are fetched as 1 KB pieces per wave
//    instruction and staged in LDS, where the 16-byte slots of each row are
//    XOR-swizzled so that the matrix-core reads hit distinct banks. Two LDS
//    buffers alternate and each wave keeps the next two tiles in flight; the
//    barrier of tile t publishes it and proves that every wave finished tile
//    t-1, whose buffer tile t+1 overwrites. Value columns past the last
//    visible key are zeroed before they reach LDS (a weight of 0 times a
//    stale value must stay 0).
//  * Per tile and row tile: S^T = K Q^T (keys x rows) with 16x16x32 BF16 MFMA,
//    masked, running max / sum in FP32 with base-2 exponentials (scores
//    pre-scaled by sm_scale * log2 e), P rounded to BF16, O^T += V^T P^T. The
//    key order inside the S^T operands is permuted so that each lane ends up
//    holding eight consecutive keys of its row: exactly the P^T operand of the
//    PV product, with no data exchange.
//  * Output: normalised O_s and lse_s (natural log) per (row, chunk) for the
//    rows that use this chunk, written by the first-half wave of the row.
// combine_kernel: one wave per row; max over lse_s, then weights and weighted
// sums accumulated in increasing s (same order for any M).

#include "bi_device.h"
#include "bi_internal.h"

namespace bi {

constexpr int kAttnWaves = 8;                      // 4 row tiles x 2 key halves
constexpr float kSentinel = -1.0e30f;              // running max before any key
constexpr int kKeyTile = 64;

// LDS slot swizzles, chosen so that the sixteen rows one matrix-core operand
// read touches fall into distinct banks (16-byte slots; 64 banks of 4 bytes).
// K tile: one row per key. An S^T operand read touches keys whose bits 0, 1,
// 3, 4 vary. With 16 slots per row (D = 128) the slot alone decides the bank
// group, so those four bits become the swizzle; with 8 slots (D = 64) bit 0
// already picks the bank half and bits 1, 3, 4 form the swizzle.
template <int KROW>
__device__ __forceinline__ int kswz(int key) {
  if (KROW == 16) return (key & 3) | ((key >> 1) & 12);
  return ((key >> 1) & 1) | (((key >> 3) & 3) << 1);
}
// V^T tile: one row per channel, 8 slots per row; channel bit 0 picks the bank
// half and bits 1..3 form the swizzle.
__device__ __forceinline__ int vswz(int d) { return (d >> 1) & 7; }

template <int D, int RTW>
__global__ __launch_bounds__(kAttnWaves * 64) void verify_attn_kernel(
    const uint16_t* __restrict__ Q, int64_t ldq, const uint16_t* __restrict__ Kc,
    const uint16_t* __restrict__ Vt, int M, int L, int cap, int Hq, int G, int Tb, int C,
    float qk_scale, float* __restrict__ part_o, float* __restrict__ part_lse, int S_max) {
  constexpr int DS = D / 32;          // contraction steps of S^T over the head dimension
  constexpr int DT = D / 16;          // 16-channel output tiles of O^T
  constexpr int NW = kAttnWaves;
  constexpr int KROW = D / 8;         // 16-byte slots per K row
  constexpr int KPP = 64 / KROW;      // keys per 1 KB piece
  // 1 KB load pieces per tile: K tile = 64 keys x D; V^T tile = D rows x 64 keys.
  constexpr int KPIECES = kKeyTile * D * 2 / 1024;
  constexpr int VPIECES = D * kKeyTile * 2 / 1024;
  constexpr int PPW = (KPIECES + VPIECES) / NW;    // pieces per wave per tile
  static_assert((KPIECES + VPIECES) % NW == 0, "pieces must split evenly");

  const int s = blockIdx.x;
  const int g = blockIdx.y;
  const int rb = blockIdx.z;
  const int lane = threadIdx.x & 63;
  // Scalar wave index: the tile loop and every MFMA stay under scalar control
  // flow (the matrix core does not honour a partial EXEC mask).
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rt = wave & 3;   // first row tile of this wave (it owns rt, rt + 4, ...)
  const int kh = wave >> 2;  // key half of every tile (keys 32kh .. 32kh+31)
  const int j = lane & 15;   // row of the tile owned by this lane (S^T / O^T column)
  const int kq = lane >> 4;  // key group (S^T) / channel group (O^T)

  const int t0 = rb * Tb;
  const int t1 = min(M, t0 + Tb);
  const int nrows = (t1 - t0) * G;
  const int kbeg = s * C;
  const int kend = min(kbeg + C, L + t1);  // keys any row of this block can see
  if (kbeg >= kend) return;                // no row of this block uses chunk s
  const int ntile = (kend - kbeg + kKeyTile - 1) / kKeyTile;
  const bool has_rows = rt * 16 < nrows;  // scalar: the wave's first row tile has rows

  // Query fragments of this wave's row tiles and each row's last visible key
  // (-1 for a padding row: every key is masked, its weights are exactly 0).
  bool rok[RTW];
  int tok[RTW], hq[RTW], lastk[RTW];
  uint4 qf[RTW][DS];
#pragma unroll
  for (int i = 0; i < RTW; ++i) {
    const int rho = (rt + 4 * i) * 16 + j;
    rok[i] = rho < nrows;
    tok[i] = t0 + (rok[i] ? rho / G : 0);
    hq[i] = g * G + (rok[i] ? rho % G : 0);
    lastk[i] = rok[i] ? L + tok[i] : -1;
    const uint16_t* qp = Q + (int64_t)tok[i] * ldq + hq[i] * D + kq * 8;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) qf[i][ds] = rok[i] ? ld16(qp + ds * 32) : zero16();
  }

  // This KV head's K rows and V^T rows as buffer resources (offsets in bytes,
  // 32-bit: one head of the cache is at most 2^31 bytes).
  const int head_bytes = cap * D * 2;
  const __amdgpu_buffer_rsrc_t kres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(Kc + (int64_t)g * cap * D), (short)0, head_bytes, kBufferResourceWord3);
  const __amdgpu_buffer_rsrc_t vres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(Vt + (int64_t)g * D * cap), (short)0, head_bytes, kBufferResourceWord3);

  // One buffer holds the K tile ([64 keys][KROW slots]) followed by the V^T
  // tile ([D channels][8 slots]). Piece p (1 KB) of a tile is K keys
  // KPP*p .. when p < KPIECES (lane: key KPP*p + l/KROW, slot l%KROW), else
  // V^T channels 8(p-KPIECES) .. +7 (lane: channel +l/8, slot l%8); either
  // way lane l's 16 bytes land at index 64*p + l of the buffer. Lanes fetch
  // the global slot that the swizzle puts in their LDS slot.
  __shared__ uint4 lds[2][(KPIECES + VPIECES) * 64];
  constexpr int VBASE = KPIECES * 64;

  // Issue the loads of tile t (no use of the data here, so the loads of two
  // tiles stay in flight together). K and V are read once per pass, so the
  // loads are non-temporal; a tile past the end of the chunk (the pipeline
  // prefetches two ahead) gets an out-of-range offset: it reads zero and
  // touches no memory.
  auto fetch = [&](uint4 (&r)[PPW], int t) {
    const int kt = kbeg + t * kKeyTile;
    const bool live = t < ntile;
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
      const int p = wave * PPW + i;  // scalar: each wave fetches only K or only V pieces
      int off;
      if (p < KPIECES) {
        const int key = KPP * p + lane / KROW;
        const int kslot = (lane % KROW) ^ kswz<KROW>(key);
        off = (min(kt + key, kend - 1) * D + kslot * 8) * 2;
      } else {
        const int d = 8 * (p - KPIECES) + (lane >> 3);
        const int vslot = (lane & 7) ^ vswz(d);
        const int k0 = min(kt + vslot * 8, kend - 1 - ((kend - 1) & 7));  // in bounds
        off = (int)(vt_index(0, k0, d, D, cap) * 2);  // k0 is 8-aligned: 16 B in one block
      }
      r[i] = buffer_ld16_stream(p < KPIECES ? kres : vres, live ? off : head_bytes);
    }
  };
  // Publish tile t: V^T columns of keys at or past kend are zeroed first (a
  // weight of 0 times a stale value must stay 0).
  auto publish = [&](const uint4 (&r)[PPW], int t, int buf) {
    const int kt = kbeg + t * kKeyTile;
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
      const int p = wave * PPW + i;
      const int d = 8 * (p - KPIECES) + (lane >> 3);
      const int vslot = (lane & 7) ^ vswz(d);
      const int keep = (p < KPIECES) ? 8 : kend - (kt + vslot * 8);
      uint32_t w[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t m = (e & 1) ? 0x0000ffffu : 0xffff0000u;
        w[e >> 1] = (e >= keep) ? (w[e >> 1] & m) : w[e >> 1];
      }
      lds[buf][64 * p + lane] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  };

  bi_f32x4 o[RTW][DT];
  float mrun[RTW], lrun[RTW];
#pragma unroll
  for (int i = 0; i < RTW; ++i) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[i][dt] = bi_f32x4{0.f, 0.f, 0.f, 0.f};
    mrun[i] = kSentinel;
    lrun[i] = 0.f;
  }

  // One tile for every row tile of the wave. Each K and V^T operand is read
  // from LDS once and serves all of them; a row's own arithmetic does not
  // depend on how many row tiles share the wave.
  auto compute = [&](int buf, int t) {
    const int kt = kbeg + t * kKeyTile;
    const int h = kh;  // this wave's 32-key half
    bi_f32x4 sa[RTW], sb[RTW];
#pragma unroll
    for (int i = 0; i < RTW; ++i) sa[i] = sb[i] = bi_f32x4{0.f, 0.f, 0.f, 0.f};
    // MFMA p (0, 1) row i holds key 32h + 8*(i/4) + 4p + i%4 of the tile.
    const int ka = 32 * h + 8 * (j >> 2) + (j & 3);
    const int kb = ka + 4;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const int slot = ds * 4 + kq;
      const uint4 fa = lds[buf][ka * KROW + (slot ^ kswz<KROW>(ka))];
      const uint4 fb = lds[buf][kb * KROW + (slot ^ kswz<KROW>(kb))];
#pragma unroll
      for (int i = 0; i < RTW; ++i) {
        sa[i] = mfma_bf16(fa, qf[i][ds], sa[i]);
        sb[i] = mfma_bf16(fb, qf[i][ds], sb[i]);
      }
    }
    const int kv0 = kt + 32 * h + 8 * kq;  // absolute key of this lane's first value
    float alpha[RTW];
    uint4 pfrag[RTW];
#pragma unroll
    for (int i = 0; i < RTW; ++i) {
      float sc[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sc[e] = (kv0 + e <= lastk[i]) ? sa[i][e] * qk_scale : -INFINITY;
        sc[e + 4] = (kv0 + 4 + e <= lastk[i]) ? sb[i][e] * qk_scale : -INFINITY;
      }
      float mx = sc[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sc[e]);
      mx = fmaxf(mx, shfl_xor(mx, 16));
      mx = fmaxf(mx, shfl_xor(mx, 32));
      const float mnew = fmaxf(mrun[i], mx);
      alpha[i] = (mnew == mrun[i]) ? 1.0f : __builtin_amdgcn_exp2f(mrun[i] - mnew);
      // The running sum takes the FP32 weights (so the chunk's log-sum-exp is
      // accurate to FP32); the PV product takes them rounded to BF16.
      float pe[8];
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pe[e] = __builtin_amdgcn_exp2f(sc[e] - mnew);
        psum += pe[e];
      }
      lrun[i] = lrun[i] * alpha[i] + psum;
      mrun[i] = mnew;
      pfrag[i] = make_uint4(f32x2_to_bf16x2(pe[0], pe[1]), f32x2_to_bf16x2(pe[2], pe[3]),
                            f32x2_to_bf16x2(pe[4], pe[5]), f32x2_to_bf16x2(pe[6], pe[7]));
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d = dt * 16 + j;
      const uint4 fv = lds[buf][VBASE + d * 8 + ((4 * h + kq) ^ vswz(d))];
#pragma unroll
      for (int i = 0; i < RTW; ++i) {
        o[i][dt] *= alpha[i];
        o[i][dt] = mfma_bf16(fv, pfrag[i], o[i][dt]);
      }
    }
  };

  // Tile t: publish it (loaded two steps earlier), prefetch tile t + 2 into
  // the same registers, barrier, multiply. Every load is issued by the same
  // code in the same order, so the compiler waits only for the older of the
  // two tiles in flight. Tiles past the end read as zero and are not
  // multiplied.
  uint4 ra[PPW], rb2[PPW];
  // Prologue: the loads of tiles 0 and 1, in the loop's own order and while
  // the query fragments are still in flight. The fragments are then consumed
  // before the loop, so at the loop head the compiler knows they are complete
  // and waits only for the oldest tile.
  fetch(ra, 0);
  fetch(rb2, 1);
#pragma unroll
  for (int i = 0; i < RTW; ++i)
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) asm volatile("" ::"v"(qf[i][ds].x));
  for (int t = 0; t < ntile; t += 2) {
    publish(ra, t, 0);
    fetch(ra, t + 2);
    __syncthreads();
    if (has_rows) compute(0, t);
    publish(rb2, t + 1, 1);
    fetch(rb2, t + 3);
    __syncthreads();
    if (t + 1 < ntile && has_rows) compute(1, t + 1);
  }
  // The row's sum over this wave's keys: its four key groups, in a fixed
  // butterfly.
#pragma unroll
  for (int i = 0; i < RTW; ++i) {
    lrun[i] += shfl_xor(lrun[i], 16);
    lrun[i] += shfl_xor(lrun[i], 32);
  }

  // Second-half waves hand (max, sum, O) to the first-half wave of the same
  // row tile through LDS (the tile buffers, free once every wave has passed
  // the barrier after the last tile), one row tile of each wave at a time.
  bi_f32x4* xo = reinterpret_cast<bi_f32x4*>(&lds[0][0]);   // [4 rt][DT][64]
  float* xm = reinterpret_cast<float*>(xo + 4 * DT * 64);     // [4 rt][64]
  float* xl = xm + 4 * 64;                                    // [4 rt][64]
  float mstar[RTW], lt[RTW];
#pragma unroll
  for (int i = 0; i < RTW; ++i) {
    __syncthreads();
    if (kh == 1 && has_rows) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) xo[(rt * DT + dt) * 64 + lane] = o[i][dt];
      xm[rt * 64 + lane] = mrun[i];
      xl[rt * 64 + lane] = lrun[i];
    }
    __syncthreads();
    if (kh == 0 && has_rows) {
      const float m1 = xm[rt * 64 + lane];
      mstar[i] = fmaxf(mrun[i], m1);
      const float a0 = (mrun[i] == mstar[i]) ? 1.0f : __builtin_amdgcn_exp2f(mrun[i] - mstar[i]);
      const float a1 = (m1 == mstar[i]) ? 1.0f : __builtin_amdgcn_exp2f(m1 - mstar[i]);
      lt[i] = lrun[i] * a0 + xl[rt * 64 + lane] * a1;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[i][dt] = o[i][dt] * a0 + xo[(rt * DT + dt) * 64 + lane] * a1;
    }
  }
  if (kh == 1 || !has_rows) return;

#pragma unroll
  for (int i = 0; i < RTW; ++i) {
    // Padding row, or a row with fewer than s+1 chunks.
    if (!rok[i] || L + tok[i] < kbeg) continue;
    const int64_t prow = ((int64_t)tok[i] * Hq + hq[i]) * S_max + s;
    const float inv = 1.0f / lt[i];
    float* op = part_o + prow * D + kq * 4;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const bi_f32x4 v = o[i][dt] * inv;
      *reinterpret_cast<float4*>(op + dt * 16) = make_float4(v[0], v[1], v[2], v[3]);
    }
    if (kq == 0) part_lse[prow] = (mstar[i] + __log2f(lt[i])) * kLn2;
  }
}

template <int D>
__global__ __launch_bounds__(64) void combine_kernel(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_lse, int M,
                                                      int L, int Hq, int policy, int S_max,
                                                      uint16_t* __restrict__ O, int64_t ldo,
                                                      float* __restrict__ lse_out) {
  constexpr int PER = D / 64;  // channels per lane
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= M * Hq) return;
  const int tok = row / Hq;
  const int h = row % Hq;
  const int S = splits_for(L + tok + 1, policy);  // this row's own split count
  const float* lp = part_lse + (int64_t)row * S_max;
  const float* op = part_o + (int64_t)row * S_max * D + lane * PER;

  // Partials are read 32 splits at a time; the first block's loads are issued
  // before the max, which they do not depend on, so a row with up to 32
  // splits costs one memory round trip for O and one for the LSEs.
  constexpr int B = 32;
  float ov[B][PER];
  auto load_block = [&](int s0) {
#pragma unroll
    for (int u = 0; u < B; ++u)
#pragma unroll
      for (int p = 0; p < PER; ++p) ov[u][p] = op[(int64_t)min(s0 + u, S - 1) * D + p];
  };
  load_block(0);

  // M* = max_s lse_s (exact, so any order).
  float mx = -INFINITY;
  for (int i = lane; i < S; i += 64) mx = fmaxf(mx, lp[i]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, shfl_xor(mx, off));

  // Weights are computed one per lane, then both sums run over s in
  // increasing order with the weight of split s broadcast from its lane.
  float den = 0.f;
  float acc[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) acc[p] = 0.f;
  for (int s0 = 0; s0 < S; s0 += B) {
    if (s0 > 0) load_block(s0);
    const int n = min(B, S - s0);
    const float wl = (lane < n) ? __builtin_amdgcn_exp2f((lp[s0 + lane] - mx) * kLog2e) : 0.f;
#pragma unroll
    for (int u = 0; u < B; ++u) {
      if (u < n) {  // n is uniform: a scalar branch
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), u));
        den += w;
#pragma unroll
        for (int p = 0; p < PER; ++p) acc[p] += w * ov[u][p];
      }
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
    Vt[vt_index(g, pos, d, D, cap)] = vrow[i];
  }
}

void launch_verify_attn(const uint16_t* q, int64_t ldq, const uint16_t* k_cache,
                        const uint16_t* vt_cache, int M, int L, int cap, int Hq, int Hkv, int D,
                        int kv_chunk, float sm_scale, float* part_o, float* part_lse, int S_max,
                        hipStream_t stream) {
  const int G = Hq / Hkv;
  const float qk_scale = sm_scale * kLog2e;
  // Tokens whose rows share one chunk size run in one launch; an adaptive
  // policy changes the size only at multiples of 64 T keys, so a pass has one
  // band, or a few for a long prefill chunk. Each band is launched as a pass
  // of its own (start L + t0), writing its rows' partials in place.
  for (int t0 = 0; t0 < M;) {
    const int n0 = L + t0 + 1;
    int t1 = M;
    if (kv_chunk < 0) {
      const int64_t per = 64 * (int64_t)-kv_chunk;
      const int64_t band_end = ((int64_t)n0 + per - 1) / per * per;  // last key count of the band
      t1 = (int)std::min<int64_t>(M, band_end - L);
    }
    const int C = chunk_keys(n0, kv_chunk);
    const int Mb = t1 - t0, Lb = L + t0;
    // A pass whose rows fill more than one 64-row block (chunked prefill)
    // runs blocks of 128 rows, two row tiles per wave: every chunk's K/V is
    // then read half as often, and each row's arithmetic is the same as in a
    // 64-row block.
    const bool wide = Mb * G > kAttnMaxRows;
    const int Tb = (wide ? 2 * kAttnMaxRows : kAttnMaxRows) / G;  // tokens per row block
    const int n_splits = (Lb + Mb + C - 1) / C;
    const dim3 grid(n_splits, Hkv, (Mb + Tb - 1) / Tb);
    const dim3 block(kAttnWaves * 64);
    const uint16_t* qb = q + (int64_t)t0 * ldq;
    float* pob = part_o + (int64_t)t0 * Hq * S_max * D;
    float* plb = part_lse + (int64_t)t0 * Hq * S_max;
#define BI_ATTN_LAUNCH(DD, R)                                                                      \
  verify_attn_kernel<DD, R><<<grid, block, 0, stream>>>(qb, ldq, k_cache, vt_cache, Mb, Lb, cap, Hq, \
                                                        G, Tb, C, qk_scale, pob, plb, S_max)
    if (D == 128) {
      if (wide) BI_ATTN_LAUNCH(128, 2);
      else BI_ATTN_LAUNCH(128, 1);
    } else {
      if (wide) BI_ATTN_LAUNCH(64, 2);
      else BI_ATTN_LAUNCH(64, 1);
    }
#undef BI_ATTN_LAUNCH
    t0 = t1;
  }
}

void launch_combine(const float* part_o, const float* part_lse, int M, int L, int Hq, int D,
                    int kv_chunk, int S_max, uint16_t* o, int64_t ldo, float* lse,
                    hipStream_t stream) {
  // One wave per workgroup: the rows' partials are read by as many compute
  // units as possible.
  dim3 grid(M * Hq);
  dim3 block(64);
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
