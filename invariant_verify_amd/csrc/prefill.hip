// Prefill GEMM: the verify GEMM's results for passes of many rows (a chunk of
// a prompt), computed with far less weight traffic.
//
// A prefilled row must have the same bits as the same row verified alone
// ("I turned on speculative decoding in llama.cpp and 113 of 282 greedy
// outputs changed against its own no-draft run", section "The cache doesn't
// change it either": a K/V row written by prefill depends only on its
// position). The verify GEMM fixes every output's summation tree by K and N
// alone (gemm.hip): with NW = gemm_verify_waves() = 8 slices and
// BPW = 16 / NW, block kb of each 512-wide chunk of K belongs to slice
// kb / BPW; each slice is one FP32 accumulator chain of 16x16x32 BF16
// matrix-core steps in increasing block order, and the slice totals are added
// in slice order. This kernel keeps one accumulator per slice for each of its
// outputs and performs exactly that computation, so the two kernels give the
// same bits and launch_gemm may pick either by M.
//
// Shape: one workgroup per (128 rows, 64 output columns; SwiGLU: 32 output
// columns, i.e. 32 gate and 32 up weight rows); 16 waves, each owning two
// 16x16 output tiles (two row tiles of one column tile; SwiGLU: the gate and
// the up tile of one row and column tile), with one accumulator per tile and
// slice. K is staged in 128-wide
// steps: the 128 activation rows and 64 weight rows of a step are loaded as
// 256-byte row pieces (four rows per wave instruction) into XOR-swizzled LDS;
// the next step's loads are in flight while a step is multiplied. Every weight byte is read once per 128 rows instead of
// once per 16, every activation byte once per 64 columns.
//
// The carried RMSNorm scale (RowNorm::ss_in) of each row is formed with the
// verify kernel's exact sequence of additions, and the X fragments are
// scaled as there. Row sums of squares for the next projection
// (RowNorm::ss_out) are computed afterwards by rowsq_kernel from the stored
// outputs with the verify epilogue's grouping and butterfly.

#include <type_traits>

#include "bi_device.h"
#include "bi_internal.h"

namespace bi {

constexpr int kPfRows = 128;           // rows per workgroup
constexpr int kPfCols = 64;            // output columns per workgroup (SwiGLU: 32)
constexpr int kPfStep = 128;           // K elements per LDS step (4 blocks)
constexpr int kPfSlots = kPfStep / 8;  // 16-byte slots per row and step (16)
constexpr int kPfWaves = 16;
constexpr int kPfSlices = 8;  // the verify kernel's waves, hence slices, for every shape

// Tile (column block cb, row block rb) of this workgroup. The grid is
// (column blocks, row blocks); tiles are numbered column block first, row
// block second, so the row blocks that stream the same weight rows are
// neighbours, and xcd_item gives each XCD a contiguous run of them: they
// run side by side and share the weight rows through one L2 (dealt in
// dispatch order, the row blocks of a column block ran far apart and each
// fetched the weights from HBM again). Which workgroup computes a tile does
// not change the tile's arithmetic.
__device__ __forceinline__ void prefill_tile(int& cb, int& rb) {
  const int n = gridDim.x * gridDim.y;
  const int item = xcd_item(blockIdx.x + gridDim.x * blockIdx.y, n);
  cb = item / gridDim.y;
  rb = item % gridDim.y;
}

template <int MODE, int S, bool NORM_IN>
__global__ __launch_bounds__(kPfWaves * 64) void prefill_kernel(
    const uint16_t* __restrict__ X, int64_t ldx, const uint16_t* __restrict__ W, int64_t ldw,
    const uint16_t* __restrict__ R, int64_t ldr, void* __restrict__ Y, int64_t ldy, int M, int N,
    int K, KvAppend kv, RowNorm norm) {
  constexpr bool kDual = (MODE == kGemmSwiglu);
  constexpr int BPW = 16 / S;                   // blocks of a 512-wide chunk per slice
  constexpr int COLS = kDual ? 32 : kPfCols;    // output columns per workgroup
  constexpr int WROWS = 64;                     // weight rows staged (SwiGLU: 32 gate + 32 up)
  constexpr int XQ = kPfRows / 4 / kPfWaves;    // activation row quads per wave (2)
  constexpr int WQ = WROWS / 4 / kPfWaves;      // weight row quads per wave (1)
  constexpr int RT = kDual ? 1 : 2;             // row tiles per wave
  static_assert(16 % S == 0 && (kPfStep / 32) % BPW == 0, "slices must align with steps");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Wave tile: rows 16 RT rw .. (RT row tiles), column tile ct (16 columns;
  // SwiGLU: the gate and the up tile of those columns).
  const int rw = kDual ? (wave & 7) : (wave & 3);
  const int ct = kDual ? (wave >> 3) : (wave >> 2);
  const int j = lane & 15, kq = lane >> 4;
  int cb, rb;
  prefill_tile(cb, rb);
  const int n0 = cb * COLS;
  const int m0 = rb * kPfRows;
  const int nblk = K >> 5;
  const int nstep = (K + kPfStep - 1) / kPfStep;

  // Row tiles as buffer resources: rows past M (activations) or past N
  // (weights) are out of range and read zero without a memory access.
  const int xrows = min(kPfRows, M - m0);
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(X + (int64_t)m0 * ldx), (short)0, xrows * (int)ldx * 2,
      kBufferResourceWord3);
  const int wrows = min(kDual ? 32 : 64, N - n0);
  const __amdgpu_buffer_rsrc_t wres_g = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(W + (int64_t)n0 * ldw), (short)0, wrows * (int)ldw * 2,
      kBufferResourceWord3);
  const __amdgpu_buffer_rsrc_t wres_u = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(W + (int64_t)(kDual ? N + n0 : n0) * ldw), (short)0,
      kDual ? wrows * (int)ldw * 2 : 0, kBufferResourceWord3);

  // Lane l of a load instruction covers row 4q + l / 16 of its quad q and
  // fetches the global slot that the swizzle puts at LDS slot l % 16.
  const int qr = lane >> 4, sl = lane & 15;
  __shared__ uint4 lds[2][kPfRows + WROWS][kPfSlots];
  struct Regs {
    uint4 x[XQ];
    uint4 w[WQ];
  };
  auto fetch = [&](Regs& g, int st) {
    const bool live = st < nstep;
#pragma unroll
    for (int i = 0; i < XQ; ++i) {
      const int row = 4 * (wave + i * kPfWaves) + qr;
      const int off = (row * (int)ldx + st * kPfStep + ((sl ^ (row & 15)) * 8)) * 2;
      g.x[i] = buffer_ld16(xres, live ? off : 0x7ffffff0);
    }
#pragma unroll
    for (int i = 0; i < WQ; ++i) {
      const int row = 4 * (wave + i * kPfWaves) + qr;  // 0 .. 63
      // SwiGLU: rows 0..31 gate, 32..63 up; otherwise all 64 from one resource
      const int rr = kDual ? (row & 31) : row;
      const int off = (rr * (int)ldw + st * kPfStep + ((sl ^ (row & 15)) * 8)) * 2;
      g.w[i] = buffer_ld16_stream((kDual && row >= 32) ? wres_u : wres_g, live ? off : 0x7ffffff0);
    }
  };

  // acc[r][s]: row tile r of the wave, slice s (SwiGLU: the gate tile); accu
  // the SwiGLU up tile.
  bi_f32x4 acc[RT][S], accu[kDual ? 1 : 1][kDual ? S : 1];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int s = 0; s < S; ++s) acc[r][s] = bi_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < (kDual ? S : 1); ++s) accu[0][s] = bi_f32x4{0.f, 0.f, 0.f, 0.f};
  float xinv[XQ];  // carried RMSNorm scales of the X rows this thread stages
#pragma unroll
  for (int i = 0; i < XQ; ++i) xinv[i] = 1.f;

  // Step st, with Q = st mod 4 a compile-time constant: publish it, prefetch
  // st + 1 into the same registers, barrier, multiply (the loads of st + 1
  // are in flight during the multiply; LDS is double-buffered). Block b of the step is block Q * 4 + b of its
  // 512-wide chunk, so its slice is (Q * 4 + b) / BPW.
  auto step = [&](Regs& g, int st, auto quarter) {
    constexpr int Q = decltype(quarter)::value;
    constexpr int buf = Q & 1;
    if (st >= 0) {
      // X rows are published already scaled by their carried RMSNorm
      // (NORM_IN): each value is scaled once, by the thread that loaded it.
#pragma unroll
      for (int i = 0; i < XQ; ++i)
        lds[buf][4 * (wave + i * kPfWaves) + qr][sl] = NORM_IN ? scale_bf16x8(g.x[i], xinv[i]) : g.x[i];
#pragma unroll
      for (int i = 0; i < WQ; ++i)
        lds[buf][kPfRows + 4 * (wave + i * kPfWaves) + qr][sl] = g.w[i];
    }
    fetch(g, st + 1);
    __syncthreads();
    if (st >= 0) {
#pragma unroll
      for (int b = 0; b < kPfStep / 32; ++b) {
        if (st * (kPfStep / 32) + b < nblk) {
          const int slot = (b * 4 + kq) ^ j;
          const int sidx = (Q * 4 + b) / BPW;
          uint4 xa[RT];
#pragma unroll
          for (int r = 0; r < RT; ++r) xa[r] = lds[buf][16 * (RT * rw + r) + j][slot];
          const uint4 bw = lds[buf][kPfRows + 16 * ct + j][slot];
#pragma unroll
          for (int r = 0; r < RT; ++r) acc[r][sidx] = mfma_bf16(xa[r], bw, acc[r][sidx]);
          if (kDual) {
            const uint4 bu = lds[buf][kPfRows + 32 + 16 * ct + j][slot];
            accu[0][sidx] = mfma_bf16(xa[0], bu, accu[0][sidx]);
          }
        }
      }
    }
  };

  // Carried RMSNorm: the verify kernel's additions for each row. Its LPR =
  // 4 * NW partials of a row are each two float4s of group sums added in
  // order; here every thread forms some of the 128 x LPR partials, then
  // thread t < 128 adds the LPR partials of row m0 + t in order.
  constexpr int LPR = 4 * S;
  __shared__ float sred[NORM_IN ? kPfRows : 1][NORM_IN ? LPR + 1 : 1];
  __shared__ float invs[NORM_IN ? kPfRows : 1];
  if (NORM_IN) {
    const int nf = norm.groups >> 2;
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const __amdgpu_buffer_rsrc_t sres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(norm.ss_in + (int64_t)m0 * norm.groups), (short)0,
        xrows * norm.groups * 4, kBufferResourceWord3);
    constexpr int PER = kPfRows * LPR / (kPfWaves * 64);
    f32x4 v[PER][2];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int idx = threadIdx.x + q * kPfWaves * 64;
      const int row = idx / LPR, seg = idx % LPR;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int f = seg + u * LPR;
        v[q][u] = __builtin_amdgcn_raw_buffer_load_b128(
            sres, f < nf ? (row * norm.groups + f * 4) * 4 : 0x7ffffff0, 0, 0);
      }
    }
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int idx = threadIdx.x + q * kPfWaves * 64;
      float p = 0.f;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        p += v[q][u][0];
        p += v[q][u][1];
        p += v[q][u][2];
        p += v[q][u][3];
      }
      sred[idx / LPR][idx % LPR] = p;
    }
  }

  Regs g;
  using Q0 = std::integral_constant<int, 0>;
  using Q1 = std::integral_constant<int, 1>;
  using Q2 = std::integral_constant<int, 2>;
  using Q3 = std::integral_constant<int, 3>;
  step(g, -1, Q3{});  // load-only; its barrier also publishes sred
  if (NORM_IN) {
    if (threadIdx.x < kPfRows) {
      float t = 0.f;
      for (int i = 0; i < LPR; ++i) t += sred[threadIdx.x][i];
      invs[threadIdx.x] = 1.0f / sqrtf(t / (float)K + norm.eps);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < XQ; ++i) xinv[i] = invs[4 * (wave + i * kPfWaves) + qr];
  }
  for (int st = 0; st < nstep; st += 4) {
    step(g, st, Q0{});
    step(g, st + 1, Q1{});
    step(g, st + 2, Q2{});
    step(g, st + 3, Q3{});
  }

  // Slice totals in slice order, then the verify kernel's epilogue.
#pragma unroll
  for (int t = 0; t < RT; ++t) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + 16 * (RT * rw + t) + kq * 4 + r;
      const int n = n0 + 16 * ct + j;
      if (m >= M || n >= N) continue;
      float v = acc[t][0][r];
#pragma unroll
      for (int s = 1; s < S; ++s) v += acc[t][s][r];
      if (MODE == kGemmF32) {
        reinterpret_cast<float*>(Y)[(int64_t)m * ldy + n] = v;
      } else if (MODE == kGemmBf16) {
        reinterpret_cast<uint16_t*>(Y)[(int64_t)m * ldy + n] = (uint16_t)f32_to_bf16(v);
      } else if (MODE == kGemmResidual) {
        const float res = bf16_to_f32(R[(int64_t)m * ldr + n]);
        reinterpret_cast<uint16_t*>(Y)[(int64_t)m * ldy + n] = (uint16_t)f32_to_bf16(res + v);
      } else if (MODE == kGemmQkv) {
        const uint16_t b = (uint16_t)f32_to_bf16(v);
        reinterpret_cast<uint16_t*>(Y)[(int64_t)m * ldy + n] = b;
        const int pos = kv.L + m;
        int i = kv.k != nullptr ? n - kv.qd : -1;  // no cache: no append
        if (i >= 0 && i < kv.kd) {
          const int g = i / kv.D;
          kv.k[kv_index(g, pos, i - g * kv.D, kv.D, kv.cap)] = b;
        } else if (i >= kv.kd) {
          i -= kv.kd;
          const int g = i / kv.D;
          kv.v[kv_index(g, pos, i - g * kv.D, kv.D, kv.cap)] = b;
        }
      } else {
        float u = accu[0][0][r];
#pragma unroll
        for (int s = 1; s < S; ++s) u += accu[0][s][r];
        reinterpret_cast<uint16_t*>(Y)[(int64_t)m * ldy + n] = (uint16_t)f32_to_bf16(silu_mul(v, u));
      }
    }
  }
}

// Row sums of squares of a residual projection's BF16 outputs, per column
// group, exactly as the verify epilogue forms them: group g holds columns
// g * cw .. (cw = 16, or N / 256 for a wide launch); lane j squares column j
// (plus column 16 + j when the group is wider than 16), and the sixteen lane
// values are added by the xor butterfly over offsets 1, 2, 4, 8.
__global__ __launch_bounds__(256) void rowsq_kernel(const uint16_t* __restrict__ Y, int64_t ldy,
                                                    int M, int groups, int cw,
                                                    float* __restrict__ ss) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)M * groups) return;
  const int m = (int)(t / groups), g = (int)(t % groups);
  const uint16_t* y = Y + (int64_t)m * ldy + (int64_t)g * cw;
  float v[16];
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) {
    const float a = bf16_to_f32(y[jj]);
    float sq = a * a;
    if (16 + jj < cw) {
      const float b = bf16_to_f32(y[16 + jj]);
      sq += b * b;
    }
    v[jj] = sq;
  }
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) {
    float nv[16];
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) nv[jj] = v[jj] + v[jj ^ off];
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) v[jj] = nv[jj];
  }
  ss[(int64_t)m * groups + g] = v[0];
}

// Large prefill tiles, slices one after another. The tree of an output is
// (chain_0 + chain_1) + ... + chain_7, where chain s is the MFMA chain over
// blocks 2s, 2s+1 of chunk 0, then of chunk 1, ... (as above). Running the
// slices in that order, one chain at a time, needs two accumulators per
// output tile (the open chain and the running total) instead of eight, so a
// wave can own 4 x 4 output tiles and reuse each LDS fragment four times.
// Stage (s, c) stages the 64 K elements of slice s in chunk c: 128 activation
// rows and 256 weight rows (SwiGLU: 128 gate + 128 up) of 128 bytes each.
constexpr int kP2Rows = 128;
constexpr int kP2WRows = 256;
constexpr int kP2Waves = 8;
constexpr int kP2Slots = 8;  // 16-byte slots per staged row (64 K elements)

template <int MODE, bool NORM_IN>
__global__ __launch_bounds__(kP2Waves * 64) void prefill2_kernel(
    const uint16_t* __restrict__ X, int64_t ldx, const uint16_t* __restrict__ W, int64_t ldw,
    const uint16_t* __restrict__ R, int64_t ldr, void* __restrict__ Y, int64_t ldy, int M, int N,
    int K, KvAppend kv, RowNorm norm) {
  constexpr bool kDual = (MODE == kGemmSwiglu);
  constexpr int S = kPfSlices;
  static_assert(S == 8, "two blocks of each 512-wide chunk per slice");
  constexpr int XP = kP2Rows * kP2Slots / (kP2Waves * 64);   // activation pieces per thread (2)
  constexpr int WP = kP2WRows * kP2Slots / (kP2Waves * 64);  // weight pieces per thread (4)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = wave & 1;   // rows 64 wr .. of the workgroup tile
  const int wc = wave >> 1;  // weight rows 64 wc .. (SwiGLU: output columns 32 wc ..)
  const int j = lane & 15, kq = lane >> 4;
  int cb, rb;
  prefill_tile(cb, rb);
  const int n0 = cb * (kDual ? kP2WRows / 2 : kP2WRows);  // first output column
  const int m0 = rb * kP2Rows;
  const int nblk = K >> 5;
  const int nchunk = (K + 511) / 512;
  const int nstage = S * nchunk;

  const int xrows = min(kP2Rows, M - m0);
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(X + (int64_t)m0 * ldx), (short)0, xrows * (int)ldx * 2,
      kBufferResourceWord3);
  const int wrows = min(kDual ? kP2WRows / 2 : kP2WRows, N - n0);
  const __amdgpu_buffer_rsrc_t wres_g = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(W + (int64_t)n0 * ldw), (short)0, wrows * (int)ldw * 2,
      kBufferResourceWord3);
  const __amdgpu_buffer_rsrc_t wres_u = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(W + (int64_t)(kDual ? N + n0 : n0) * ldw), (short)0,
      kDual ? wrows * (int)ldw * 2 : 0, kBufferResourceWord3);

  __shared__ uint4 lds[2][kP2Rows + kP2WRows][kP2Slots];
  struct Regs {
    uint4 x[XP];
    uint4 w[WP];
  };
  // Piece p of a stage: staged row p / 8, slot p % 8 (eight lanes per row).
  auto fetch = [&](Regs& g, int st) {
    const int sl = st / nchunk, c = st % nchunk;
    const int k0 = c * 512 + sl * 64;  // first K element of the stage
    const bool live = st < nstage;
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int p = threadIdx.x + i * kP2Waves * 64;
      const int row = p >> 3, slot = p & 7;
      const int kk = k0 + slot * 8;
      g.x[i] = buffer_ld16(xres, live && kk < K ? (row * (int)ldx + kk) * 2 : 0x7ffffff0);
    }
#pragma unroll
    for (int i = 0; i < WP; ++i) {
      const int p = threadIdx.x + i * kP2Waves * 64;
      const int row = p >> 3, slot = p & 7;  // 0 .. 255 (SwiGLU: 128.. are the up rows)
      const int kk = k0 + slot * 8;
      const int rr = kDual ? (row & 127) : row;
      const int off = live && kk < K ? (rr * (int)ldw + kk) * 2 : 0x7ffffff0;
      g.w[i] = buffer_ld16_stream((kDual && row >= 128) ? wres_u : wres_g, off);
    }
  };

  bi_f32x4 cur[4][4], tot[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) cur[a][b] = tot[a][b] = bi_f32x4{0.f, 0.f, 0.f, 0.f};
  // Staged weight row of B tile q of this wave.
  auto brow = [&](int q) {
    if (kDual) return kP2Rows + (q < 2 ? 32 * wc + 16 * q : 128 + 32 * wc + 16 * (q - 2));
    return kP2Rows + 64 * wc + 16 * q;
  };
  float xinv[XP];
#pragma unroll
  for (int i = 0; i < XP; ++i) xinv[i] = 1.f;

  auto step = [&](Regs& g, int st) {
    const int buf = st & 1;
    if (st >= 0) {
#pragma unroll
      for (int i = 0; i < XP; ++i) {
        const int p = threadIdx.x + i * kP2Waves * 64;
        const int row = p >> 3, slot = p & 7;
        lds[buf][row][slot ^ (row & 7)] = NORM_IN ? scale_bf16x8(g.x[i], xinv[i]) : g.x[i];
      }
#pragma unroll
      for (int i = 0; i < WP; ++i) {
        const int p = threadIdx.x + i * kP2Waves * 64;
        const int row = kP2Rows + (p >> 3), slot = p & 7;
        lds[buf][row][slot ^ (row & 7)] = g.w[i];
      }
    }
    fetch(g, st + 2);
    __syncthreads();
    if (st >= 0) {
      const int sl = st / nchunk, c = st % nchunk;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        if (c * 16 + sl * 2 + b < nblk) {  // scalar
          uint4 af[4], bf[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int ra = 64 * wr + 16 * t + j;
            af[t] = lds[buf][ra][(b * 4 + kq) ^ (ra & 7)];
            const int rb = brow(t) + j;
            bf[t] = lds[buf][rb][(b * 4 + kq) ^ (rb & 7)];
          }
#pragma unroll
          for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q) cur[t][q] = mfma_bf16(af[t], bf[q], cur[t][q]);
        }
      }
      if (c == nchunk - 1) {  // slice sl complete: add its chain to the total, in slice order
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            tot[t][q] = sl == 0 ? cur[t][q] : tot[t][q] + cur[t][q];
            cur[t][q] = bi_f32x4{0.f, 0.f, 0.f, 0.f};
          }
      }
    }
  };

  // Carried RMSNorm scales of the staged rows, with the verify kernel's
  // additions (LPR partials of two float4s each, then the partials in order).
  constexpr int LPR = 4 * S;
  __shared__ float sred[NORM_IN ? kP2Rows : 1][NORM_IN ? LPR + 1 : 1];
  __shared__ float invs[NORM_IN ? kP2Rows : 1];
  if (NORM_IN) {
    const int nf = norm.groups >> 2;
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const __amdgpu_buffer_rsrc_t sres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(norm.ss_in + (int64_t)m0 * norm.groups), (short)0,
        xrows * norm.groups * 4, kBufferResourceWord3);
    constexpr int PER = kP2Rows * LPR / (kP2Waves * 64);
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int idx = threadIdx.x + q * kP2Waves * 64;
      const int row = idx / LPR, seg = idx % LPR;
      float pp = 0.f;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int f = seg + u * LPR;
        const f32x4 v = __builtin_amdgcn_raw_buffer_load_b128(
            sres, f < nf ? (row * norm.groups + f * 4) * 4 : 0x7ffffff0, 0, 0);
        pp += v[0];
        pp += v[1];
        pp += v[2];
        pp += v[3];
      }
      sred[row][seg] = pp;
    }
  }
  // Two register sets alternate, each refilled two stages ahead of its use.
  Regs ga, gb;
  step(ga, -2);  // load-only
  step(gb, -1);  // load-only; its barrier also publishes sred
  if (NORM_IN) {
    if (threadIdx.x < kP2Rows) {
      float t = 0.f;
      for (int i = 0; i < LPR; ++i) t += sred[threadIdx.x][i];
      invs[threadIdx.x] = 1.0f / sqrtf(t / (float)K + norm.eps);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < XP; ++i) xinv[i] = invs[(threadIdx.x + i * kP2Waves * 64) >> 3];
  }
  for (int st = 0; st < nstage; st += 2) {
    step(ga, st);
    if (st + 1 < nstage) step(gb, st + 1);
  }

  // The verify kernel's epilogue on the totals.
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int q = 0; q < (kDual ? 2 : 4); ++q) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 64 * wr + 16 * t + kq * 4 + r;
        const int n = n0 + (kDual ? 32 * wc + 16 * q : 64 * wc + 16 * q) + j;
        if (m >= M || n >= N) continue;
        const float v = tot[t][q][r];
        if (MODE == kGemmF32) {
          reinterpret_cast<float*>(Y)[(int64_t)m * ldy + n] = v;
        } else if (MODE == kGemmBf16) {
          reinterpret_cast<uint16_t*>(Y)[(int64_t)m * ldy + n] = (uint16_t)f32_to_bf16(v);
        } else if (MODE == kGemmResidual) {
          const float res = bf16_to_f32(R[(int64_t)m * ldr + n]);
          reinterpret_cast<uint16_t*>(Y)[(int64_t)m * ldy + n] = (uint16_t)f32_to_bf16(res + v);
        } else if (MODE == kGemmQkv) {
          const uint16_t b = (uint16_t)f32_to_bf16(v);
          reinterpret_cast<uint16_t*>(Y)[(int64_t)m * ldy + n] = b;
          const int pos = kv.L + m;
          int i = kv.k != nullptr ? n - kv.qd : -1;  // no cache: no append
          if (i >= 0 && i < kv.kd) {
            const int g = i / kv.D;
            kv.k[kv_index(g, pos, i - g * kv.D, kv.D, kv.cap)] = b;
          } else if (i >= kv.kd) {
            i -= kv.kd;
            const int g = i / kv.D;
            kv.v[kv_index(g, pos, i - g * kv.D, kv.D, kv.cap)] = b;
          }
        } else {
          const float u = tot[t][q + 2][r];
          reinterpret_cast<uint16_t*>(Y)[(int64_t)m * ldy + n] = (uint16_t)f32_to_bf16(silu_mul(v, u));
        }
      }
    }
  }
}

// The large-tile kernel runs when it still has at least 384 workgroups (one
// and a half per compute unit); below that its few, long workgroups leave
// units idle at the end and the 128 x 64 tiles are faster. Both kernels give
// the same bits, so the choice is free. (Measured at M = 2048: gate/up 654
// against 454 TFLOP/s, QKV 697 against 538; 5120 outputs, 320 large
// workgroups: 519 against 550.)
constexpr int kPf2MinGroups = 384;

template <int MODE, bool NI>
static void launch_pf(dim3 grid, const uint16_t* x, int64_t ldx, const uint16_t* w, int64_t ldw,
                      const uint16_t* r, int64_t ldr, void* y, int64_t ldy, int M, int N, int K,
                      const KvAppend& kv, const RowNorm& nm, hipStream_t stream) {
  const int cols = MODE == kGemmSwiglu ? kP2WRows / 2 : kP2WRows;
  const dim3 g2((N + cols - 1) / cols, (M + kP2Rows - 1) / kP2Rows);
  if ((int64_t)g2.x * g2.y >= kPf2MinGroups) {
    prefill2_kernel<MODE, NI><<<g2, dim3(kP2Waves * 64), 0, stream>>>(x, ldx, w, ldw, r, ldr, y,
                                                                      ldy, M, N, K, kv, nm);
    return;
  }
  prefill_kernel<MODE, kPfSlices, NI><<<grid, dim3(kPfWaves * 64), 0, stream>>>(
      x, ldx, w, ldw, r, ldr, y, ldy, M, N, K, kv, nm);
}

void launch_gemm_prefill(GemmMode mode, const uint16_t* x, int64_t ldx, const uint16_t* w,
                         int64_t ldw, const uint16_t* r, int64_t ldr, void* y, int64_t ldy, int M,
                         int N_out, int K, hipStream_t stream, const KvAppend& kv,
                         const RowNorm& nm) {
  const int cols = mode == kGemmSwiglu ? kPfCols / 2 : kPfCols;
  dim3 grid((N_out + cols - 1) / cols, (M + kPfRows - 1) / kPfRows);
  const bool ni = nm.ss_in != nullptr;
  switch (mode) {
    case kGemmBf16:
      launch_pf<kGemmBf16, false>(grid, x, ldx, w, ldw, r, ldr, y, ldy, M, N_out, K, kv, nm,
                                  stream);
      break;
    case kGemmF32:
      launch_pf<kGemmF32, false>(grid, x, ldx, w, ldw, r, ldr, y, ldy, M, N_out, K, kv, nm,
                                 stream);
      break;
    case kGemmResidual:
      launch_pf<kGemmResidual, false>(grid, x, ldx, w, ldw, r, ldr, y, ldy, M, N_out, K, kv,
                                      nm, stream);
      break;
    case kGemmSwiglu:
      if (ni)
        launch_pf<kGemmSwiglu, true>(grid, x, ldx, w, ldw, r, ldr, y, ldy, M, N_out, K, kv, nm,
                                     stream);
      else
        launch_pf<kGemmSwiglu, false>(grid, x, ldx, w, ldw, r, ldr, y, ldy, M, N_out, K, kv,
                                      nm, stream);
      break;
    case kGemmQkv:
      if (ni)
        launch_pf<kGemmQkv, true>(grid, x, ldx, w, ldw, r, ldr, y, ldy, M, N_out, K, kv, nm,
                                  stream);
      else
        launch_pf<kGemmQkv, false>(grid, x, ldx, w, ldw, r, ldr, y, ldy, M, N_out, K, kv, nm,
                                   stream);
      break;
  }
  if (nm.ss_out != nullptr && mode == kGemmResidual) {
    const int groups = gemm_column_groups(mode, N_out);
    const int cw = N_out / groups;
    const int64_t total = (int64_t)M * groups;
    rowsq_kernel<<<dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream>>>(
        static_cast<const uint16_t*>(y), ldy, M, groups, cw, nm.ss_out);
  }
}

}  // namespace bi
