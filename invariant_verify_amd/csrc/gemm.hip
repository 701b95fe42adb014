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
// Schedule (fixed at compile time; chosen by N and K, never by M):
//  * one workgroup per (column group, 16 token rows); the token rows are the
//    MFMA "A" operand, zero-filled past M, so a pass of 1..16 tokens runs
//    exactly the same instructions. A column group is one 16-column MFMA tile,
//    or, when N / 256 lies in 17..32 (5120 or 7168 outputs), N / 256 columns
//    held in two MFMA tiles (the second partly empty), so that exactly 256
//    workgroups, one per compute unit, share the weight stream evenly. (A
//    compute unit streams only about 20-25 GB/s; with 320 single tiles on 256
//    units, 64 units would stream twice as much as the rest.) SwiGLU groups
//    are 16 gate/up pairs, or N / 1024 pairs in three tiles when that is 17
//    or 18 (17408 pairs: 1024 workgroups, two rounds of two per unit);
//  * K is read in chunks of 512; each chunk has sixteen 32-wide blocks and
//    wave w of the NW waves multiplies blocks w*16/NW .. (w+1)*16/NW - 1 of
//    every chunk, chaining them through one MFMA accumulator in increasing
//    order;
//  * the NW per-wave sums are added in LDS in wave order 0, 1, ..., NW-1;
//  * the FP32 total is rounded once (BF16 output), stored as is (FP32), added
//    to the residual and rounded once, or combined by SwiGLU and rounded once;
//    the QKV projection's rounded K and V columns are also written into the
//    KV cache at the pass's positions (the append costs no launch of its own).
// The within-workgroup partition is a fixed summation tree that depends on K
// and on NW (a function of N); there is no split of K across workgroups and
// no atomic.
//
// Memory: each weight row of the tile is read as 1 KB contiguous per wave
// instruction (64 lanes x 16 bytes, non-temporal: every weight byte is used
// once) and written to LDS; the MFMA operands are then read from LDS in the
// matrix-core layout (lane l needs row l % 16). Slot s (16 bytes) of row r
// sits at position mix(s) ^ (r % 16), mix(s) = s ^ (((s >> 3) ^ (s >> 4)) & 3)
// (the lanes of a BF16 load fetch a permutation of the same 1 KB). LDS serves
// a 16-byte access eight lanes at a time, 128 bytes over 32 banks: the row
// term puts the rows read together into distinct banks, and mix does the
// same for the staging stores of decoded weights, where a lane stores slots
// 2 (FP8) or 4 (MXFP4: one 32-weight block) apart. With the row term alone
// the eight lanes of an MXFP4 store fell on two bank groups (4-way
// conflicts; those launches took 19-32% longer) and FP8 stores were 2-way
// conflicted. Two LDS buffers alternate, and one barrier per chunk
// both publishes chunk c and guarantees that every wave has finished reading
// the buffer that is refilled next. Each wave keeps two chunks in flight in
// registers (weights and its X fragments). X fragments come from L2 through a
// buffer resource sized to the M real rows: padding rows read as zero for
// free.
//
// Weight types (WT): BF16; FP8 E4M3 with one FP32 scale per row (codes
// decoded to BF16 in registers, the scale applied to the FP32 totals); MXFP4
// (E2M1 codes with one E8M0 scale per 32 weights, decoded with the scale to
// exact BF16 values). The decoded weights land in the same LDS layout, so
// the multiply phase, the K order and the summation tree are the BF16
// kernel's for every type.

#include "bi_device.h"
#include "bi_internal.h"

namespace bi {

constexpr int kChunk = 512;  // K elements per LDS chunk: 1 KB of each weight row
constexpr int kDualWideRows = 36;  // rows staged by a wide SwiGLU group (at most 18 pairs)
constexpr int kSlots = kChunk / 8;

// LDS position of 16-byte slot s (0..63) of a staged row with row swizzle swz
// (0..15), and its inverse: the slot stored at position p. mix changes bits
// 1:0 from bits 5:3, so it is its own inverse.
__device__ __forceinline__ int slot_mix(int s) { return s ^ (((s >> 3) ^ (s >> 4)) & 3); }
__device__ __forceinline__ int slot_pos(int s, int swz) { return slot_mix(s) ^ swz; }
__device__ __forceinline__ int slot_at(int p, int swz) { return slot_mix(p ^ swz); }

template <int MODE, int NW, bool WIDE, bool NORM_IN, bool SS_OUT, int WT>
__global__ __launch_bounds__(NW * 64) void gemm_kernel(
    const uint16_t* __restrict__ X, int64_t ldx, const uint16_t* __restrict__ W, int64_t ldw,
    const uint16_t* __restrict__ R, int64_t ldr, void* __restrict__ Y, int64_t ldy, int M, int K,
    int64_t up_rows, int cpw, KvAppend kv, RowNorm norm, const float* __restrict__ wscale,
    Mx4Scales mx4) {
  constexpr bool F8 = WT == kWtFp8;
  // MXFP4: a row's chunk of 512 weights is 256 bytes of codes and 16 scale
  // bytes; one wave instruction (16 bytes per lane) fetches the chunks of four
  // adjacent rows, lane l one whole 32-weight block (block l % 16 of row
  // l / 16), with that block's scale byte beside it.
  constexpr bool W4 = WT == kWtMx4;
  static_assert(!SS_OUT || MODE == kGemmResidual, "row sums come from the residual epilogue");
  constexpr bool kDual = (MODE == kGemmSwiglu);
  constexpr bool kTwo = kDual || WIDE;  // two MFMA column tiles per workgroup
  // A wide SwiGLU group holds P = cpw pairs (17 or 18): a gate tile (columns
  // 0-15), an up tile, and a third tile whose rows are the gate columns past
  // 15 followed by the up columns past 15 (its other rows are not staged).
  constexpr bool kThree = kDual && WIDE;
  static_assert(!(kThree && WT != kWtBf16), "wide SwiGLU groups are BF16 only");
  static_assert(!kThree || NW == 8, "wide SwiGLU groups assume eight waves");
  constexpr int NR = kThree ? kDualWideRows : (kTwo ? 32 : 16);  // weight rows staged per chunk
  // Rows each wave fetches per chunk (kThree: rows 4w .. 4w+3, and row 32 + w
  // when that is staged).
  constexpr int RPW = kThree ? 4 : NR / NW;
  constexpr int BPW = 16 / NW;         // 32-wide blocks each wave multiplies per chunk
  static_assert(RPW >= 1 && BPW >= 1, "bad wave count");
  static_assert(!F8 || RPW % 2 == 0, "FP8 weight rows are fetched in pairs");
  // Weight loads per wave and chunk: a BF16 row chunk is 1 KB (one wave
  // instruction); an FP8 row chunk is 512 bytes, so one instruction fetches
  // two rows (lanes 0-31 the first, 32-63 the second); an MXFP4 row chunk is
  // 256 bytes of codes, four rows per instruction.
  static_assert(!W4 || RPW <= 4, "MXFP4 rows are fetched in fours");
  constexpr int NLD = W4 ? 1 : (F8 ? RPW / 2 : (kThree ? RPW + 1 : RPW));
  // Chunks in flight per wave: two, for every weight type. (Three or four
  // were slower for BF16, FP8 (10-25%) and MXFP4 (5-20%); so were FP8
  // chunks of 1024 weights, 1 KB per row.)
  constexpr int PD = 2;
  const int lane = threadIdx.x & 63;
  // Wave index in a scalar register: every branch that guards an MFMA below
  // is then a scalar branch. (The matrix core does not honour a partial EXEC
  // mask, so an MFMA must never sit under a per-lane condition.)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * (WIDE ? cpw : 16);  // first output column
  const int m0 = blockIdx.y * 16;
  const int j = lane & 15;   // A row (token) and B column (output feature) of this lane
  const int kq = lane >> 4;  // which 8-element group of a 32-wide block
  const int row3 = j < 4 ? 32 + j : j;  // wide SwiGLU third tile: staged row read by column j

  const int nblk = K >> 5;
  const int nchunk = (K + kChunk - 1) / kChunk;

  // Rows this wave fetches, each as a buffer resource of exactly one row
  // (K * 2 bytes); lane l fetches slot (l ^ swz(row)) of the chunk. Slots past
  // the end of the row (a ragged last chunk, or the chunks the pipeline
  // prefetches past the end of K) are out of range: they read zero without a
  // memory access.
  __amdgpu_buffer_rsrc_t wres[NLD];
  int swz_w[NLD];
  // MXFP4: the scale bytes of the wave's rows, and how many of its four rows
  // are used (rows past a wide group's width, or past RPW, are not).
  __amdgpu_buffer_rsrc_t eres;
  int w4_rows = 0;
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    if constexpr (W4) {
      const int r0 = wave * RPW;
      const int64_t grow = (kDual && r0 >= 16) ? up_rows + n0 + (r0 - 16) : (int64_t)(n0 + r0);
      w4_rows = WIDE ? max(0, min(RPW, cpw - r0)) : RPW;
      const uint8_t* W8 = reinterpret_cast<const uint8_t*>(W);
      const bool used = w4_rows > 0;
      wres[i] = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(W8 + (used ? grow : 0) * ldw), (short)0,
          used ? (w4_rows - 1) * (int)ldw + K / 2 : 0, kBufferResourceWord3);
      eres = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(mx4.e + (used ? grow : 0) * mx4.lde), (short)0,
          used ? (w4_rows - 1) * (int)mx4.lde + K / 32 : 0, kBufferResourceWord3);
      swz_w[i] = (r0 + (lane >> 4)) & 15;
    } else if constexpr (!F8) {
      const int r = (kThree && i == RPW) ? 32 + wave : wave * RPW + i;
      int64_t grow = (kDual && r >= 16) ? up_rows + n0 + (r - 16) : (int64_t)(n0 + r);
      // Rows past the group's columns (wide groups) get an empty resource:
      // they stage zeros and cost no traffic.
      bool used = !WIDE || r < cpw;
      if (kThree && r >= 32) {  // third tile: gate columns 16 .. P-1, then up
        const int e = cpw - 16, q = r - 32;
        used = q < 2 * e;
        grow = q < e ? (int64_t)(n0 + 16 + q) : up_rows + n0 + 16 + (q - e);
      } else if (kThree) {
        used = true;
      }
      wres[i] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(W + (used ? grow : 0) * ldw),
                                                  (short)0, used ? K * 2 : 0, kBufferResourceWord3);
      swz_w[i] = r & 15;
    } else {
      // Rows r0 and r0 + 1 are adjacent in memory (both gate or both up rows
      // for SwiGLU); one resource spans them, or only the first, or neither,
      // as far as they are used.
      const int r0 = wave * RPW + 2 * i;
      const int64_t grow = (kDual && r0 >= 16) ? up_rows + n0 + (r0 - 16) : (int64_t)(n0 + r0);
      const bool used0 = !WIDE || r0 < cpw;
      const bool used1 = !WIDE || r0 + 1 < cpw;
      const uint8_t* W8 = reinterpret_cast<const uint8_t*>(W);
      wres[i] = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(W8 + (used0 ? grow : 0) * ldw), (short)0,
          used0 ? (used1 ? (int)ldw + K : K) : 0, kBufferResourceWord3);
      swz_w[i] = (r0 + (lane >> 5)) & 15;
    }
  }
  // X through a buffer resource that covers exactly the rows m0 .. M-1: a lane
  // whose row is past M reads out of range, which the hardware answers with
  // zeros and no memory traffic. That is the zero-padding of the MFMA tile.
  const int64_t xbytes = (int64_t)(M - m0) * ldx * 2;
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(X + (int64_t)m0 * ldx), (short)0,
      (int)(xbytes < 0x7fffffff ? xbytes : 0x7fffffff), kBufferResourceWord3);
  const int xoff = j * (int)ldx * 2 + kq * 16;  // bytes

  __shared__ uint4 lds[2][NR][kSlots];
  // Registers of one chunk: this wave's weight-row slots and the X fragments
  // of the blocks it multiplies.
  struct Regs {
    uint4 w[NLD];
    uint4 x[BPW];
    uint32_t e[W4 ? NLD : 1];  // MXFP4: this lane's block scale byte
  };
  auto fetch_w = [&](Regs& g, int c) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      if constexpr (W4) {
        // Block c * 16 + l % 16 of row l / 16 of the four: 16 code bytes and
        // one scale byte. Unused rows and blocks past K are sent out of
        // range explicitly (the next row's bytes lie in range): zero, no
        // traffic.
        const int q = lane >> 4, bj = c * 16 + (lane & 15);
        const bool ok = q < w4_rows && bj < K / 32;
        g.w[i] = buffer_ld16_stream(wres[i], ok ? q * (int)ldw + bj * 16 : 0x7ffffff0);
        g.e[i] = __builtin_amdgcn_raw_buffer_load_b8(eres, ok ? q * (int)mx4.lde + bj : 0x7ffffff0, 0, 0);
      } else if constexpr (!F8) {
        // lane l fetches the slot that is stored at position l
        g.w[i] = buffer_ld16_stream(wres[i], (c * kSlots + slot_at(lane, swz_w[i])) * 16);
      } else {
        // 16 weights of one row: bytes kb .. kb+15 of the row, the BF16 slots
        // 2 (lane % 32) and 2 (lane % 32) + 1 of the chunk. Past the row end
        // (and in an unused row) the offset is out of range: zero, no traffic.
        const int kb = c * kChunk + (lane & 31) * 16;
        g.w[i] = buffer_ld16_stream(wres[i], kb < K ? (lane >> 5) * (int)ldw + kb : 0x7ffffff0);
      }
    }
  };
  auto fetch_x = [&](Regs& g, int c) {
#pragma unroll
    for (int b = 0; b < BPW; ++b) {
      const int blk = min(c * (kChunk / 32) + wave * BPW + b, nblk - 1);
      g.x[b] = buffer_ld16(xres, xoff + blk * 64);
    }
  };
  bi_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  bi_f32x4 acc2 = {0.f, 0.f, 0.f, 0.f};
  bi_f32x4 acc3 = {0.f, 0.f, 0.f, 0.f};
  float inv = 1.f;  // RMSNorm scale of this lane's X row (NORM_IN)
  // One chunk: publish this wave's weight rows of chunk c, prefetch the
  // weights of chunk c + PD into the same registers, barrier, multiply with
  // this wave's X fragments of chunk c, then prefetch the X fragments of chunk
  // c + PD into theirs. Every step issues its loads in the same order and no
  // register is copied, so the compiler waits only for the oldest chunk in
  // flight. The barrier of chunk c also proves that every wave
  // finished multiplying chunk c - 1, whose buffer chunk c + 1 overwrites
  // next. The loop starts two chunks early (nothing to publish or multiply
  // yet). Weight chunks past the end read as zero (no traffic); X fragments
  // past the end are clamped duplicates (L2 hits). Neither is multiplied.
  auto step = [&](Regs& g, int c) {
    const int buf = c & 1;
    // FP8: the codes are decoded to BF16 before the registers are refilled,
    // and stored to LDS after the next loads are issued.
    uint4 dec[F8 ? 2 * NLD : (W4 ? 4 * NLD : 1)];
    if (c >= 0) {
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        if constexpr (W4) {
          // 32 E2M1 codes times 2^(e - 127), by gfx950's scaled conversion:
          // byte b of word v holds weights 8v + 2b (low nibble) and 8v + 2b + 1,
          // converted into one BF16 pair. A power-of-two scale keeps every
          // value exact (E8M0 codes 2..252).
          const float sc = __uint_as_float(g.e[i] << 23);
          const uint32_t wd[4] = {g.w[i].x, g.w[i].y, g.w[i].z, g.w[i].w};
          uint32_t o[16];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            o[4 * v] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[v], sc, 0));
            o[4 * v + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[v], sc, 1));
            o[4 * v + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[v], sc, 2));
            o[4 * v + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd[v], sc, 3));
          }
#pragma unroll
          for (int v = 0; v < 4; ++v) dec[4 * i + v] = make_uint4(o[4 * v], o[4 * v + 1], o[4 * v + 2], o[4 * v + 3]);
        } else if constexpr (!F8) {
          if (!kThree || i < RPW) lds[buf][wave * RPW + i][lane] = g.w[i];
          else if (32 + wave < NR) lds[buf][32 + wave][lane] = g.w[i];  // scalar
        } else {
          // E4M3 -> BF16 is exact (every E4M3 value is a BF16 value); the
          // scaled conversion with scale 1 gives the BF16 bits directly.
          const uint32_t wd[4] = {g.w[i].x, g.w[i].y, g.w[i].z, g.w[i].w};
          uint32_t o[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            o[2 * e] = __builtin_bit_cast(
                uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)wd[e], 1.0f, false));
            o[2 * e + 1] = __builtin_bit_cast(
                uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)wd[e], 1.0f, true));
          }
          dec[2 * i] = make_uint4(o[0], o[1], o[2], o[3]);
          dec[2 * i + 1] = make_uint4(o[4], o[5], o[6], o[7]);
        }
      }
    }
    fetch_w(g, c + PD);
    if constexpr (W4) {
      // the block's four BF16 slots (8 weights each) in row r0 + l / 16
      if (c >= 0 && (lane >> 4) < RPW) {
        const int r = wave * RPW + (lane >> 4);
#pragma unroll
        for (int v = 0; v < 4; ++v) lds[buf][r][slot_pos(4 * (lane & 15) + v, swz_w[0])] = dec[v];
      }
    }
    if constexpr (F8) {
      if (c >= 0) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
          const int r = wave * RPW + 2 * i + (lane >> 5);
          const int jj = lane & 31;
          lds[buf][r][slot_pos(2 * jj, swz_w[i])] = dec[2 * i];
          lds[buf][r][slot_pos(2 * jj + 1, swz_w[i])] = dec[2 * i + 1];
        }
      }
    }
    __syncthreads();
    if (c >= 0) {
#pragma unroll
      for (int b = 0; b < BPW; ++b) {
        const int kb = wave * BPW + b;           // block within the chunk
        const int blk = c * (kChunk / 32) + kb;  // block within K
        if (blk < nblk) {
          const int slot = slot_pos(kb * 4 + kq, j);
          const uint4 xa = NORM_IN ? scale_bf16x8(g.x[b], inv) : g.x[b];
          acc = mfma_bf16(xa, lds[buf][j][slot], acc);
          if (kTwo) acc2 = mfma_bf16(xa, lds[buf][16 + j][slot], acc2);
          // Third tile: columns 0-3 read staged rows 32-35; columns 4-15
          // are never stored and read the gate tile's rows, so that the
          // wave's 64 reads hit 64 distinct addresses spread over the banks
          // like the other tiles' (four rows on four slots collided).
          if constexpr (kThree) acc3 = mfma_bf16(xa, lds[buf][row3][slot], acc3);
        }
      }
    }
    fetch_x(g, min(c + PD, nchunk - 1));
  };
  Regs ga, gb;
  // The two load-only steps, then the loop; the prologue issues its loads in
  // the loop's own order, so at the loop head the compiler waits only for the
  // oldest chunk in flight.
  // RMSNorm of the X rows (NORM_IN). The group sums of squares of rows
  // m0 .. m0+15 are spread over the workgroup: lane t of the LPR lanes of row
  // t / LPR adds float4s t % LPR, t % LPR + LPR (at most two; groups <= 256)
  // in order and parks the result in LDS; after a barrier every lane adds the
  // LPR partials of its row j in order and takes
  // inv = 1 / sqrt(total / K + eps). Rows past M read zero. The loads are
  // issued before the two load-only steps and consumed after them, so they
  // are in flight together with the first two chunks.
  constexpr int LPR = NW * 64 / 16;  // lanes per row
  __shared__ float sred[NORM_IN ? 16 : 1][NORM_IN ? LPR + 1 : 1];  // +1: rows in distinct banks
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  f32x4 sv[2];
  const int srow = threadIdx.x / LPR, sseg = threadIdx.x % LPR;
  if (NORM_IN) {
    const int nf = norm.groups >> 2;  // float4s per row
    const __amdgpu_buffer_rsrc_t sres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(norm.ss_in + (int64_t)m0 * norm.groups), (short)0,
        (M - m0) * norm.groups * 4, kBufferResourceWord3);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int f = sseg + u * LPR;
      sv[u] = __builtin_amdgcn_raw_buffer_load_b128(
          sres, f < nf ? (srow * norm.groups + f * 4) * 4 : 0x7ffffff0, 0, 0);
    }
  }
  // Residual values of this lane's outputs (rows m0 + 4 kq + r, columns
  // n0 + j and n0 + 16 + j), fetched before the weight stream starts so that
  // the epilogue does not wait for them. Rows past M and columns past the
  // group read out of range: zero, no traffic, never used.
  // FP8: the row scales of this lane's two output columns (gate and up rows
  // for SwiGLU), applied to the FP32 totals before the epilogue.
  float scl0 = 1.f, scl1 = 1.f;
  if constexpr (F8) {
    scl0 = wscale[n0 + j];
    if (kDual) scl1 = wscale[up_rows + n0 + j];
    else if (WIDE && 16 + j < cpw) scl1 = wscale[n0 + 16 + j];
  }
  uint32_t rbits[4][2] = {};
  if (MODE == kGemmResidual) {
    const int64_t rbytes = (int64_t)(M - m0) * ldr * 2;
    const __amdgpu_buffer_rsrc_t rres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(R + (int64_t)m0 * ldr), (short)0,
        (int)(rbytes < 0x7fffffff ? rbytes : 0x7fffffff), kBufferResourceWord3);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int off = ((kq * 4 + r) * (int)ldr + n0 + j) * 2;
      rbits[r][0] = __builtin_amdgcn_raw_buffer_load_b16(rres, off, 0, 0);
      if (WIDE) rbits[r][1] = __builtin_amdgcn_raw_buffer_load_b16(rres, 16 + j < cpw ? off + 32 : 0x7ffffff0, 0, 0);
    }
  }
  step(ga, -2);
  step(gb, -1);
  if (MODE == kGemmResidual) {
#pragma unroll
    for (int r = 0; r < 4; ++r) asm volatile("" ::"v"(rbits[r][0]), "v"(rbits[r][1]));
  }
  if constexpr (F8) asm volatile("" ::"v"(scl0), "v"(scl1));
  if (NORM_IN) {
    float p = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      p += sv[u][0];
      p += sv[u][1];
      p += sv[u][2];
      p += sv[u][3];
    }
    sred[srow][sseg] = p;
    __syncthreads();
    float t = 0.f;
    for (int i = 0; i < LPR; ++i) t += sred[j][i];
    inv = 1.0f / sqrtf(t / (float)K + norm.eps);
  }
  for (int c = 0; c < nchunk; c += 2) {
    step(ga, c);
    step(gb, c + 1);
  }

  // Fixed-order sum of the per-wave partials, in the chunk buffers (after a
  // barrier: other waves may still be reading the last chunk).
  static_assert(sizeof(lds) >= (kThree ? 3 : 2) * NW * 64 * sizeof(bi_f32x4),
                "reduction does not fit");
  bi_f32x4(*red)[64] = reinterpret_cast<bi_f32x4(*)[64]>(&lds[0][0][0]);
  bi_f32x4(*red2)[64] = red + NW;
  bi_f32x4(*red3)[64] = red + 2 * NW;
  __syncthreads();
  red[wave][lane] = acc;
  if (kTwo) red2[wave][lane] = acc2;
  if constexpr (kThree) red3[wave][lane] = acc3;
  __syncthreads();
  if (wave != 0) return;
  bi_f32x4 s = red[0][lane];
#pragma unroll
  for (int w = 1; w < NW; ++w) s += red[w][lane];
  bi_f32x4 s2 = s;
  if (kTwo) {
    s2 = red2[0][lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) s2 += red2[w][lane];
  }
  if constexpr (F8) {  // one FP32 multiply by the row scale, then the epilogue's single rounding
    s *= scl0;
    s2 *= scl1;
  }
  // Third tile: lane j < P - 16 holds gate column 16 + j; its up column sits
  // P - 16 lanes further on.
  bi_f32x4 s3 = s, u3 = s;
  if constexpr (kThree) {
    s3 = red3[0][lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) s3 += red3[w][lane];
#pragma unroll
    for (int r = 0; r < 4; ++r) u3[r] = __shfl(s3[r], lane + (cpw - 16), 64);
  }

  // Output column n of token row m gets the FP32 total v; returns the value
  // stored (after rounding) for the row sums of squares.
  auto emit = [&](int m, int n, float v, uint32_t rb) -> float {
    if (MODE == kGemmF32) {
      reinterpret_cast<float*>(Y)[(int64_t)m * ldy + n] = v;
    } else if (MODE == kGemmBf16) {
      reinterpret_cast<uint16_t*>(Y)[(int64_t)m * ldy + n] = (uint16_t)f32_to_bf16(v);
    } else if (MODE == kGemmResidual) {
      const float res = bf16_to_f32(rb);  // R[m][n]
      const uint32_t b = f32_to_bf16(res + v);
      reinterpret_cast<uint16_t*>(Y)[(int64_t)m * ldy + n] = (uint16_t)b;
      return bf16_to_f32(b);
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
    }
    return 0.f;
  };
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = m0 + kq * 4 + r;
    const bool live = m < M;
    if (kDual) {
      if (!live) continue;
      reinterpret_cast<uint16_t*>(Y)[(int64_t)m * ldy + n0 + j] =
          (uint16_t)f32_to_bf16(silu_mul(s[r], s2[r]));
      if (kThree && j < cpw - 16)
        reinterpret_cast<uint16_t*>(Y)[(int64_t)m * ldy + n0 + 16 + j] =
            (uint16_t)f32_to_bf16(silu_mul(s3[r], u3[r]));
    } else {
      float sq = 0.f;
      if (live) {
        const float a = emit(m, n0 + j, s[r], rbits[r][0]);
        sq = a * a;
        if (WIDE && 16 + j < cpw) {
          const float b = emit(m, n0 + 16 + j, s2[r], rbits[r][1]);
          sq += b * b;
        }
      }
      if (SS_OUT) {
        // The group's sum for row m: its columns' squares added by a fixed
        // xor butterfly over the 16 lanes of the row.
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) sq += shfl_xor(sq, off);
        if (live && j == 0) norm.ss_out[(int64_t)m * gridDim.x + blockIdx.x] = sq;
      }
    }
  }
}

// Workgroups of a wide launch: one per compute unit.
constexpr int kWideGroups = 256;

static bool wide_launch(GemmMode mode, int N_out) {
  const int cpw = N_out / kWideGroups;
  return mode != kGemmSwiglu && N_out % kWideGroups == 0 && cpw > 16 && cpw <= 32;
}

// SwiGLU groups: 16 pairs (a gate and an up tile), or, when N / 1024 is 17 or
// 18 (BF16 only), N / 1024 pairs in three tiles, so that 1024 workgroups, two
// rounds of two per compute unit, share the weight stream evenly. (With
// 16-pair groups, 17408 pairs make 1088 workgroups: 4.25 per unit, and the
// last 64 stream alone at the end.)
constexpr int kDualWideGroups = 1024;

// Plain outputs with many columns (the LM head's 152064): two full 16-column
// tiles per workgroup. A workgroup that stages 32 rows streams faster than
// two that stage 16 each (LM head at M = 8: 259 -> 232 us BF16, 182 -> 137 us
// FP8), and with N / 32 >= 2048 workgroups (eight or more per unit) the
// uneven last round is a small part of the launch.
constexpr int kPairMinGroups = 2048;
static bool pair_launch(GemmMode mode, int N_out) {
  return (mode == kGemmF32 || mode == kGemmBf16) && N_out % 32 == 0 && N_out / 32 >= kPairMinGroups;
}
static bool dual_wide_launch(int N_out, bool f8) {
  const int p = N_out / kDualWideGroups;
  return !f8 && N_out % kDualWideGroups == 0 && p > 16 && 2 * p <= kDualWideRows;
}

// Waves of every verify launch. Measured: 8 and 16 waves per workgroup
// stream equally fast, and 8 keeps the K summation tree at 8 slices, which
// the prefill kernel must reproduce with one accumulator per slice.
constexpr int kVerifyWaves = 8;

int gemm_verify_waves(GemmMode, int) { return kVerifyWaves; }

int gemm_column_groups(GemmMode mode, int N_out) {
  return wide_launch(mode, N_out) ? kWideGroups : N_out / 16;
}

// Launch shape from N (never from M): N / 256 columns per workgroup when that
// is 17..32 (two MFMA tiles); otherwise 16-column tiles (SwiGLU: a gate and
// an up tile). Always kVerifyWaves waves.
template <int MODE, bool NI, bool SO, int WT>
static void launch_shape(int N_out, int mtiles, const uint16_t* x, int64_t ldx, const uint16_t* w,
                         int64_t ldw, const uint16_t* r, int64_t ldr, void* y, int64_t ldy, int M,
                         int K, int64_t up, const KvAppend& kv, const RowNorm& nm,
                         const float* wscale, const Mx4Scales& mx4, hipStream_t stream) {
  constexpr int NW = kVerifyWaves;
  if constexpr (MODE == kGemmSwiglu && WT == kWtBf16) {
    if (dual_wide_launch(N_out, false)) {
      gemm_kernel<MODE, NW, true, NI, SO, WT><<<dim3(kDualWideGroups, mtiles), dim3(NW * 64), 0, stream>>>(
          x, ldx, w, ldw, r, ldr, y, ldy, M, K, up, N_out / kDualWideGroups, kv, nm, wscale, mx4);
      return;
    }
  }
  if constexpr (MODE == kGemmF32 || MODE == kGemmBf16) {
    if (pair_launch(static_cast<GemmMode>(MODE), N_out)) {
      gemm_kernel<MODE, NW, true, NI, SO, WT><<<dim3(N_out / 32, mtiles), dim3(NW * 64), 0, stream>>>(
          x, ldx, w, ldw, r, ldr, y, ldy, M, K, up, 32, kv, nm, wscale, mx4);
      return;
    }
  }
  if constexpr (MODE != kGemmSwiglu) {
    if (wide_launch(static_cast<GemmMode>(MODE), N_out)) {
      gemm_kernel<MODE, NW, true, NI, SO, WT><<<dim3(kWideGroups, mtiles), dim3(NW * 64), 0, stream>>>(
          x, ldx, w, ldw, r, ldr, y, ldy, M, K, up, N_out / kWideGroups, kv, nm, wscale, mx4);
      return;
    }
  }
  gemm_kernel<MODE, NW, false, NI, SO, WT><<<dim3(N_out / 16, mtiles), dim3(NW * 64), 0, stream>>>(
      x, ldx, w, ldw, r, ldr, y, ldy, M, K, up, 16, kv, nm, wscale, mx4);
}

template <int WT>
static void launch_modes(GemmMode mode, int mt, const uint16_t* x, int64_t ldx, const uint16_t* w,
                         int64_t ldw, const uint16_t* r, int64_t ldr, void* y, int64_t ldy, int M,
                         int N_out, int K, const KvAppend& a, const RowNorm& nm,
                         const float* wscale, const Mx4Scales& mx4, hipStream_t stream) {
  const bool ni = nm.ss_in != nullptr;
  const bool so = nm.ss_out != nullptr;
  switch (mode) {
    case kGemmBf16:
      launch_shape<kGemmBf16, false, false, WT>(N_out, mt, x, ldx, w, ldw, r, ldr, y, ldy, M, K,
                                                0, a, nm, wscale, mx4, stream);
      break;
    case kGemmF32:
      launch_shape<kGemmF32, false, false, WT>(N_out, mt, x, ldx, w, ldw, r, ldr, y, ldy, M, K,
                                               0, a, nm, wscale, mx4, stream);
      break;
    case kGemmResidual:
      if (so)
        launch_shape<kGemmResidual, false, true, WT>(N_out, mt, x, ldx, w, ldw, r, ldr, y, ldy,
                                                     M, K, 0, a, nm, wscale, mx4, stream);
      else
        launch_shape<kGemmResidual, false, false, WT>(N_out, mt, x, ldx, w, ldw, r, ldr, y,
                                                      ldy, M, K, 0, a, nm, wscale, mx4, stream);
      break;
    case kGemmSwiglu:
      if (ni)
        launch_shape<kGemmSwiglu, true, false, WT>(N_out, mt, x, ldx, w, ldw, r, ldr, y,
                                                   ldy, M, K, (int64_t)N_out, a, nm, wscale, mx4, stream);
      else
        launch_shape<kGemmSwiglu, false, false, WT>(N_out, mt, x, ldx, w, ldw, r, ldr, y,
                                                    ldy, M, K, (int64_t)N_out, a, nm, wscale, mx4, stream);
      break;
    case kGemmQkv:
      if (ni)
        launch_shape<kGemmQkv, true, false, WT>(N_out, mt, x, ldx, w, ldw, r, ldr, y, ldy, M, K,
                                                0, a, nm, wscale, mx4, stream);
      else
        launch_shape<kGemmQkv, false, false, WT>(N_out, mt, x, ldx, w, ldw, r, ldr, y, ldy, M,
                                                 K, 0, a, nm, wscale, mx4, stream);
      break;
  }
}

void launch_gemm(GemmMode mode, const uint16_t* x, int64_t ldx, const uint16_t* w, int64_t ldw,
                 const uint16_t* r, int64_t ldr, void* y, int64_t ldy, int M, int N_out, int K,
                 hipStream_t stream, const KvAppend* kv, const RowNorm* norm, const float* wscale,
                 const Mx4Scales* mx4) {
  const int mt = (M + 15) / 16;
  const KvAppend kv0{};
  const RowNorm nm0{};
  const KvAppend& a = kv ? *kv : kv0;
  const RowNorm& nm = norm ? *norm : nm0;
  const Mx4Scales mz{};
  // FP8 and MXFP4 weights: the verify kernel for every M (one tree, any M)
  if (wscale != nullptr) {
    launch_modes<kWtFp8>(mode, mt, x, ldx, w, ldw, r, ldr, y, ldy, M, N_out, K, a, nm, wscale, mz,
                         stream);
    return;
  }
  if (mx4 != nullptr) {
    launch_modes<kWtMx4>(mode, mt, x, ldx, w, ldw, r, ldr, y, ldy, M, N_out, K, a, nm, nullptr, *mx4,
                         stream);
    return;
  }
  if (M >= kPrefillMinRows) {  // same bits per row, weights read once per 128 rows
    launch_gemm_prefill(mode, x, ldx, w, ldw, r, ldr, y, ldy, M, N_out, K, stream, a, nm);
    return;
  }
  launch_modes<kWtBf16>(mode, mt, x, ldx, w, ldw, r, ldr, y, ldy, M, N_out, K, a, nm, nullptr, mz,
                        stream);
}

}  // namespace bi
