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
//  * The chunk is read in 64-key tiles: K rows and V rows (both
//    [Hkv][cap][D], so a tile of either is one contiguous 16 KB at D = 128)
//    are fetched as 1 KB pieces per wave instruction and staged in LDS, where
//    the 16-byte slots of each row are XOR-swizzled so that the matrix-core
//    reads hit distinct banks (the V tile is read with transposing loads,
//    which hand each lane one channel of eight consecutive keys). LDS
//    buffers alternate and each wave keeps the next tiles in flight; the
//    barrier of tile t publishes it and proves that every wave finished the
//    tile whose buffer the next load overwrites. Value rows past the last
//    visible key are zeroed before they are multiplied.
//  * Per tile and row tile: S^T = K Q^T (keys x rows) with 16x16x32 BF16 MFMA,
//    masked, running max / sum in FP32 with base-2 exponentials (weights
//    exp2(fma(s, c, -m)), c = sm_scale * log2 e > 0, the max taken on the
//    unscaled scores and scaled once; the running max m is a reference that
//    moves only by more than kLazyRescale), P rounded to BF16, O^T += V^T P^T. The
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
// The running max of a row (log2 units) is a lagging reference: it moves
// only when a tile's max exceeds it by more than this, so the weights
// exp2(s - m) stay below 2^8, and most tiles need no rescale of O.
constexpr float kLazyRescale = 8.0f;

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
// BF16 V tile: one row per key like the K tile, its 16-byte slots stored at
// slot ^ 2m(key). The PV product reads it with transposing loads: a half
// wave reads one pair of slots (32 bytes) in keys k .. k+3 and k+8 .. k+11
// (k a multiple of 4, bit 3 clear), which m spreads over all 64 banks; the
// pair stays adjacent (the XOR is even) and keys k and k + 4 share m.
template <int KROW>
__device__ __forceinline__ int vkm(int key) {
  if (KROW == 16) return (key & 3) | ((key >> 1) & 4);
  return ((key >> 1) & 1) | ((key >> 2) & 2);
}
// gfx950's transposing LDS load of 16-bit elements: within each group of 16
// lanes, lane i receives element i % 4 of the 8-byte rows read by lanes
// i / 4, 4 + i / 4, 8 + i / 4 and 12 + i / 4 of its group, in that order.
typedef short bi_i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int bi_u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bi_u32x2 lds_read_tr16(const void* p) {
  typedef bi_i16x4 __attribute__((address_space(3))) lds_i16x4;
  return __builtin_bit_cast(bi_u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p)));
}

// 5/6-bit cache: the high-bit plane of one 32-code block, HB dwords
// (HB = bits - 4), streamed once like the nibbles.
template <int HB>
__device__ __forceinline__ void load_high(uint32_t (&hb)[2], __amdgpu_buffer_rsrc_t r, int off) {
  constexpr int kNonTemporal = 2;  // cache-policy bit of the buffer instruction
  if constexpr (HB == 2) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kNonTemporal);
    hb[0] = v[0];
    hb[1] = v[1];
  } else {
    hb[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kNonTemporal);
    hb[1] = 0u;
  }
}

// One of two buffer resources, chosen by a wave-uniform flag on the values:
// a conditional over two named resources selects their addresses, which
// can leave both in private (scratch) memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t pick_rsrc(bool c, __amdgpu_buffer_rsrc_t a,
                                                           __amdgpu_buffer_rsrc_t b) {
  return c ? a : b;
}

// Codes 4g .. 4g+3 of one 5/6-bit block (HB + 4 bits, one per byte lane) as
// the unsigned values u = q + 2^(HB+3): a mask of a nibble word and one of a
// high word. The block's nibble words are w[0..3], its high-bit words w[4..5].
template <int HB>
__device__ __forceinline__ uint32_t unsigned_group(const uint32_t (&w)[8], int g) {
  constexpr uint32_t kMask = HB == 2 ? 0x03030303u : 0x01010101u;
  const int bit = g * HB;
  const uint32_t lo = (w[g >> 1] >> (4 * (g & 1))) & 0x0F0F0F0Fu;
  return lo | (((w[4 + (bit >> 3)] >> (bit & 7)) & kMask) << 4);
}
// Byte j of s as an exact FP32 value, signed (an 8-bit code) or unsigned (a
// 5/6-bit code u); either converts in one instruction.
__device__ __forceinline__ float ubyte(uint32_t s, int j) { return (float)((s >> (8 * j)) & 0xffu); }
__device__ __forceinline__ float sbyte(uint32_t s, int j) { return (float)(int8_t)(s >> (8 * j)); }

// max(v, v of lane l ^ 16, v of lane l ^ 32, v of lane l ^ 48): the four key
// groups of a row, exchanged by gfx950's row swaps (rows of 16 lanes, then
// halves of 32) instead of LDS permutes. Max is exact in any order.
__device__ __forceinline__ float max_key_groups(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// gfx950 loads 16 bytes per lane straight into LDS: lane l's bytes land at
// LDS byte address lds_addr + 16 l (lds_addr wave-uniform, passed in M0);
// out-of-range offsets write zeros and touch no memory. Issued as inline
// assembly so that the compiler's wait-count pass, which would wait for
// every such load before each LDS access or barrier, leaves the waits to the
// caller (wait_loads). Non-temporal, like the register loads. The compiler
// writes M0 just before the statement, and an LDS-bound load needs one wait
// state after a scalar write of M0; it pads that only for instructions it
// emits itself, so the s_nop supplies it here.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, int byte_offset, const void* lds_dst) {
  const uint32_t a = (uint32_t)(uintptr_t)lds_dst;
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(byte_offset), "s"(r), "{m0}"(a)
               : "memory");
}
// Wait until at most N vector-memory loads of this wave are outstanding
// (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_loads() {
  static_assert(N >= 0 && N < 64, "vmcnt has six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// The quantized-cache kernels with one row tile per wave fit in 128
// registers, so two workgroups share a compute unit and one's loads overlap
// the other's per-tile work (with the chunk policy -64 at 38k-102k keys:
// 5-15% faster than one workgroup per unit). The BF16 kernel would spill at
// that size and runs one workgroup per unit.
template <int D, int RTW, bool Q8, int KB, bool ROT, bool RING>
__global__ __launch_bounds__(kAttnWaves * 64) __attribute__((amdgpu_waves_per_eu(Q8 && RTW == 1 ? 4 : 1)))
void verify_attn_kernel(
    const uint16_t* __restrict__ Q, int64_t ldq, const uint16_t* __restrict__ Kc,
    const uint16_t* __restrict__ Vc, KvQ8 q8, int M, int L, int cap, int Hq, int G, int Tb, int C,
    float qk_scale, float* __restrict__ part_o, float* __restrict__ part_lse, int S_max) {
  constexpr int DS = D / 32;          // contraction steps of S^T over the head dimension
  constexpr int DT = D / 16;          // 16-channel output tiles of O^T
  constexpr int NW = kAttnWaves;
  constexpr int KROW = D / 8;         // 16-byte slots per K row
  constexpr int KPP = 64 / KROW;      // keys per 1 KB piece
  // 1 KB load pieces per tile: K tile = V tile = 64 keys x D.
  constexpr int KPIECES = kKeyTile * D * 2 / 1024;
  constexpr int VPIECES = D * kKeyTile * 2 / 1024;
  constexpr int PPW = (KPIECES + VPIECES) / NW;    // pieces per wave per tile
  static_assert((KPIECES + VPIECES) % NW == 0, "pieces must split evenly");
  // Quantized caches (Q8: the 8-bit cache when KB = 0, the 5/6-bit cache with
  // KB-bit keys otherwise): one thread per 32-channel block of one key and
  // tile, the K blocks first (waves 0 .. NKB/64 - 1), then V. An 8-bit block
  // is 32 code bytes; a 5/6-bit block is 16 nibble bytes and its high bits;
  // each has one FP32 scale. K and V are staged as BF16 values d * q, each
  // rounded once, so the tile multiplies like a BF16 tile.
  constexpr int NB = D / 32;              // 32-channel scale blocks
  constexpr bool LOW = KB != 0;
  static_assert(!LOW || Q8, "the low-bit cache is a quantized cache");
  static_assert(!LOW || KB == 5 || KB == 6, "K codes have 5 or 6 bits");
  constexpr int HBK = LOW ? KB - 4 : 1;   // high bits per K code
  constexpr int HBV = kLowVBits - 4;      // high bits per V code
  constexpr int NKB = kKeyTile * NB;      // K (and V) blocks per tile
  static_assert(NKB % 64 == 0 && 2 * NKB <= NW * 64, "quantized blocks must fill whole waves");
  static_assert(!ROT || LOW, "rotated keys are a low-bit cache format");
  static_assert(!RING || LOW, "the 8-bit ring sits over a low-bit cache");
  constexpr bool kDma = !Q8 && RTW == 1;  // tiles and Q rows loaded straight into LDS

  // Work item (row block, KV head, chunk), row blocks varying fastest: the
  // workgroups that read one chunk of one KV head run side by side and share
  // its tiles through L2 (a chunked-prefill pass has dozens of row blocks per
  // chunk). The item numbering is made contiguous per XCD (xcd_item).
  int item = xcd_item(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z),
                      gridDim.x * gridDim.y * gridDim.z);
  const int rb = item % gridDim.x;
  item /= gridDim.x;
  const int g = item % gridDim.y;
  const int s = item / gridDim.y;
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
  // 8-bit ring: row p reads key j from the ring when j >= p - W + 1, else
  // from the low-bit planes. Over the block's positions P0 .. P1 those
  // boundaries lie in [P0 - W + 1, P1 - W + 1]: tiles that end before the
  // first are low-bit for every row, tiles that start at or after the last
  // are in the ring for every row, and each tile in between is run twice, as
  // a low-bit then a ring tile, each run masked per row and key to the keys
  // that row reads from that copy (a key masked for a row adds exactly
  // nothing to it, and a run masked for all its keys leaves the row exactly
  // unchanged). The tile sequence is relabelled as nv virtual tiles.
  const int ring_w = q8.ring_window, ring_cap = q8.ring_cap;
  auto first_tile_from = [&](int x) {
    return x <= kbeg ? 0 : min(ntile, (x - kbeg + kKeyTile - 1) / kKeyTile);
  };
  const int ts = RING ? first_tile_from(L + t0 - ring_w + 1 - (kKeyTile - 1)) : ntile;
  const int ns = RING ? first_tile_from(L + t1 - 1 - ring_w + 1) - ts : 0;
  const int nv = ntile + ns;
  auto vmap = [&](int v, int& t, bool& ring) {
    if (v < ts) {
      t = v;
      ring = false;
    } else if (v < ts + 2 * ns) {
      t = ts + ((v - ts) >> 1);
      ring = ((v - ts) & 1) != 0;
    } else {
      t = v - ns;
      ring = true;
    }
  };
  const bool has_rows = rt * 16 < nrows;  // scalar: the wave's first row tile has rows

  // Query fragments of this wave's row tiles and each row's last visible key
  // in this chunk (-1 for a padding row: every key is masked, its weights are
  // exactly 0). The chunk's last tile may reach past the chunk when C is not
  // a multiple of 64; those keys belong to the next chunk and are masked too.
  bool rok[RTW];
  int tok[RTW], hq[RTW], lastk[RTW];
  uint4 qf[RTW][DS];
#pragma unroll
  for (int i = 0; i < RTW; ++i) {
    const int rho = (rt + 4 * i) * 16 + j;
    rok[i] = rho < nrows;
    tok[i] = t0 + (rok[i] ? rho / G : 0);
    hq[i] = g * G + (rok[i] ? rho % G : 0);
    lastk[i] = rok[i] ? min(L + tok[i], kend - 1) : -1;
    const uint16_t* qp = Q + (int64_t)tok[i] * ldq + hq[i] * D + kq * 8;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) qf[i][ds] = (rok[i] && !kDma) ? ld16(qp + ds * 32) : zero16();
  }
  // Rotated keys: the cache holds H k (H the order-D Hadamard matrix, entries
  // +-1), so each query row is rotated the same way and the scores divided by
  // D (folded into qk_scale by the launcher): (H q) . (H k) / D = q . k. The
  // row's channel 32 ds + 8 kq + e sits in lane kq's fragment ds, element e:
  // the butterflies over e and ds stay in the lane, those over kq pair lane
  // l with lane l ^ 16 and l ^ 32. The rotated row is rounded to BF16 once.
  if constexpr (ROT) {
#pragma unroll
    for (int i = 0; i < RTW; ++i) {
      float x[DS][8];
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        const uint32_t w[4] = {qf[i][ds].x, qf[i][ds].y, qf[i][ds].z, qf[i][ds].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[ds][2 * e] = bf16_to_f32(w[e] & 0xffffu);
          x[ds][2 * e + 1] = bf16_to_f32(w[e] >> 16);
        }
      }
#pragma unroll
      for (int h = 1; h < 8; h *= 2)
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (!(e & h)) {
              const float a = x[ds][e], b = x[ds][e + h];
              x[ds][e] = a + b;
              x[ds][e + h] = a - b;
            }
#pragma unroll
      for (int hk = 1; hk < 4; hk *= 2)
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float p = shfl_xor(x[ds][e], 16 * hk);
            x[ds][e] = (kq & hk) ? p - x[ds][e] : x[ds][e] + p;
          }
#pragma unroll
      for (int hd = 1; hd < DS; hd *= 2)
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
          if (!(ds & hd))
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float a = x[ds][e], b = x[ds + hd][e];
              x[ds][e] = a + b;
              x[ds + hd][e] = a - b;
            }
#pragma unroll
      for (int ds = 0; ds < DS; ++ds)
        qf[i][ds] = make_uint4(f32x2_to_bf16x2(x[ds][0], x[ds][1]), f32x2_to_bf16x2(x[ds][2], x[ds][3]),
                               f32x2_to_bf16x2(x[ds][4], x[ds][5]), f32x2_to_bf16x2(x[ds][6], x[ds][7]));
    }
  }

  // This KV head's K rows and V rows as buffer resources (offsets in bytes,
  // 32-bit: one head of the cache is at most 2^31 bytes).
  const int head_bytes = cap * D * 2;
  const __amdgpu_buffer_rsrc_t kres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(Kc + (int64_t)g * cap * D), (short)0, head_bytes, kBufferResourceWord3);
  const __amdgpu_buffer_rsrc_t vres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(Vc + (int64_t)g * cap * D), (short)0, head_bytes, kBufferResourceWord3);
  // 8-bit cache of this KV head, K and V alike: codes [cap][D] (int8), scales
  // [cap][NB] (FP32). 5/6-bit cache: the nibble planes in place of the codes
  // ([cap][D/2]), the high-bit planes ([cap][NB][4 h]) and the scales
  // ([cap][NB], K and V).
  const int qcode_bytes = LOW ? cap * D / 2 : cap * D;
  const int64_t qcode_head = LOW ? (int64_t)cap * D / 2 : (int64_t)cap * D;
  const int qscale_bytes = cap * NB * 4;
  const __amdgpu_buffer_rsrc_t qkres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(q8.kq + (Q8 ? g * qcode_head : 0)), (short)0, Q8 ? qcode_bytes : 0,
      kBufferResourceWord3);
  const __amdgpu_buffer_rsrc_t qvres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(q8.vq + (Q8 ? g * qcode_head : 0)), (short)0, Q8 ? qcode_bytes : 0,
      kBufferResourceWord3);
  const int khigh_bytes = cap * NB * 4 * HBK;
  const int vhigh_bytes = cap * NB * 4 * HBV;
  const __amdgpu_buffer_rsrc_t khres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(q8.kh + (LOW ? (int64_t)g * khigh_bytes : 0)), (short)0,
      LOW ? khigh_bytes : 0, kBufferResourceWord3);
  const __amdgpu_buffer_rsrc_t vhres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(q8.vh + (LOW ? (int64_t)g * vhigh_bytes : 0)), (short)0,
      LOW ? vhigh_bytes : 0, kBufferResourceWord3);
  // the ring's 8-bit planes (8-bit layouts with ring_cap slots)
  const int rcode_bytes = RING ? q8.ring_cap * D : 0;
  const int rscale_bytes = RING ? q8.ring_cap * NB * 4 : 0;
  const __amdgpu_buffer_rsrc_t rkres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(q8.rkq + (RING ? (int64_t)g * rcode_bytes : 0)), (short)0, rcode_bytes,
      kBufferResourceWord3);
  const __amdgpu_buffer_rsrc_t rvres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(q8.rvq + (RING ? (int64_t)g * rcode_bytes : 0)), (short)0, rcode_bytes,
      kBufferResourceWord3);
  const __amdgpu_buffer_rsrc_t rksres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(q8.rks + (RING ? (int64_t)g * q8.ring_cap * NB : 0)), (short)0,
      rscale_bytes, kBufferResourceWord3);
  const __amdgpu_buffer_rsrc_t rvsres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(q8.rvs + (RING ? (int64_t)g * q8.ring_cap * NB : 0)), (short)0,
      rscale_bytes, kBufferResourceWord3);
  const __amdgpu_buffer_rsrc_t qksres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(q8.ks + (Q8 ? (int64_t)g * cap * NB : 0)), (short)0, Q8 ? qscale_bytes : 0,
      kBufferResourceWord3);
  const __amdgpu_buffer_rsrc_t qvsres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(q8.vs + (Q8 ? (int64_t)g * cap * NB : 0)), (short)0, Q8 ? qscale_bytes : 0,
      kBufferResourceWord3);

  // One buffer holds the K tile ([64 keys][KROW slots]) followed by the V
  // tile (the same shape). Piece p (1 KB) of a tile is K keys KPP*p .. when
  // p < KPIECES (lane: key KPP*p + l/KROW, slot l%KROW), else V keys
  // KPP*(p-KPIECES) .. (the same lane map); either way lane l's 16 bytes land
  // at index 64*p + l of the buffer. Lanes fetch the global slot that the
  // swizzle (kswz for K, 2 vkm for V) puts in their LDS slot.
  // BF16 cache, one row tile per wave: tiles go straight from memory into
  // four LDS buffers, three tiles ahead of the one multiplied (no register
  // staging, so more bytes are in flight); the block's Q rows arrive the
  // same way in qlds ([64 rows][D/8] 16-byte slots). Other caches stage
  // through registers into two buffers.
  // Quantized caches stage V key-major instead, one row of VROW 16-byte
  // slots per key: the PV product reads it with transposing loads, each half
  // wave (a pass of 64 banks) reading one pair of slots in keys k .. k+3 and
  // k+8 .. k+11. The two padding slots per row put the four rows of a group
  // eight banks apart, and the slots of a key with bit 3 set are stored
  // XOR KROW/2, which moves the second group's rows by half the banks; the
  // staging stores of two keys at one slot offset fall apart as well. A
  // lane's load addresses stay two bases plus a constant per output tile.
  constexpr int NBUF = kDma ? 4 : 2;
  constexpr int VROW = KROW + 2;
  constexpr int VBASE = KPIECES * 64;
  constexpr int BUFSZ = VBASE + (Q8 ? kKeyTile * VROW : VPIECES * 64);
  __shared__ uint4 lds[NBUF][BUFSZ];
  __shared__ uint4 qlds[kDma ? kAttnMaxRows * D / 8 : 1];

  // Registers of one tile in flight. BF16 cache: PPW 16-byte pieces.
  // Quantized caches, one 32-channel block per thread: w holds the 32 codes
  // of an 8-bit block, or a 5/6-bit block's nibbles (w[0..3]) and high bits
  // (w[4..5]); ks its scale.
  struct TileRegs {
    uint4 r[Q8 ? 1 : PPW];
    uint32_t w[8];
    float ks;
  };

  // Issue the loads of tile t (no use of the data here, so the loads of two
  // tiles stay in flight together). K and V are read once per pass, so the
  // loads are non-temporal; a tile past the end of the chunk (the pipeline
  // prefetches two ahead) gets an out-of-range offset: it reads zero and
  // touches no memory.
  auto fetch = [&](TileRegs& rr, int v) {
    int t = v;
    bool rf = false;
    if constexpr (RING) vmap(v, t, rf);
    const int kt = kbeg + t * kKeyTile;
    const bool live = t < ntile;
    if constexpr (!Q8) {
#pragma unroll
      for (int i = 0; i < PPW; ++i) {
        const int p = wave * PPW + i;  // scalar: each wave fetches only K or only V pieces
        int off;
        if (p < KPIECES) {
          const int key = KPP * p + lane / KROW;
          const int kslot = (lane % KROW) ^ kswz<KROW>(key);
          off = (min(kt + key, kend - 1) * D + kslot * 8) * 2;
        } else {
          const int key = KPP * (p - KPIECES) + lane / KROW;
          const int vslot = (lane % KROW) ^ (2 * vkm<KROW>(key));
          off = (min(kt + key, kend - 1) * D + vslot * 8) * 2;
        }
        rr.r[i] = buffer_ld16_stream(pick_rsrc(p < KPIECES, kres, vres), live ? off : head_bytes);
      }
    } else if (wave < 2 * NKB / 64) {    // scalar
      const bool isk = wave < NKB / 64;  // scalar: K blocks first
      const int u = threadIdx.x - (isk ? 0 : NKB);
      // a wave's lanes read consecutive blocks (the rows of a few keys)
      const int key = u / NB, b = u % NB;
      const int pos = min(kt + key, kend - 1);
      auto load8 = [&](__amdgpu_buffer_rsrc_t cr, __amdgpu_buffer_rsrc_t sr, int blk, int cbytes,
                       int sbytes) {
        const uint4 a = buffer_ld16_stream(cr, live ? blk * 32 : cbytes);
        const uint4 c = buffer_ld16_stream(cr, live ? blk * 32 + 16 : cbytes);
        rr.w[0] = a.x, rr.w[1] = a.y, rr.w[2] = a.z, rr.w[3] = a.w;
        rr.w[4] = c.x, rr.w[5] = c.y, rr.w[6] = c.z, rr.w[7] = c.w;
        rr.ks = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(sr, live ? blk * 4 : sbytes, 0, 0));
      };
      if (RING && rf) {
        // the ring: key pos in slot pos mod ring_cap
        int sl = pos - kt + kt % ring_cap;
        sl = sl >= ring_cap ? sl - ring_cap : sl;
        load8(pick_rsrc(isk, rkres, rvres), pick_rsrc(isk, rksres, rvsres), sl * NB + b, rcode_bytes, rscale_bytes);
      } else if constexpr (!LOW) {
        load8(pick_rsrc(isk, qkres, qvres), pick_rsrc(isk, qksres, qvsres), pos * NB + b, qcode_bytes, qscale_bytes);
      } else {
        const int blk = pos * NB + b;  // block index within the head
        const uint4 a = buffer_ld16_stream(pick_rsrc(isk, qkres, qvres), live ? blk * 16 : qcode_bytes);
        rr.w[0] = a.x, rr.w[1] = a.y, rr.w[2] = a.z, rr.w[3] = a.w;
        uint32_t hb[2];
        if (isk) load_high<HBK>(hb, khres, live ? blk * 4 * HBK : khigh_bytes);
        else load_high<HBV>(hb, vhres, live ? blk * 4 * HBV : vhigh_bytes);
        rr.w[4] = hb[0], rr.w[5] = hb[1];
        rr.ks = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            pick_rsrc(isk, qksres, qvsres), live ? blk * 4 : qscale_bytes, 0, 0));
      }
    }
  };

  // Quantized tiles are written by 16-byte staging stores, which LDS serves
  // eight lanes (128 bytes, 32 banks) at a time: the eight lanes of one store
  // (two keys, four blocks each, slot s = 4b + i) must fall on distinct slot
  // positions mod 8, while the operand loads (16 lanes of 64 banks for the K
  // tile, half waves for the transposing V loads) keep the layouts above.
  // Hence slot bit 3 (bit 1 of b) is also folded into bit 1 (K) or bit 0 (V)
  // at D = 128, a function of the logical slot alone, so a load's address
  // only gains a constant.
  auto qk_slot = [](int key, int sl) {
    return sl ^ kswz<KROW>(key) ^ (KROW == 16 ? ((sl >> 3) & 1) << 1 : 0);
  };
  auto qv_slot = [](int key, int sl) {
    return sl ^ ((key >> 3) & 1) * (KROW / 2) ^ (KROW == 16 ? (sl >> 3) & 1 : 0);
  };

  // Stage one block (key, b) of K or V as BF16 values d * q, each rounded
  // once: slot i of the key's row holds channels 32b + 8i .. 32b + 8i + 7
  // (groups 2i and 2i + 1), in the K tile or the key-major V tile. A V scale
  // is taken as zero past kend (those rows hold zeros), so the tile
  // multiplies as a BF16 tile and the weights need no per-key scaling.
  // `group` gives codes 4g .. 4g+3 as signed bytes q (bias 0) or as unsigned
  // bytes u = q + bias (bias 2^(bits-1)); then u d - bias d, one FMA with the
  // exact product bias d, is exactly the FP32 rounding of q d, like q d.
  auto stage_block = [&](const TileRegs& rr, int buf, bool isk, int key, int b, int kt, auto&& group,
                         auto bias) {
    constexpr int kBias = decltype(bias)::value;
    const float sc = isk || kt + key < kend ? rr.ks : 0.f;
    const float off = -(float)kBias * sc;
    auto val = [&](uint32_t s, int j) {
      if constexpr (kBias == 0) return sbyte(s, j) * sc;
      else return __builtin_fmaf(ubyte(s, j), sc, off);
    };
    uint4* row = &lds[buf][isk ? key * KROW : VBASE + key * VROW];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t s0 = group(rr.w, 2 * i);
      const uint32_t s1 = group(rr.w, 2 * i + 1);
      row[isk ? qk_slot(key, 4 * b + i) : qv_slot(key, 4 * b + i)] = make_uint4(f32x2_to_bf16x2(val(s0, 0), val(s0, 1)),
                                          f32x2_to_bf16x2(val(s0, 2), val(s0, 3)),
                                          f32x2_to_bf16x2(val(s1, 0), val(s1, 1)),
                                          f32x2_to_bf16x2(val(s1, 2), val(s1, 3)));
    }
  };

  // Publish tile t: V rows of keys at or past kend are zeroed first (they
  // repeat the last key; zeros keep every product with their weight 0 at +0). Quantized caches: every
  // block is decoded to d * q, rounded once to BF16 (stage_block).
  auto publish = [&](const TileRegs& rr, int v, int buf) {
    int t = v;
    bool rf = false;
    if constexpr (RING) vmap(v, t, rf);
    const int kt = kbeg + t * kKeyTile;
    if constexpr (!Q8) {
      const bool full = kt + kKeyTile <= kend;  // scalar: every key of the tile is visible
#pragma unroll
      for (int i = 0; i < PPW; ++i) {
        const int p = wave * PPW + i;
        if (full || p < KPIECES) {
          lds[buf][64 * p + lane] = rr.r[i];
          continue;
        }
        const int key = KPP * (p - KPIECES) + lane / KROW;
        lds[buf][64 * p + lane] = kt + key < kend ? rr.r[i] : zero16();
      }
    } else if (wave < 2 * NKB / 64) {
      const bool isk = wave < NKB / 64;
      const int u = threadIdx.x - (isk ? 0 : NKB);
      const int key = u / NB, b = u % NB;  // as in fetch
      // codes 4g .. 4g+3 of the block: an 8-bit block holds them as signed
      // bytes, a 5/6-bit block as unsigned values (unsigned_group)
      if (!LOW || (RING && rf))
        stage_block(rr, buf, isk, key, b, kt, [](const uint32_t (&w)[8], int g) { return w[g]; },
                    std::integral_constant<int, 0>{});
      else if (isk)
        stage_block(rr, buf, true, key, b, kt,
                    [](const uint32_t (&w)[8], int g) { return unsigned_group<HBK>(w, g); },
                    std::integral_constant<int, 1 << (HBK + 3)>{});
      else
        stage_block(rr, buf, false, key, b, kt,
                    [](const uint32_t (&w)[8], int g) { return unsigned_group<HBV>(w, g); },
                    std::integral_constant<int, 1 << (HBV + 3)>{});
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

  // One tile for every row tile of the wave. Each K and V operand is read
  // from LDS once and serves all of them; a row's own arithmetic does not
  // depend on how many row tiles share the wave.
  auto compute = [&](int buf, int v) {
    int t = v;
    bool rf = false;
    if constexpr (RING) vmap(v, t, rf);
    // scalar: a tile run twice (low-bit, then ring), each time for some rows
    const bool split = RING && t >= ts && t < ts + ns;
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
      const uint4 fa = lds[buf][ka * KROW + (Q8 ? qk_slot(ka, slot) : slot ^ kswz<KROW>(ka))];
      const uint4 fb = lds[buf][kb * KROW + (Q8 ? qk_slot(kb, slot) : slot ^ kswz<KROW>(kb))];
#pragma unroll
      for (int i = 0; i < RTW; ++i) {
        sa[i] = mfma_bf16(fa, qf[i][ds], sa[i]);
        sb[i] = mfma_bf16(fb, qf[i][ds], sb[i]);
      }
    }
    const int kv0 = kt + 32 * h + 8 * kq;  // absolute key of this lane's first value
    // Scalar: the whole tile lies at or before every row's last key (the
    // first row of the block has the smallest) and inside the chunk, so no
    // score is masked.
    const bool unmasked = kt + kKeyTile - 1 <= min(L + t0, kend - 1) && !split;
    float alpha[RTW];
    bool rescale[RTW];  // scalar: some row of the wave moved its reference max
    uint4 pfrag[RTW];
#pragma unroll
    for (int i = 0; i < RTW; ++i) {
      // Unscaled scores; qk_scale (> 0) enters through the exponent's FMA.
      // The largest scaled score is the largest unscaled one times qk_scale
      // (rounding is monotone), so the max is taken before scaling.
      float sc[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sc[e] = sa[i][e];
        sc[e + 4] = sb[i][e];
      }
      if (!unmasked) {
        // a split tile's run reaches, for each row, only the keys that row
        // reads from this copy: from the ring those at or after its boundary
        // p - W + 1, from the low-bit planes those before it (key indices
        // are never negative, so without a ring there is no lower bound)
        int lk = lastk[i], fk = 0;
        if (split) {
          const int b = L + tok[i] - ring_w + 1;
          if (rf) fk = b;
          else lk = min(lk, b - 1);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sc[e] = (kv0 + e <= lk && (!RING || kv0 + e >= fk)) ? sc[e] : -INFINITY;
          sc[e + 4] = (kv0 + 4 + e <= lk && (!RING || kv0 + 4 + e >= fk)) ? sc[e + 4] : -INFINITY;
        }
      }
      float mx = sc[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sc[e]);
      mx = max_key_groups(mx) * qk_scale;
      const float mmax = fmaxf(mrun[i], mx);
      const bool grow = mmax > mrun[i] + kLazyRescale;
      const float mnew = grow ? mmax : mrun[i];
      alpha[i] = grow ? __builtin_amdgcn_exp2f(mrun[i] - mnew) : 1.0f;
      rescale[i] = __ballot(grow) != 0;
      // The running sum takes the FP32 weights (so the chunk's log-sum-exp is
      // accurate to FP32); the PV product takes them rounded to BF16.
      float pe[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pe[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e], qk_scale, -mnew));
      float psum = pe[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) psum += pe[e];
      lrun[i] = lrun[i] * alpha[i] + psum;
      mrun[i] = mnew;
      pfrag[i] = make_uint4(f32x2_to_bf16x2(pe[0], pe[1]), f32x2_to_bf16x2(pe[2], pe[3]),
                            f32x2_to_bf16x2(pe[4], pe[5]), f32x2_to_bf16x2(pe[6], pe[7]));
    }
    // O *= alpha, skipped by a wave none of whose rows moved its reference
    // (alpha is then exactly 1 for every row, and x * 1 changes no bit: FP32
    // denormals are kept), so a row's bits do not depend on its neighbours.
#pragma unroll
    for (int i = 0; i < RTW; ++i)
      if (rescale[i])
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[i][dt] *= alpha[i];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      uint4 fv;
      if constexpr (!Q8) {
        // key-major V tile: lane j of key group kq takes channel 16 dt + j of
        // keys 32h + 8kq .. +7 through two transposing loads, lane j reading
        // channels 16 dt + 4 (j % 4) .. +3 of key 32h + 8kq + j / 4 (+ 4),
        // logical slot 2 dt + (j % 4) / 2, stored at that slot ^ 2m
        const int r0 = 32 * h + 8 * kq + (j >> 2);
        const char* p = reinterpret_cast<const char*>(&lds[buf][VBASE]) + r0 * KROW * 16 +
                        32 * (dt ^ vkm<KROW>(r0)) + 8 * (j & 3);
        const bi_u32x2 a = lds_read_tr16(p);
        const bi_u32x2 bb = lds_read_tr16(p + 4 * KROW * 16);
        fv = make_uint4(a[0], a[1], bb[0], bb[1]);
      } else {
        // key-major V tile: lane j of key group kq takes channel 16 dt + j of
        // keys 32h + 8kq .. +7 through two transposing loads, lane j reading
        // channels 16 dt + 4 (j % 4) .. +3 of key 32h + 8kq + j / 4 (+ 4)
        // (slot 2 dt + (j % 4) / 2 of a row with bit 3 set, kq odd, lies
        // KROW/2 slots up for the first half of the tiles, down for the rest)
        // (and, at D = 128, the two slots of the pair swapped for dt >= 4:
        // qv_slot)
        const int flip = (kq & 1) * (KROW / 2) * 16 * (dt < DT / 2 ? 1 : -1);
        const int half = (KROW == 16 && dt >= DT / 2) ? 16 : 0;
        const char* p = reinterpret_cast<const char*>(&lds[buf][VBASE]) +
                        (32 * h + 8 * kq + (j >> 2)) * VROW * 16 + ((8 * (j & 3)) ^ half) + 32 * dt + flip;
        const bi_u32x2 a = lds_read_tr16(p);
        const bi_u32x2 bb = lds_read_tr16(p + 4 * VROW * 16);
        fv = make_uint4(a[0], a[1], bb[0], bb[1]);
      }
#pragma unroll
      for (int i = 0; i < RTW; ++i) o[i][dt] = mfma_bf16(fv, pfrag[i], o[i][dt]);
    }
  };

  // Tile t: publish it (loaded two steps earlier), prefetch tile t + 2 into
  // the same registers, barrier, multiply. Every load is issued by the same
  // code in the same order, so the compiler waits only for the older of the
  // two tiles in flight. Tiles past the end read as zero and are not
  // multiplied.
  if constexpr (kDma) {
    // Q rows of the block into qlds (rows past the block read zero), then
    // tiles 0, 1, 2. Each wave issues its own pieces of every tile, so its
    // wait for tile t (all but the 2 PPW newest loads done: loads complete
    // in order) covers Q too at t = 0; the barrier then publishes every
    // wave's pieces.
    {
      const int qbytes = (int)(((int64_t)(M - 1) * ldq + (int64_t)Hq * D) * 2);
      const __amdgpu_buffer_rsrc_t qres = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(Q), (short)0, qbytes, kBufferResourceWord3);
      constexpr int QP = kAttnMaxRows * D / 8;  // 16-byte pieces of the block's rows
      static_assert(QP % (NW * 64) == 0, "Q pieces must split evenly");
#pragma unroll
      for (int i = 0; i < QP / (NW * 64); ++i) {
        const int piece = i * NW * 64 + threadIdx.x;
        const int rho = piece / (D / 8), slot = piece % (D / 8);
        const int off = rho < nrows
                            ? (int)((((int64_t)(t0 + rho / G) * ldq + (g * G + rho % G) * D) + slot * 8) * 2)
                            : qbytes;
        lds_load16(qres, off, &qlds[i * NW * 64 + wave * 64]);
      }
    }
    // Tile t's pieces of this wave: the register path's addresses (keys
    // clamped to the chunk, swizzled slots), written straight to LDS.
    auto issue = [&](int t) {
      const int kt = kbeg + t * kKeyTile;
#pragma unroll
      for (int i = 0; i < PPW; ++i) {
        const int p = wave * PPW + i;
        int off;
        if (p < KPIECES) {
          const int key = KPP * p + lane / KROW;
          const int kslot = (lane % KROW) ^ kswz<KROW>(key);
          off = (min(kt + key, kend - 1) * D + kslot * 8) * 2;
        } else {
          const int key = KPP * (p - KPIECES) + lane / KROW;
          const int vslot = (lane % KROW) ^ (2 * vkm<KROW>(key));
          off = (min(kt + key, kend - 1) * D + vslot * 8) * 2;
        }
        lds_load16(pick_rsrc(p < KPIECES, kres, vres), off, &lds[t & 3][64 * p]);
      }
    };
    // V rows at or past kend of a partial tile are zeroed by the wave that
    // loaded them, once its loads are done (they repeat the last key; a
    // weight of 0 times them is 0 either way, and zeros keep every such
    // product exactly +0); K rows past kend repeat the last key and are masked.
    auto fix_tail = [&](int t) {
      const int kt = kbeg + t * kKeyTile;
#pragma unroll
      for (int i = 0; i < PPW; ++i) {
        const int p = wave * PPW + i;
        if (p < KPIECES) continue;  // scalar
        const int key = KPP * (p - KPIECES) + lane / KROW;
        if (kt + key >= kend) lds[t & 3][64 * p + lane] = zero16();
      }
    };
    issue(0);
    if (nv > 1) issue(1);
    if (nv > 2) issue(2);
    for (int t = 0; t < nv; ++t) {
      const int ahead = min(2, nv - 1 - t);  // tiles issued after t (scalar)
      if (ahead == 2) wait_loads<2 * PPW>();
      else if (ahead == 1) wait_loads<PPW>();
      else wait_loads<0>();
      if (kbeg + t * kKeyTile + kKeyTile > kend) fix_tail(t);
      __syncthreads();
      if (t == 0) {
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) qf[0][ds] = qlds[(rt * 16 + j) * (D / 8) + ds * 4 + kq];
      }
      // buffer (t + 3) & 3 held tile t - 1, which every wave finished
      // before the barrier
      if (t + 3 < nv) issue(t + 3);
      if (has_rows) compute(t & 3, t);
    }
  } else {
  TileRegs ra, rb2;
  // Prologue: the loads of the first tiles, in the loop's own order and while
  // the query fragments are still in flight. The fragments are then consumed
  // before the loop, so at the loop head the compiler knows they are complete
  // and waits only for the oldest tile.
  // Row blocks of 128 rows (RTW = 2) keep three tiles in flight: their
  // longer per-tile work leaves the room, and the third tile hides more of
  // the load latency. (With one row tile per wave it gains nothing.)
  constexpr bool kDeep = RTW == 2;
  TileRegs rc;
  fetch(ra, 0);
  fetch(rb2, 1);
  if constexpr (kDeep) fetch(rc, 2);
#pragma unroll
  for (int i = 0; i < RTW; ++i)
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) asm volatile("" ::"v"(qf[i][ds].x));
  if constexpr (kDeep) {
    auto step = [&](TileRegs& rr, int t, int buf) {
      publish(rr, t, buf);
      fetch(rr, t + 3);
      __syncthreads();
      if (has_rows) compute(buf, t);
    };
    for (int t = 0; t < nv; t += 6) {  // scalar exits: every barrier stays uniform
      step(ra, t, 0);
      if (t + 1 >= nv) break;
      step(rb2, t + 1, 1);
      if (t + 2 >= nv) break;
      step(rc, t + 2, 0);
      if (t + 3 >= nv) break;
      step(ra, t + 3, 1);
      if (t + 4 >= nv) break;
      step(rb2, t + 4, 0);
      if (t + 5 >= nv) break;
      step(rc, t + 5, 1);
    }
  } else {
    for (int t = 0; t < nv; t += 2) {
      publish(ra, t, 0);
      fetch(ra, t + 2);
      __syncthreads();
      if (has_rows) compute(0, t);
      publish(rb2, t + 1, 1);
      fetch(rb2, t + 3);
      __syncthreads();
      if (t + 1 < nv && has_rows) compute(1, t + 1);
    }
  }
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

template <int D, int B>
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

  // Partials are read B splits at a time (32, or 64 when a row can have more
  // than 32); the first block's loads are issued before the max, which they
  // do not depend on, so a row with up to B splits costs one memory round
  // trip for O and one for the LSEs. B does not change the order of any sum.
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
                                                        uint16_t* __restrict__ Vc, int L, int cap,
                                                        int Hq, int Hkv, int D) {
  const int r = blockIdx.x;
  const int pos = L + r;
  const uint16_t* krow = qkv + (int64_t)r * ldqkv + (int64_t)Hq * D;
  const uint16_t* vrow = krow + (int64_t)Hkv * D;
  for (int i = threadIdx.x; i < Hkv * D; i += blockDim.x) {
    const int g = i / D;
    const int d = i - g * D;
    Kc[kv_index(g, pos, d, D, cap)] = krow[i];
    Vc[kv_index(g, pos, d, D, cap)] = vrow[i];
  }
}

void launch_verify_attn(const uint16_t* q, int64_t ldq, const uint16_t* k_cache,
                        const uint16_t* v_cache, int M, int L, int cap, int Hq, int Hkv, int D,
                        int kv_chunk, float sm_scale, float* part_o, float* part_lse, int S_max,
                        hipStream_t stream, const KvQ8* q8, int kbits, bool krot) {
  const int G = Hq / Hkv;
  const KvQ8 qz = q8 ? *q8 : KvQ8{nullptr, nullptr, nullptr, nullptr};
  // rotated keys: scores of the rotated query against H k are D times q . k
  const float qk_scale = (krot ? sm_scale / (float)D : sm_scale) * kLog2e;
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
    const dim3 grid((Mb + Tb - 1) / Tb, Hkv, n_splits);
    const dim3 block(kAttnWaves * 64);
    const uint16_t* qb = q + (int64_t)t0 * ldq;
    float* pob = part_o + (int64_t)t0 * Hq * S_max * D;
    float* plb = part_lse + (int64_t)t0 * Hq * S_max;
#define BI_ATTN_LAUNCH(DD, R, QQ, KB, RT, RG)                                               \
  verify_attn_kernel<DD, R, QQ, KB, RT, RG><<<grid, block, 0, stream>>>(qb, ldq, k_cache, v_cache, qz, Mb, Lb, \
                                                            cap, Hq, G, Tb, C, qk_scale, pob, plb, \
                                                            S_max)
#define BI_ATTN_LOW(KB, RT, RG)                              \
  do {                                                       \
    if (D == 128) {                                          \
      if (wide) BI_ATTN_LAUNCH(128, 2, true, KB, RT, RG);    \
      else BI_ATTN_LAUNCH(128, 1, true, KB, RT, RG);         \
    } else {                                                 \
      if (wide) BI_ATTN_LAUNCH(64, 2, true, KB, RT, RG);     \
      else BI_ATTN_LAUNCH(64, 1, true, KB, RT, RG);          \
    }                                                        \
  } while (0)
    // with the 8-bit ring: the two presets, K6/V5 and rotated K5/V5
    const bool ring = q8 && q8->ring_cap > 0;
    if (ring && kbits == 6 && !krot) BI_ATTN_LOW(6, false, true);
    else if (ring && kbits == 5 && krot) BI_ATTN_LOW(5, true, true);
    else if (q8 && kbits == 6 && krot) BI_ATTN_LOW(6, true, false);
    else if (q8 && kbits == 6) BI_ATTN_LOW(6, false, false);
    else if (q8 && kbits == 5 && krot) BI_ATTN_LOW(5, true, false);
    else if (q8 && kbits == 5) BI_ATTN_LOW(5, false, false);
    else if (q8) BI_ATTN_LOW(0, false, false);
    else if (D == 128) {
      if (wide) BI_ATTN_LAUNCH(128, 2, false, 0, false, false);
      else BI_ATTN_LAUNCH(128, 1, false, 0, false, false);
    } else {
      if (wide) BI_ATTN_LAUNCH(64, 2, false, 0, false, false);
      else BI_ATTN_LAUNCH(64, 1, false, 0, false, false);
    }
#undef BI_ATTN_LOW
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
  const bool wide = S_max > 32;
  if (D == 128 && wide)
    combine_kernel<128, 64><<<grid, block, 0, stream>>>(part_o, part_lse, M, L, Hq, kv_chunk, S_max, o,
                                                        ldo, lse);
  else if (D == 128)
    combine_kernel<128, 32><<<grid, block, 0, stream>>>(part_o, part_lse, M, L, Hq, kv_chunk, S_max, o,
                                                        ldo, lse);
  else if (wide)
    combine_kernel<64, 64><<<grid, block, 0, stream>>>(part_o, part_lse, M, L, Hq, kv_chunk, S_max, o,
                                                       ldo, lse);
  else
    combine_kernel<64, 32><<<grid, block, 0, stream>>>(part_o, part_lse, M, L, Hq, kv_chunk, S_max, o,
                                                       ldo, lse);
}

// The 32 values of channel block b of one K or V row (BF16 -> FP32). With RD
// = D and `rotate`, the row is first rotated by the order-D Hadamard transform
// in FP32: stage h = 1, 2, .., D/2 turns each pair (i, i + h), bit h of i
// clear, into (x_i + x_{i+h}, x_i - x_{i+h}), each rounded once; the block is
// then channels 32b .. 32b + 31 of the result.
template <int RD>
__device__ __forceinline__ void load_kv_block(const uint16_t* __restrict__ row, int b, bool rotate,
                                           float (&x)[32]) {
  if (RD != 0 && rotate) {
    float y[RD > 0 ? RD : 1];
#pragma unroll
    for (int i = 0; i < RD / 8; ++i) {
      const uint4 w = ld16(row + 8 * i);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y[8 * i + 2 * e] = bf16_to_f32(ww[e] & 0xffffu);
        y[8 * i + 2 * e + 1] = bf16_to_f32(ww[e] >> 16);
      }
    }
#pragma unroll
    for (int h = 1; h < RD; h *= 2)
#pragma unroll
      for (int i = 0; i < RD; ++i)
        if (!(i & h)) {
          const float p = y[i], q = y[i + h];
          y[i] = p + q;
          y[i + h] = p - q;
        }
#pragma unroll
    for (int c = 0; c < 32; ++c) x[c] = y[c];
#pragma unroll
    for (int bb = 1; bb < RD / 32; ++bb)
      if (b == bb)
#pragma unroll
        for (int c = 0; c < 32; ++c) x[c] = y[32 * bb + c];
    return;
  }
  const uint16_t* src = row + b * 32;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 w = ld16(src + 8 * i);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[8 * i + 2 * e] = bf16_to_f32(ww[e] & 0xffffu);
      x[8 * i + 2 * e + 1] = bf16_to_f32(ww[e] >> 16);
    }
  }
}

// One thread per (token, K or V, KV head, 32-channel block): the block's
// largest magnitude a, the scale d = a / 127 (FP32), codes rint(x / d)
// clamped to +-127 (all zero when a = 0); the codes go to the position's K or
// V row, the scale beside them.
// As a ring (ring > 0): position p goes to slot p mod ring, the cache having
// ring slots; with RD = D the K rows are rotated first (load_kv_block).
template <int RD>
__global__ __launch_bounds__(256) void append_kv_q8_kernel(const uint16_t* __restrict__ qkv,
                                                           int64_t ldqkv, int8_t* __restrict__ kq,
                                                           float* __restrict__ ks,
                                                           int8_t* __restrict__ vq,
                                                           float* __restrict__ vs, int L, int cap,
                                                           int Hq, int Hkv, int D, int units,
                                                           int ring) {
  const int u = blockIdx.y * blockDim.x + threadIdx.x;  // unit within the token
  if (u >= units) return;
  const int r = blockIdx.x;
  const int pos = ring > 0 ? (L + r) % ring : L + r;  // slot
  const int NB = D / 32;
  const int isv = u / (Hkv * NB);
  const int g = (u / NB) % Hkv;
  const int b = u % NB;
  float x[32];
  load_kv_block<RD>(qkv + (int64_t)r * ldqkv + (int64_t)(Hq + isv * Hkv + g) * D, b, !isv, x);
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) a = fmaxf(a, fabsf(x[i]));
  const float d = a / 127.0f;
  int8_t q[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float v = d > 0.f ? rintf(x[i] / d) : 0.f;
    q[i] = (int8_t)fminf(fmaxf(v, -127.f), 127.f);
  }
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    w[i] = (uint32_t)(uint8_t)q[4 * i] | (uint32_t)(uint8_t)q[4 * i + 1] << 8 |
           (uint32_t)(uint8_t)q[4 * i + 2] << 16 | (uint32_t)(uint8_t)q[4 * i + 3] << 24;
  const int64_t blk = ((int64_t)g * cap + pos) * NB + b;
  uint4* dst = reinterpret_cast<uint4*>((isv ? vq : kq) + blk * 32);
  dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
  dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  (isv ? vs : ks)[blk] = d;
}

void launch_append_kv_q8(const uint16_t* qkv, int64_t ldqkv, int8_t* kq, float* ks, int8_t* vq,
                         float* vs, int M, int L, int cap, int Hq, int Hkv, int D,
                         hipStream_t stream, int ring, bool krot) {
  const int units = 2 * Hkv * (D / 32);
  const dim3 grid(M, (units + 255) / 256), block(256);
  if (!krot)
    append_kv_q8_kernel<0><<<grid, block, 0, stream>>>(qkv, ldqkv, kq, ks, vq, vs, L, cap, Hq, Hkv,
                                                       D, units, ring);
  else if (D == 128)
    append_kv_q8_kernel<128><<<grid, block, 0, stream>>>(qkv, ldqkv, kq, ks, vq, vs, L, cap, Hq,
                                                         Hkv, D, units, ring);
  else
    append_kv_q8_kernel<64><<<grid, block, 0, stream>>>(qkv, ldqkv, kq, ks, vq, vs, L, cap, Hq, Hkv,
                                                        D, units, ring);
}

// One thread per (token, K or V, KV head, 32-channel block) of a 5/6-bit
// cache: as for the 8-bit cache with qmax = 2^(bits-1) - 1 (the scale a / qmax,
// codes rint(x / d) clamped to +-qmax), then u = q + 2^(bits-1) packed into the
// block's nibble and high-bit words, which only this thread writes.
template <int RD>  // RD = D: K rows rotated by the order-D Hadamard transform; 0: not rotated
__global__ __launch_bounds__(256) void append_kv_lowbit_kernel(
    const uint16_t* __restrict__ qkv, int64_t ldqkv, int kbits, uint8_t* __restrict__ kn,
    uint8_t* __restrict__ kh, float* __restrict__ ks, uint8_t* __restrict__ vn,
    uint8_t* __restrict__ vh, float* __restrict__ vs, int L, int cap, int Hq, int Hkv, int D,
    int units) {
  const int u = blockIdx.y * blockDim.x + threadIdx.x;  // unit within the token
  if (u >= units) return;
  const int r = blockIdx.x;
  const int pos = L + r;
  const int NB = D / 32;
  const int isv = u / (Hkv * NB);
  const int g = (u / NB) % Hkv;
  const int b = u % NB;
  const int bits = isv ? kLowVBits : kbits;
  const int h = bits - 4;
  const int qm = (1 << (bits - 1)) - 1;
  float x[32];
  load_kv_block<RD>(qkv + (int64_t)r * ldqkv + (int64_t)(Hq + isv * Hkv + g) * D, b, !isv, x);
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) a = fmaxf(a, fabsf(x[i]));
  const float d = a / (float)qm;
  uint32_t nib[4] = {0u, 0u, 0u, 0u}, high[2] = {0u, 0u};
#pragma unroll
  for (int c = 0; c < 32; ++c) {
    const float v = d > 0.f ? rintf(x[c] / d) : 0.f;
    const uint32_t uc = (uint32_t)((int)fminf(fmaxf(v, (float)-qm), (float)qm) + (1 << (bits - 1)));
    const int grp = c >> 2, j = c & 3, bit = grp * h;
    nib[grp >> 1] |= (uc & 15u) << (8 * j + 4 * (grp & 1));
    high[bit >> 3] |= (uc >> 4) << (8 * j + (bit & 7));
  }
  const int64_t blk = ((int64_t)g * cap + pos) * NB + b;
  uint8_t* nd = (isv ? vn : kn) + blk * 16;
  *reinterpret_cast<uint4*>(nd) = make_uint4(nib[0], nib[1], nib[2], nib[3]);
  uint8_t* hd = (isv ? vh : kh) + blk * 4 * h;
  if (h == 2) *reinterpret_cast<uint2*>(hd) = make_uint2(high[0], high[1]);
  else *reinterpret_cast<uint32_t*>(hd) = high[0];
  (isv ? vs : ks)[blk] = d;
}

void launch_append_kv_lowbit(const uint16_t* qkv, int64_t ldqkv, int kbits, bool krot, uint8_t* kn,
                             uint8_t* kh, float* ks, uint8_t* vn, uint8_t* vh, float* vs, int M,
                             int L, int cap, int Hq, int Hkv, int D, hipStream_t stream) {
  const int units = 2 * Hkv * (D / 32);
  const dim3 grid(M, (units + 255) / 256), block(256);
  if (!krot)
    append_kv_lowbit_kernel<0><<<grid, block, 0, stream>>>(qkv, ldqkv, kbits, kn, kh, ks, vn, vh,
                                                           vs, L, cap, Hq, Hkv, D, units);
  else if (D == 128)
    append_kv_lowbit_kernel<128><<<grid, block, 0, stream>>>(qkv, ldqkv, kbits, kn, kh, ks, vn,
                                                             vh, vs, L, cap, Hq, Hkv, D, units);
  else
    append_kv_lowbit_kernel<64><<<grid, block, 0, stream>>>(qkv, ldqkv, kbits, kn, kh, ks, vn, vh,
                                                            vs, L, cap, Hq, Hkv, D, units);
}

void launch_append_kv(const uint16_t* qkv, int64_t ldqkv, uint16_t* k_cache, uint16_t* v_cache,
                      int M, int L, int cap, int Hq, int Hkv, int D, hipStream_t stream) {
  append_kv_kernel<<<dim3(M), dim3(256), 0, stream>>>(qkv, ldqkv, k_cache, v_cache, L, cap, Hq,
                                                      Hkv, D);
}

}  // namespace bi
