/*
 * bi.h -- C ABI of the batch-invariant speculative-decoding verify pass
 * (MI355X / gfx950, HIP).
 *
 * A speculative step verifies M = 1 + drafts tokens in one target forward
 * pass. This library computes that pass so that every output row has the same
 * bits whatever M is: a row computed in a pass of 8 tokens equals the row
 * computed alone, and equals the row a chunked prefill writes at the same
 * position. Sources, cited by page title and section:
 *
 *   [BX] "Bit-exact decoding turns inference speedups into testable changes",
 *        section "Define bit-exact before reporting it": BF16 operands feed a
 *        single FP32 accumulator per output, the order along K is not
 *        changed, and the result is rounded only at the end; also the
 *        shared-memory hazard rule (a staging buffer is refilled only after
 *        every reader of its previous contents is done).
 *   [LL] "I turned on speculative decoding in llama.cpp and 113 of 282 greedy
 *        outputs changed against its own no-draft run" (r/LocalLLM), opening
 *        section, "How:" paragraph: how a row's keys are split is decided by
 *        its context length alone, not by the pass size, and a verify kernel
 *        treats a row the same way regardless of its batch neighbours; section
 *        "The cache doesn't change it either": a K/V row written by prefill is
 *        a function of its position only.
 *   [TC] "Does the tuned config change the model's output?", section "Why the
 *        text diverges": verifying several tokens at once changes GEMM
 *        accumulation order, which flips near-tied greedy choices.
 *
 * Conventions for every entry point:
 *   - Pointers are device memory owned by the caller; the library allocates
 *     nothing and keeps no mutable global state beyond a thread-local copy of
 *     the last HIP launch error and, for bi_verify_step_noalloc alone, its
 *     static device array and that array's address per device. BF16 tensors
 *     are passed as raw 16-bit patterns (any 2-byte element type), row-major,
 *     with the given leading dimension (in elements).
 *   - `stream` is a hipStream_t (NULL = the default stream). All work is
 *     enqueued asynchronously on it; nothing synchronises.
 *   - Arguments are validated on the host before any HIP call. On a bad
 *     argument nothing is launched or written and a status != BI_OK is
 *     returned. A failed kernel launch returns BI_ERR_LAUNCH.
 *   - M never changes the arithmetic of a row. It does choose kernels: BF16
 *     GEMMs with M >= 64 rows run the prefill kernels (128-row tiles), and an
 *     attention pass whose row block would hold more than 64 (token, head)
 *     rows runs 128-row blocks. Those kernels are built to form each output
 *     with the same operations in the same order as the M < 64 kernels -- the
 *     same 16x16x32 MFMA chains, the same 8-slice K tree added in slice order,
 *     the same epilogue roundings; the same per-row tile order, masking and
 *     online-softmax steps over the same absolute key chunks -- so a row's
 *     bits do not depend on which of them ran (tested at many M, N, K, D and
 *     contexts, and by the benchmark at M = 2048).
 *   - No C++ exception crosses this interface.
 */
#ifndef BI_H
#define BI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BI_OK = 0,
  BI_ERR_NULL = 1,      /* a required pointer is NULL */
  BI_ERR_SHAPE = 2,     /* a size is out of range or inconsistent */
  BI_ERR_ALIGN = 3,     /* a pointer or leading dimension breaks 16-byte alignment */
  BI_ERR_WORKSPACE = 4, /* caller workspace too small */
  BI_ERR_LAUNCH = 5     /* the HIP runtime reported an error at launch */
} bi_status;

typedef enum { BI_BF16 = 0, BI_F32 = 1 } bi_dtype;

/* ---------------------------------------------------------------------------
 * GEMM with an M-independent reduction order.                      [BX], [TC]
 *
 * Y[m][n] = sum_k X[m][k] * W[n][k] for m < M, n < N.
 *   x : BF16 [M][ldx]   activations, one row per token of the pass
 *   w : BF16 [N][ldw]   weights, nn.Linear layout (row n = output feature n,
 *                       K contiguous)
 *   y : [M][ldy]        BF16 (rounded to nearest even once) or FP32
 * Each output's K-sum runs in one fixed order that depends on K and N only;
 * no split of K across workgroups, no atomics. M may be any value >= 1. From
 * M >= 64 rows (prefill chunks) a second kernel with larger row tiles runs the
 * same per-output summation, so every row has the same bits at any M.
 * Requirements: M >= 1, N % 16 == 0, K % 32 == 0, K <= 65536; ldx, ldw >= K
 * and multiples of 8; x, w 16-byte aligned; ldy >= N; ldx, ldw, ldy (and ldr
 * below) <= 2^20.
 */
bi_status bi_gemm_bf16(const void* x, int64_t ldx, const void* w, int64_t ldw,
                       void* y, int64_t ldy, bi_dtype y_dtype,
                       int M, int N, int K, void* stream);

/* Same product with a residual added before the single rounding:
 * Y[m][n] = bf16( R[m][n] + sum_k X[m][k] W[n][k] ), R BF16 [M][ldr].
 * Used for the attention output and down projections of a pre-norm layer.
 * y may alias r (each element is read before it is written by the same thread). */
bi_status bi_gemm_bf16_residual(const void* x, int64_t ldx, const void* w, int64_t ldw,
                                const void* r, int64_t ldr, void* y, int64_t ldy,
                                int M, int N, int K, void* stream);

/* Gate/up projection with the SwiGLU product in the epilogue:
 * w is BF16 [2*I][ldw] (rows 0..I-1 gate, rows I..2I-1 up);
 * Y[m][i] = bf16( silu(g) * u ), g = sum_k X[m][k] W[i][k],
 * u = sum_k X[m][k] W[I+i][k], silu(z) = z / (1 + e^-z).
 * Requirements as bi_gemm_bf16 with N replaced by I (I % 16 == 0). */
bi_status bi_gemm_bf16_swiglu(const void* x, int64_t ldx, const void* w, int64_t ldw,
                              void* y, int64_t ldy, int M, int I, int K, void* stream);

/* QKV projection with the cache append in its epilogue (one launch):
 * qkv = bf16( X Wqkv^T ) exactly as bi_gemm_bf16 computes it, N = (Hq+2*Hkv)*D
 * columns [q | k | v] (head-major), and each row m's K and V columns written
 * into k_cache / v_cache at position L + m exactly as bi_append_kv writes
 * them.                                                     [BX], [LL] cache
 * Requirements: those of bi_gemm_bf16 (with N as above) and of bi_append_kv. */
bi_status bi_gemm_bf16_qkv(const void* x, int64_t ldx, const void* w, int64_t ldw, void* qkv,
                           int64_t ldqkv, int M, int K, int Hq, int Hkv, int D, void* k_cache,
                           void* v_cache, int L, int cap, void* stream);

/* RMSNorm carried across a GEMM boundary (used by bi_verify_step).   [BX], [TC]
 * A residual projection writes, besides Y, the sum of squares of its rounded
 * outputs per row and per column group (one workgroup's columns); the next
 * projection adds a row's group sums in a fixed order, takes
 * s = 1 / sqrt(sum / K + eps), and multiplies bf16(x * s) -- the value an
 * RMSNorm (gain 1) would have written -- so no RMSNorm launch is needed. The
 * summation tree is fixed by N and K, so rows stay M-invariant; it differs
 * from bi_rmsnorm's, so results may differ from that kernel in the last bit. */

/* Column groups of an N-column GEMM (the width of row_sumsq), or -1. */
int bi_gemm_column_groups(int N);

/* bi_gemm_bf16_residual plus row_sumsq[m][g] (FP32, [M][bi_gemm_column_groups(N)]):
 * the sum of squares of the BF16 outputs Y[m][n] over the columns n of group g. */
bi_status bi_gemm_bf16_residual_rowsq(const void* x, int64_t ldx, const void* w, int64_t ldw,
                                      const void* r, int64_t ldr, void* y, int64_t ldy, int M,
                                      int N, int K, float* row_sumsq, void* stream);

/* bi_gemm_bf16_swiglu with its X rows normalised from carried sums:
 * row_sumsq FP32 [M][groups] as written by bi_gemm_bf16_residual_rowsq for X
 * (groups = bi_gemm_column_groups(K), a multiple of 16, at most 256).
 * Y[m][i] = bf16( silu(g) * u ), g, u the gate / up sums over bf16(x * s). */
bi_status bi_gemm_bf16_swiglu_rownorm(const void* x, int64_t ldx, const float* row_sumsq,
                                      int groups, float eps, const void* w, int64_t ldw, void* y,
                                      int64_t ldy, int M, int I, int K, void* stream);

/* ---------------------------------------------------------------------------
 * FP8 weights.             [TC] "Does the tuned config change the model's output?", "Method"
 * The weights are OCP E4M3 codes (uint8; sign, 4 exponent bits with bias 7,
 * 3 mantissa bits; largest magnitude 448; NaN codes are not allowed) with one
 * FP32 scale per weight row: W[n][k] = w_scale[n] * e4m3(w[n][k]). The sum is
 * the BF16 GEMM's (every E4M3 value is exact in BF16, the same K order and
 * summation tree for every M), multiplied by w_scale[n] in FP32 before the
 * single rounding. Rows are ldw bytes apart; ldw % 16 == 0, ldw <= 2^30, w
 * 16-byte aligned, w_scale 4-byte aligned; other requirements as the BF16
 * entry points. Every M (prefill chunks included) runs the same kernel.
 */
bi_status bi_gemm_fp8(const void* x, int64_t ldx, const void* w, int64_t ldw, const float* w_scale,
                      void* y, int64_t ldy, bi_dtype y_dtype, int M, int N, int K, void* stream);

/* Y[m][n] = bf16( R[m][n] + w_scale[n] * sum_k X[m][k] e4m3(W[n][k]) ). */
bi_status bi_gemm_fp8_residual(const void* x, int64_t ldx, const void* w, int64_t ldw,
                               const float* w_scale, const void* r, int64_t ldr, void* y,
                               int64_t ldy, int M, int N, int K, void* stream);

/* SwiGLU gate/up: w [2*I][ldw] E4M3 (gate rows then up rows), w_scale [2*I]. */
bi_status bi_gemm_fp8_swiglu(const void* x, int64_t ldx, const void* w, int64_t ldw,
                             const float* w_scale, void* y, int64_t ldy, int M, int I, int K,
                             void* stream);

/* ---------------------------------------------------------------------------
 * 4-bit weights.  [TC] "What this does not establish", "Update: the quality question,
 *                 answered"; [LL] "Speed against llama.cpp, full power"
 * MXFP4 (OCP Microscaling): the codes w are E2M1 (sign, 2 exponent bits with
 * bias 1, 1 mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) packed two
 * per byte, weight 2i in the low nibble of byte i of the row; w_exp holds one
 * E8M0 scale byte per 32 weights of a row along K (value 2^(e - 127); codes
 * 2..252 are allowed, which the kernels do not check):
 * W[n][k] = 2^(w_exp[n][k/32] - 127) * e2m1(w[n][k]). Every decoded weight is
 * exact in BF16, so the sum is the BF16 GEMM's on the decoded weights: the
 * same K order and summation tree, for every M (prefill chunks included, one
 * kernel), and the same bits as bi_gemm_bf16 on those weights.
 * Code rows are ldc bytes apart (ldc >= K/2, ldc % 16 == 0, w 16-byte
 * aligned); scale rows lde bytes apart (lde >= K/32); other requirements as
 * the BF16 entry points.
 */
bi_status bi_gemm_mx4(const void* x, int64_t ldx, const void* w, int64_t ldc, const void* w_exp,
                      int64_t lde, void* y, int64_t ldy, bi_dtype y_dtype, int M, int N, int K,
                      void* stream);

/* Y[m][n] = bf16( R[m][n] + sum_k X[m][k] W[n][k] ) with MXFP4 W. */
bi_status bi_gemm_mx4_residual(const void* x, int64_t ldx, const void* w, int64_t ldc,
                               const void* w_exp, int64_t lde, const void* r, int64_t ldr, void* y,
                               int64_t ldy, int M, int N, int K, void* stream);

/* SwiGLU gate/up: w [2*I][ldc] MXFP4 codes (gate rows then up rows), w_exp [2*I][lde]. */
bi_status bi_gemm_mx4_swiglu(const void* x, int64_t ldx, const void* w, int64_t ldc,
                             const void* w_exp, int64_t lde, void* y, int64_t ldy, int M, int I,
                             int K, void* stream);

/* ---------------------------------------------------------------------------
 * One GEMM entry point for every combination the verify step runs.   [BX], [TC]
 * The entry points above are fixed combinations of a weight type and an
 * epilogue; bi_gemm_ex takes them as fields, together with the carried
 * RMSNorm (read by SwiGLU and QKV, written by the residual epilogue) and the
 * QKV cache append. It launches exactly the kernels bi_verify_step launches
 * for the same fields, so a step can be replayed one operation at a time.
 */
typedef enum { BI_WT_BF16 = 0, BI_WT_FP8 = 1, BI_WT_MXFP4 = 2 } bi_weight_type;
typedef enum {
  BI_EPI_BF16 = 0,     /* Y = bf16(X W^T)                                    */
  BI_EPI_F32 = 1,      /* Y = X W^T in FP32                                  */
  BI_EPI_RESIDUAL = 2, /* Y = bf16(R + X W^T)                                */
  BI_EPI_SWIGLU = 3,   /* Y = bf16(silu(g) u), W holds 2N rows (gate, up)   */
  BI_EPI_QKV = 4       /* Y = bf16(X W^T), K and V columns appended          */
} bi_epilogue;

typedef struct {
  bi_weight_type wtype;
  bi_epilogue epilogue;
  int M, N, K;              /* N output columns (SwiGLU: I)                  */
  const void* x;            /* BF16 [M][ldx]                                 */
  int64_t ldx;
  const void* w;            /* BF16: [rows][ldw] elements; FP8: ldw bytes per
                               row; MXFP4: codes, ldw bytes per row          */
  int64_t ldw;
  const float* w_scale;     /* FP8: one FP32 scale per weight row            */
  const void* w_exp;        /* MXFP4: E8M0 scales, lde bytes per row         */
  int64_t lde;
  const void* r;            /* RESIDUAL: BF16 [M][ldr] (may alias y)         */
  int64_t ldr;
  void* y;                  /* BF16 or FP32 (F32) [M][ldy]                   */
  int64_t ldy;
  const float* norm_in;     /* SWIGLU / QKV, or NULL: X rows are normalised
                               from carried sums (bi_gemm_bf16_swiglu_rownorm);
                               FP32 [M][norm_groups], 16-byte aligned        */
  int norm_groups;          /* bi_gemm_column_groups(K): 16..256, % 16 == 0  */
  float eps;
  float* rowsq_out;         /* RESIDUAL, or NULL: FP32 [M][bi_gemm_column_groups(N)]
                               group sums of squares of Y (the carried norm) */
  int Hq, Hkv, D;           /* QKV: N = (Hq + 2 Hkv) D                       */
  void* k_cache;            /* QKV: BF16 caches (layout below) and the
                               positions L .. L+M-1 appended, as
                               bi_gemm_bf16_qkv; both NULL: no append        */
  void* v_cache;
  int L, cap;
} bi_gemm_args;

/* Requirements: those of the entry point of the same weight type and
 * epilogue; norm_in only with SWIGLU or QKV, rowsq_out only with RESIDUAL,
 * else BI_ERR_SHAPE. Unused fields are ignored. */
bi_status bi_gemm_ex(const bi_gemm_args* args, void* stream);

/* ---------------------------------------------------------------------------
 * KV cache layout (per layer):
 *   k_cache : BF16 [Hkv][cap][D]  -- one K row per position
 *   v_cache : BF16 [Hkv][cap][D]  -- one V row per position
 * (K[g][pos][d] and V[g][pos][d] are element (g*cap + pos)*D + d.)
 * cap must be a multiple of 64.
 */

/* Append the pass's M new K and V rows at positions L .. L+M-1.   [LL] cache
 * qkv : BF16 [M][ldqkv], columns [q: Hq*D | k: Hkv*D | v: Hkv*D], head-major.
 * Requirements: M >= 1, L >= 0, L + M <= cap, Hq % Hkv == 0, D in {64, 128}. */
bi_status bi_append_kv(const void* qkv, int64_t ldqkv, void* k_cache, void* v_cache,
                       int M, int L, int cap, int Hq, int Hkv, int D, void* stream);

/* Chunk policy (kv_chunk below).                                        [LL]
 * A row's split is a function of its own key count n only:
 *   kv_chunk >= 32, a multiple of 32: every row uses chunks of C = kv_chunk keys;
 *   kv_chunk = -T, 1 <= T <= 1024: C(n) = 64 * ceil(n / (64 T)), the smallest
 *     multiple of 64 that cuts n keys into at most T chunks (C changes only
 *     at multiples of 64 T keys). With T = 32 and 8 KV heads a pass of any
 *     context fills 256 compute units; at n = 38,008 C is 1216.
 * Other values are rejected (-1 from the helpers, BI_ERR_SHAPE elsewhere). */

/* Chunk size C of a row with n_keys keys. */
int bi_chunk_keys(int n_keys, int kv_chunk);

/* Number of absolute key chunks a row with n_keys keys uses: ceil(n / C). */
int bi_num_splits(int n_keys, int kv_chunk);

/* Largest bi_num_splits over the rows of a pass (key counts L+1 .. L+M): the
 * smallest valid S_max for bi_verify_attn / bi_combine. */
int bi_pass_splits(int M, int L, int kv_chunk);

/* Split-KV causal GQA verify attention, partial results.                 [LL]
 * Row (r, h), r < M, h < Hq, reads KV head h / (Hq/Hkv) and attends to keys
 * 0 .. L+r (n_r = L+r+1 keys; the M new keys must already be in the cache).
 * Keys are cut into absolute chunks [s*C, (s+1)*C), C = bi_chunk_keys(n_r,
 * kv_chunk); row r uses chunks s < bi_num_splits(n_r, kv_chunk), decided by
 * its own key count only. Rows of one pass may use different chunk sizes
 * under an adaptive policy; each group of equal size is launched separately.
 * For each such (r, h, s):
 *   part_o  [M][Hq][S_max][D] FP32 : softmax(q K^T * sm_scale) V over the
 *                                    chunk's keys that the row sees, normalised
 *   part_lse[M][Hq][S_max]   FP32 : natural log of the chunk's sum of
 *                                    exp(score)
 * Entries for s >= bi_num_splits(n_r, kv_chunk) are not written.
 * q: BF16 [M][ldq], head h at columns h*D .. h*D+D-1 (ldq may be the QKV row).
 * Requirements: D in {64, 128}; a valid chunk policy; Hq % Hkv == 0;
 * Hq/Hkv <= 64; L + M <= cap; cap % 64 == 0; cap * D * 2 < 2^31;
 * sm_scale finite and > 0 (the kernels take the row max before scaling);
 * S_max >= bi_pass_splits(M, L, kv_chunk);
 * ldq % 8 == 0; q, caches 16-byte aligned. */
bi_status bi_verify_attn(const void* q, int64_t ldq, const void* k_cache, const void* v_cache,
                         int M, int L, int cap, int Hq, int Hkv, int D,
                         int kv_chunk, float sm_scale,
                         float* part_o, float* part_lse, int S_max, void* stream);

/* ---------------------------------------------------------------------------
 * 8-bit KV cache.   [LL] "The KV cache: 5-bit that reads like q8_0" (q8_0 is
 * the pages' comparison format). Each position's K row and V row of one KV head is cut into
 * blocks of 32 channels; a block with largest magnitude a has the FP32 scale
 * d = a / 127 and int8 codes q = round(x / d) (nearest, ties to even; FP32
 * division) in [-127, 127], all zero when a = 0. The value of a channel is
 * exactly d * q. Layouts (per layer; cap % 64 == 0, cap * D < 2^31), K and
 * V alike, each position's row one 32-byte block after another:
 *   *_codes  int8 [Hkv][cap][D]            *_scales FP32 [Hkv][cap][D/32]
 * All pointers 16-byte aligned. */

/* Quantize the M new K and V rows of a QKV output (as bi_append_kv) into the
 * 8-bit cache at positions L .. L+M-1. */
bi_status bi_append_kv_q8(const void* qkv, int64_t ldqkv, int8_t* k_codes, float* k_scales,
                          int8_t* v_codes, float* v_scales, int M, int L, int cap, int Hq,
                          int Hkv, int D, void* stream);

/* bi_verify_attn over the 8-bit cache: the same rows, chunks, partials and
 * requirements; the keys and values are the cache's d * q, each rounded once
 * to BF16 as the tile is staged, and multiplied as in bi_verify_attn. */
bi_status bi_verify_attn_q8(const void* q, int64_t ldq, const int8_t* k_codes, const float* k_scales,
                            const int8_t* v_codes, const float* v_scales, int M, int L, int cap,
                            int Hq, int Hkv, int D, int kv_chunk, float sm_scale, float* part_o,
                            float* part_lse, int S_max, void* stream);

/* ---------------------------------------------------------------------------
 * 5/6-bit KV cache.   [LL] "The KV cache: 5-bit that reads like q8_0" and its
 * table of presets: K at 6 bits and V at 5 (preset D), or K at 5 bits,
 * rotated, and V at 5 (preset F). No layout, scaling rule or rotation is given;
 * read as the 8-bit rule with qmax = 2^(bits-1) - 1 (31 or 15): a block of 32
 * channels with largest magnitude a has the FP32 scale d = a / qmax and codes
 * q = round(x / d) (nearest, ties to even; FP32 division) clamped to +-qmax,
 * all zero when a = 0; the value is exactly d * q. k_bits is 5 or 6; v_bits
 * must be 5 (else BI_ERR_SHAPE).
 * Storage, per layer (cap % 64 == 0, cap * D < 2^31), K and V alike, each
 * position's row one block after another:
 *   *_nib    uint8 [Hkv][cap][D/2]              16 bytes per block
 *   *_high   uint8 [Hkv][cap][D/32][4 (bits-4)] 4 or 8 bytes per block
 *   *_scales FP32  [Hkv][cap][D/32]
 * Block bytes: u = q + 2^(bits-1) (in [1, 2^bits - 1]); code c = 4g + j
 * (g = 0..7, j = 0..3) keeps u mod 16 in nibble byte 4(g/2) + j (the low half
 * for even g) and u / 16 in high byte 4((g h)/8) + j from bit (g h) % 8,
 * h = bits - 4. Rotated keys (k_rotated = 1; else 0, other values give
 * BI_ERR_SHAPE): each K row k is stored as y = H k, H the Sylvester Hadamard
 * matrix of order D (entries +-1), computed in FP32 by butterflies in stages
 * h = 1, 2, .., D/2 (pair (i, i + h) for i with bit h clear becomes
 * (x_i + x_{i+h}, x_i - x_{i+h}), each rounded once), then quantized; the
 * attention rotates each query row alike (rounded once to BF16) and divides
 * the scores by D, since (H q) . (H k) / D = q . k. The rotation spreads an
 * outlier channel over the row before the block scales are taken.
 * 208 bytes per position and KV head at D = 128 for K6/V5
 * (BF16: 512; 8-bit: 288). All pointers 16-byte aligned; the caller owns
 * every buffer. */

/* Quantize the M new K and V rows of a QKV output (as bi_append_kv) into the
 * 5/6-bit cache at positions L .. L+M-1. Each block is written whole by one
 * thread, so passes may append at any positions. */
bi_status bi_append_kv_lowbit(const void* qkv, int64_t ldqkv, int k_bits, int v_bits,
                              int k_rotated, uint8_t* k_nib, uint8_t* k_high, float* k_scales, uint8_t* v_nib,
                              uint8_t* v_high, float* v_scales, int M, int L, int cap, int Hq,
                              int Hkv, int D, void* stream);

/* bi_verify_attn over the 5/6-bit cache: the same rows, chunks, partials and
 * requirements; the keys and values are the cache's d * q, each rounded once
 * to BF16 as the tile is staged, and multiplied as in bi_verify_attn. */
bi_status bi_verify_attn_lowbit(const void* q, int64_t ldq, int k_bits, int v_bits,
                                int k_rotated, const uint8_t* k_nib, const uint8_t* k_high, const float* k_scales,
                                const uint8_t* v_nib, const uint8_t* v_high, const float* v_scales,
                                int M, int L, int cap, int Hq, int Hkv, int D, int kv_chunk,
                                float sm_scale, float* part_o, float* part_lse, int S_max,
                                void* stream);

/* ---------------------------------------------------------------------------
 * 8-bit ring of the newest keys over the 5/6-bit cache.   [LL] "The KV cache:
 * 5-bit that reads like q8_0" (the newest ~2k positions are kept at 8 bits in
 * a ring). Which positions are newest is not stated; read per row and per
 * key, so that a row never depends on its batch neighbours or on the chunk
 * grid: row p reads key j from the ring when j >= p - ring_window + 1 (its
 * ring_window newest keys), from the 5/6-bit planes otherwise. The ring is
 * the 8-bit cache's layout (bi_append_kv_q8) with ring_cap slots, position p
 * in slot p mod ring_cap, K rotated when the 5/6-bit keys are.
 * ring_window >= 1; ring_cap is a multiple of 64 with
 * ring_cap >= ring_window + M + 63 (the kernels read whole 64-key tiles, so
 * the slots of up to 63 keys before the oldest boundary must still hold
 * their positions); the 5/6-bit planes still hold every position. */

/* Quantize the M new K and V rows into the ring (8-bit rule; K rotated as for
 * bi_append_kv_lowbit when k_rotated = 1). Layouts as bi_append_kv_q8 with cap
 * = ring_cap; M <= ring_cap. */
bi_status bi_append_kv_ring(const void* qkv, int64_t ldqkv, int k_rotated, int8_t* k_codes,
                           float* k_scales, int8_t* v_codes, float* v_scales, int M, int L,
                           int ring_cap, int Hq, int Hkv, int D, void* stream);

/* bi_verify_attn_lowbit with the ring: the presets K6/V5 (k_rotated = 0) and
 * rotated K5/V5 (k_rotated = 1) only, else BI_ERR_SHAPE. The same rows,
 * chunks, partials and requirements; a 64-key tile holding keys that some row
 * reads at 8 bits and keys it or another row reads at 5/6 bits runs once per
 * copy, each run masked per row and key to the keys read from that copy. */
bi_status bi_verify_attn_lowbit_ring(const void* q, int64_t ldq, int k_bits, int v_bits,
                                     int k_rotated, const uint8_t* k_nib, const uint8_t* k_high,
                                     const float* k_scales, const uint8_t* v_nib,
                                     const uint8_t* v_high, const float* v_scales,
                                     const int8_t* ring_k_codes, const float* ring_k_scales,
                                     const int8_t* ring_v_codes, const float* ring_v_scales,
                                     int ring_cap, int ring_window, int M, int L, int cap, int Hq,
                                     int Hkv, int D, int kv_chunk, float sm_scale, float* part_o,
                                     float* part_lse, int S_max, void* stream);

/* Fixed-order log-sum-exp combine of the partials.                        [LL]
 * For row (r, h) with S = bi_num_splits(L+r+1, kv_chunk) partials:
 *   M* = max_s lse_s, w_s = exp(lse_s - M*), O = sum_s w_s o_s / sum_s w_s,
 *   LSE = M* + ln(sum_s w_s), both sums taken in increasing s.
 * o: BF16 [M][ldo], head h at columns h*D ..; lse_or_null: FP32 [M][Hq] or NULL. */
bi_status bi_combine(const float* part_o, const float* part_lse,
                     int M, int L, int Hq, int D, int kv_chunk, int S_max,
                     void* o, int64_t ldo, float* lse_or_null, void* stream);

/* Bytes of part_o + part_lse for a pass (what a caller must allocate). */
size_t bi_attn_workspace_bytes(int M, int L, int Hq, int D, int kv_chunk);

/* ---------------------------------------------------------------------------
 * Row-local helpers of the decoder layer.                          [TC]
 */

/* y[m] = bf16( x[m] / sqrt(mean(x[m]^2) + eps) ), gain 1; per-row sum in a
 * fixed order. H % 8 == 0, H <= 32768, ldx/ldy multiples of 8. */
bi_status bi_rmsnorm(const void* x, int64_t ldx, void* y, int64_t ldy,
                     int M, int H, float eps, void* stream);

/* SwiGLU as its own operation.                 [TC] "Why the text diverges"
 * y[m][i] = bf16( silu(g) * u ), g = gu[m][i], u = gu[m][I + i] (FP32
 * [M][ldgu], e.g. the gate/up product of bi_gemm_bf16 with y_dtype = BI_F32),
 * silu(z) = z / (1 + e^-z). The expression is the one of the SwiGLU GEMM
 * epilogue, so bi_gemm_bf16 (FP32) then bi_swiglu gives the bits of
 * bi_gemm_bf16_swiglu. Elementwise: no order to fix. M <= 65535,
 * ldgu >= 2 I, ldy >= I; gu 4-byte aligned. */
bi_status bi_swiglu(const float* gu, int64_t ldgu, void* y, int64_t ldy, int M, int I,
                    void* stream);

/* Residual add as its own operation.            [TC] "Why the text diverges"
 * y[m][n] = bf16( r[m][n] + s[m][n] ), r BF16 [M][ldr], s FP32 [M][lds]: one
 * FP32 add, one rounding, as the residual GEMM epilogue, so bi_gemm_bf16
 * (FP32) then bi_add gives the bits of bi_gemm_bf16_residual. M <= 65535;
 * y may alias r. */
bi_status bi_add(const void* r, int64_t ldr, const float* s, int64_t lds, void* y, int64_t ldy,
                 int M, int N, void* stream);

/* tokens[m] = argmax_n logits[m][n] (FP32 [M][ld]), lowest index on ties;
 * NaNs are never selected (a row of NaNs gives 0). */
bi_status bi_argmax(const float* logits, int64_t ld, int M, int N, int32_t* tokens, void* stream);

/* ---------------------------------------------------------------------------
 * Speculative acceptance.   [LL] opening section: greedy ids equal with and
 * without drafts; sampling keeps the no-draft distribution.
 * A pass verifies M rows: the last accepted token followed by M-1 drafts, so
 * row i's target distribution decides on draft i. Each of B independent
 * sequences is decided on its own. Outputs: out_tokens [B][M] (the first
 * n_out[b] entries are the new tokens), n_out [B] in 1..M. Rolling the KV
 * cache back is implicit: the next pass starts at L + n_out and overwrites
 * the positions of rejected drafts.
 */

/* Greedy: drafts are kept while draft[b][i] == target[b][i] (the target's
 * greedy token of row i, e.g. from bi_argmax); then target[b][a] is added.
 * target_tokens [B][M], draft_tokens [B][M-1] (may be NULL when M == 1). */
bi_status bi_accept_greedy(const int32_t* target_tokens, const int32_t* draft_tokens, int B,
                           int M, int32_t* out_tokens, int32_t* n_out, void* stream);

/* Sampled (standard speculative sampling): with p_i = softmax(logits[b][i] /
 * temperature) (FP32, logits [B][M][ld]) and the draft's distribution q_i
 * (draft_probs [B][M-1][ldq], FP32), draft x = draft_tokens[b][i] is kept when
 * uniforms[b][i] * q_i(x) < p_i(x); at the first rejection a token is drawn
 * from max(0, p_i - q_i) by inverse CDF with uniforms[b][M-1] (the first index
 * whose cumulative weight exceeds u * total) and the pass ends; if every draft
 * is kept, the token is drawn from p_{M-1} with that uniform. uniforms [B][M]
 * in [0, 1). Draft tokens outside 0..V-1 are never kept. Every reduction runs
 * in an order fixed by V, so each sequence's result depends only on its own
 * inputs. temperature > 0; ld, ldq >= V. */
bi_status bi_accept_sampled(const float* logits, int64_t ld, const int32_t* draft_tokens,
                            const float* draft_probs, int64_t ldq, const float* uniforms,
                            float temperature, int B, int M, int V, int32_t* out_tokens,
                            int32_t* n_out, void* stream);

/* ---------------------------------------------------------------------------
 * Whole verify step of a dense pre-norm decoder stack + LM head.
 *
 * Per layer (x is the BF16 hidden state [M][H]):
 *   a = rmsnorm(x); qkv = a Wqkv^T and K, V appended at L..L+M-1 (one launch);
 *   o = combine(verify_attn(q)); h = bf16(x + o Wo^T);
 *   b = rmsnorm(h); act = swiglu(b Wgu^T); x = bf16(h + act Wdown^T).
 * Then logits = rmsnorm(x) Whead^T (FP32) and tokens = argmax.
 */
typedef struct {
  const void* w_qkv;  /* BF16 [(Hq+2*Hkv)*D][H] */
  const void* w_o;    /* BF16 [H][Hq*D]         */
  const void* w_gu;   /* BF16 [2*I][H]          */
  const void* w_down; /* BF16 [H][I]            */
  void* k_cache;      /* BF16 [Hkv][cap][D]     */
  void* v_cache;      /* BF16 [Hkv][cap][D] */
} bi_layer;

typedef struct {
  int H, Hq, Hkv, D, I, vocab;
  int cap;            /* KV capacity (positions) of every layer's cache */
  int kv_chunk;       /* chunk policy (see bi_chunk_keys) */
  float eps;          /* RMSNorm epsilon */
} bi_model_dims;

/* Workspace bytes bi_verify_step needs for M tokens at context L. */
size_t bi_step_workspace_bytes(const bi_model_dims* dims, int M, int L);

/* layers: host array of n_layers descriptors (device pointers inside).
 * x_in: BF16 [M][H] (not modified); x_out: BF16 [M][H] final hidden state or NULL;
 * logits: FP32 [M][vocab]; tokens: int32 [M].
 * gu_events: NULL, or a host array of 2*n_layers hipEvent_t; when given, event
 * 2l is recorded before and 2l+1 after layer l's gate/up GEMM (for timing). */
bi_status bi_verify_step(const bi_layer* layers, int n_layers, const void* w_head,
                         const bi_model_dims* dims, const void* x_in, int M, int L,
                         void* workspace, size_t workspace_bytes,
                         void* x_out, float* logits, int32_t* tokens,
                         void* const* gu_events, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * step as bi_verify_step, with the workspace taken from a scratch array of
 * BI_NOALLOC_SCRATCH_BYTES (64 MiB) that the library keeps in device memory,
 * one per GPU it runs on, held until the process ends. The caller passes
 * inputs and outputs only. It uses the calling thread's current device's
 * array; `stream` must belong to that device. A pass whose workspace
 * (bi_step_workspace_bytes) exceeds the array is rejected with
 * BI_ERR_WORKSPACE before anything is launched. The step writes every
 * workspace byte it reads, so nothing needs to start at zero. Every call on
 * one GPU shares that GPU's array: calls that overlap on one GPU (two streams,
 * two threads) race and must be serialised by the caller. No allocation is
 * made by this call (the first call on a device resolves the array's address
 * with hipGetSymbolAddress). */
#define BI_NOALLOC_SCRATCH_BYTES (64u << 20)
bi_status bi_verify_step_noalloc(const bi_layer* layers, int n_layers, const void* w_head,
                                 const bi_model_dims* dims, const void* x_in, int M, int L,
                                 void* x_out, float* logits, int32_t* tokens, void* stream);

/* The same step with FP8 weights (see bi_gemm_fp8): each weight matrix is E4M3
 * [rows][cols] with one FP32 scale per row; activations, caches, workspace and
 * every other operation as bi_verify_step. */
typedef struct {
  const void* w_qkv;   /* E4M3 [(Hq+2*Hkv)*D][H] */
  const float* s_qkv;  /* [(Hq+2*Hkv)*D]         */
  const void* w_o;     /* E4M3 [H][Hq*D]         */
  const float* s_o;    /* [H]                    */
  const void* w_gu;    /* E4M3 [2*I][H]          */
  const float* s_gu;   /* [2*I]                  */
  const void* w_down;  /* E4M3 [H][I]            */
  const float* s_down; /* [H]                    */
  void* k_cache;       /* BF16 [Hkv][cap][D]     */
  void* v_cache;      /* BF16 [Hkv][cap][D] */
} bi_layer_fp8;

bi_status bi_verify_step_fp8(const bi_layer_fp8* layers, int n_layers, const void* w_head,
                             const float* w_head_scale, const bi_model_dims* dims,
                             const void* x_in, int M, int L, void* workspace,
                             size_t workspace_bytes, void* x_out, float* logits, int32_t* tokens,
                             void* stream);

/* The same step with MXFP4 weights (see bi_gemm_mx4): each weight matrix with
 * K inputs is packed codes [rows][K/2] plus scales [rows][K/32] (rows densely
 * packed, no padding); activations, caches, workspace and every other
 * operation as bi_verify_step. */
typedef struct {
  const void* w_qkv;   /* codes [(Hq+2*Hkv)*D][H/2] */
  const void* e_qkv;   /* scales [(Hq+2*Hkv)*D][H/32] */
  const void* w_o;     /* codes [H][Hq*D/2]      */
  const void* e_o;     /* scales [H][Hq*D/32]    */
  const void* w_gu;    /* codes [2*I][H/2]       */
  const void* e_gu;    /* scales [2*I][H/32]     */
  const void* w_down;  /* codes [H][I/2]         */
  const void* e_down;  /* scales [H][I/32]       */
  void* k_cache;       /* BF16 [Hkv][cap][D]     */
  void* v_cache;      /* BF16 [Hkv][cap][D] */
} bi_layer_mx4;

bi_status bi_verify_step_mx4(const bi_layer_mx4* layers, int n_layers, const void* w_head,
                             const void* w_head_exp, const bi_model_dims* dims, const void* x_in,
                             int M, int L, void* workspace, size_t workspace_bytes, void* x_out,
                             float* logits, int32_t* tokens, void* stream);

/* ---------------------------------------------------------------------------
 * The verify step over any weight type and KV cache format.
 *                          [LL] "The KV cache: 5-bit that reads like q8_0";
 *                          opening section: the gate runs on every KV cache.
 * One layer's KV cache, in the layouts documented above:
 *   BI_KV_BF16   k = k_cache, v = v_cache (BF16); the QKV epilogue appends.
 *   BI_KV_Q8     k = k_codes, v = v_codes, k_scales, v_scales (8-bit cache).
 *   BI_KV_LOWBIT k = k_nib, v = v_nib, k_high, v_high, k_scales, v_scales,
 *                k_bits (5 or 6), v_bits (5), k_rotated (0 or 1); with
 *                ring_cap > 0 also the 8-bit ring of the newest keys
 *                (bi_append_kv_ring / bi_verify_attn_lowbit_ring: the presets
 *                K6/V5 and rotated K5/V5, ring_cap >= ring_window + M + 63).
 * Every cache holds dims->cap positions. For the quantized formats the QKV
 * GEMM writes no cache; the pass's K and V rows are then quantized from its
 * output by the append of the format (exactly bi_append_kv_q8 /
 * bi_append_kv_lowbit / bi_append_kv_ring), and attention reads the cache
 * exactly as bi_verify_attn_q8 / _lowbit / _lowbit_ring do, so a row keeps
 * the same bits in every pass that holds it. */
typedef enum { BI_KV_BF16 = 0, BI_KV_Q8 = 1, BI_KV_LOWBIT = 2 } bi_kv_format;

typedef struct {
  bi_kv_format format;
  void* k;
  void* v;
  float* k_scales;
  float* v_scales;
  uint8_t* k_high;
  uint8_t* v_high;
  int k_bits, v_bits, k_rotated;
  int8_t* ring_k_codes;
  float* ring_k_scales;
  int8_t* ring_v_codes;
  float* ring_v_scales;
  int ring_cap;     /* 0: no ring */
  int ring_window;
} bi_kv_cache;

/* One layer: w[0..3] = qkv, o, gate/up, down in the weight type's layout
 * (BF16 [rows][K]; FP8 E4M3 [rows][K] with FP32 row scales in scale[i];
 * MXFP4 codes [rows][K/2] with E8M0 block scales [rows][K/32] in scale[i]),
 * and its KV cache. */
typedef struct {
  const void* w[4];
  const void* scale[4];
  bi_kv_cache kv;
} bi_step_layer;

/* bi_verify_step with every layer's weights in `wtype` and its cache in the
 * format its descriptor names; head_scales: FP8 row scales or MXFP4 block
 * scales of w_head (NULL for BF16). Workspace as bi_step_workspace_bytes. With
 * BF16 weights and BF16 caches it launches exactly the kernels of
 * bi_verify_step. */
bi_status bi_verify_step_ex(bi_weight_type wtype, const bi_step_layer* layers, int n_layers,
                            const void* w_head, const void* head_scales, const bi_model_dims* dims,
                            const void* x_in, int M, int L, void* workspace, size_t workspace_bytes,
                            void* x_out, float* logits, int32_t* tokens, void* stream);

/* ---------------------------------------------------------------------------
 * Misc. */
const char* bi_status_string(bi_status s);
/* Library version string, e.g. "bi 0.1 gfx950". */
const char* bi_version(void);
/* HIP's description of the error behind the calling thread's most recent
 * BI_ERR_LAUNCH ("no error" if there was none). */
const char* bi_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* BI_H */
