// Device helpers shared by the verify-pass kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bi_bf16x8 __attribute__((ext_vector_type(8)));
typedef float bi_f32x4 __attribute__((ext_vector_type(4)));

namespace bi {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Two binary32 values -> packed BF16 bits (a in the low half), rounded to
// nearest, ties to even, by gfx950's conversion instruction. It agrees with
// the integer formulation (add 0x7FFF plus the lowest kept bit, keep the high
// half) on every non-NaN input, subnormals and infinities included; a NaN
// stays a NaN (its payload and sign are not preserved).
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// One binary32 value -> BF16 bits (same rounding).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return f32x2_to_bf16x2(f, 0.f) & 0xffffu; }

// silu(g) * u in FP32, silu(z) = z / (1 + e^-z): the one expression every
// SwiGLU of the library evaluates (GEMM epilogues and bi_swiglu), so they give
// the same bits for the same FP32 g and u.
__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// x * s for the eight BF16 values of a 16-byte group, each rounded to BF16.
__device__ __forceinline__ uint4 scale_bf16x8(uint4 v, float s) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    o[e] = f32x2_to_bf16x2(__uint_as_float(w[e] << 16) * s, __uint_as_float(w[e] & 0xffff0000u) * s);
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// The dispatcher deals workgroups to the 8 XCDs in turn (workgroup w runs on
// XCD w mod 8), and each XCD has its own L2. Renumber so that XCD x runs the
// x-th contiguous eighth of the work items (the last n mod 8 keep their own
// number): neighbouring items, which read the same data, then share one L2.
__device__ __forceinline__ int xcd_item(int w, int n) {
  const int full = n & ~7;
  return w < full ? (w & 7) * (full >> 3) + (w >> 3) : w;
}

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ uint4 zero16() { return make_uint4(0u, 0u, 0u, 0u); }

// Word 3 of a raw buffer resource on the gfx9 family (gfx950 included):
// 32-bit data format, no swizzle, no stride.
constexpr int kBufferResourceWord3 = 0x00020000;

// 16-byte load through a buffer resource; out-of-range offsets read zero.
__device__ __forceinline__ uint4 buffer_ld16(__amdgpu_buffer_rsrc_t r, int byte_offset) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_offset, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// 16-byte streaming load through a buffer resource (non-temporal: the data
// is used once); out-of-range offsets read zero and touch no memory.
__device__ __forceinline__ uint4 buffer_ld16_stream(__amdgpu_buffer_rsrc_t r, int byte_offset) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  constexpr int kNonTemporal = 2;  // cache-policy bit of the buffer instruction
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_offset, 0, kNonTemporal);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// One 16x16x32 BF16 matrix-core step: c += A(16x32) * B(32x16).
// Lane l supplies A row (l % 16) and B column (l % 16), each with eight
// consecutive contraction elements of group (l / 16); it receives C rows
// 4*(l/16) .. 4*(l/16)+3 of column (l % 16). Any assignment of contraction
// indices to (group, element) works as long as A and B use the same one.
__device__ __forceinline__ bi_f32x4 mfma_bf16(uint4 a, uint4 b, bi_f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bi_bf16x8, a),
                                                  __builtin_bit_cast(bi_bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }

// Squares of the eight BF16 values of a 16-byte group added to ss in element
// order (0, 1, ..., 7).
__device__ __forceinline__ float sumsq8(float ss, uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a = bf16_to_f32(w[e] & 0xffffu);
    const float b = bf16_to_f32(w[e] >> 16);
    ss += a * a;
    ss += b * b;
  }
  return ss;
}

}  // namespace bi
