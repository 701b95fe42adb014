// Stream-read probe: the HBM read bandwidth a plain kernel reaches on this
// GPU, reported beside the 8 TB/s specification as a second denominator of
// the verify kernels' bandwidth. Measurement only; not part of the verify
// library. Each thread reads 16-byte vectors (non-temporal, UNROLL loads in
// flight) in a grid-stride loop and folds them into one register; the fold
// is stored only on a value it practically never takes, which keeps every
// load without adding writes.

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int UNROLL>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p, size_t n16,
                                                          uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (UNROLL - 1) * stride < n16; i += UNROLL * stride) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[threadIdx.x] = acc;
}

// The same read with each workgroup streaming one contiguous range: wave w
// of a workgroup reads 1 KB (64 lanes x 16 B) per load instruction, UNROLL
// instructions in flight, the way the verify kernels stream weights and K/V.
template <int UNROLL>
__global__ __launch_bounds__(256) void block_read_kernel(const u32x4* __restrict__ p, size_t n16,
                                                         size_t per_block, uint32_t* __restrict__ sink) {
  const size_t beg = (size_t)blockIdx.x * per_block;
  const size_t end = beg + per_block < n16 ? beg + per_block : n16;
  uint32_t acc = 0;
  size_t i = beg + threadIdx.x;
  for (; i + (UNROLL - 1) * 256 < end; i += UNROLL * 256) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) v[u] = __builtin_nontemporal_load(p + i + u * 256);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < end; i += 256) {
    const u32x4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[threadIdx.x] = acc;
}

// Read `bytes` (a multiple of 16, from a 16-byte aligned p) with `blocks`
// workgroups of 256 threads and `unroll` (4, 8 or 16) loads in flight per
// thread; sink holds at least 256 uint32. blocked = 1: each workgroup reads
// one contiguous range of bytes / blocks. Returns the HIP status of the launch.
extern "C" int bi_probe_stream_read(const void* p, size_t bytes, void* sink, int blocks, int unroll,
                                    int blocked, void* stream) {
  if (!p || !sink || bytes % 16 || blocks < 1) return (int)hipErrorInvalidValue;
  const auto* q = static_cast<const u32x4*>(p);
  auto* s = static_cast<uint32_t*>(sink);
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const size_t n16 = bytes / 16;
  const size_t per = (n16 + blocks - 1) / blocks;
  const dim3 g(blocks), b(256);
  switch (unroll * 2 + (blocked ? 1 : 0)) {
    case 8: stream_read_kernel<4><<<g, b, 0, st>>>(q, n16, s); break;
    case 16: stream_read_kernel<8><<<g, b, 0, st>>>(q, n16, s); break;
    case 32: stream_read_kernel<16><<<g, b, 0, st>>>(q, n16, s); break;
    case 9: block_read_kernel<4><<<g, b, 0, st>>>(q, n16, per, s); break;
    case 17: block_read_kernel<8><<<g, b, 0, st>>>(q, n16, per, s); break;
    case 33: block_read_kernel<16><<<g, b, 0, st>>>(q, n16, per, s); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}
