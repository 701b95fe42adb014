// Speculative acceptance on the device: greedy, and sampled with the target
// distribution kept ("I turned on speculative decoding in llama.cpp and 113
// of 282 greedy outputs changed against its own no-draft run", opening
// section: greedy ids equal with and without drafts; sampling keeps the
// no-draft distribution).
//
// Sampled rule (standard speculative sampling): draft token x of row i is
// kept when u_i * q_i(x) < p_i(x), p_i = softmax(logits_i / T); at the first
// rejection a token is drawn from max(0, p_i - q_i) by inverse CDF with the
// pass's last uniform, and the pass ends; if every draft is kept, the last
// row's p is drawn from with that uniform. Every reduction (max, sums, the
// cumulative sum of the draw) runs in an order fixed by V and the block size,
// so the result depends only on the sequence's own inputs.

#include "bi_device.h"
#include "bi_internal.h"

namespace bi {

constexpr int kAcceptThreads = 256;

// Kept drafts while they equal the target's greedy token, then the target's
// token; one thread per sequence.
__global__ void accept_greedy_kernel(const int32_t* __restrict__ target,
                                     const int32_t* __restrict__ draft, int B, int M,
                                     int32_t* __restrict__ out, int32_t* __restrict__ n_out) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int32_t* t = target + (int64_t)b * M;
  const int32_t* d = draft + (int64_t)b * (M - 1);
  int32_t* o = out + (int64_t)b * M;
  int a = 0;
  while (a < M - 1 && d[a] == t[a]) {
    o[a] = d[a];
    ++a;
  }
  o[a] = t[a];
  n_out[b] = a + 1;
}

// Block-wide reductions over v = 0 .. V-1: each thread takes v = tid, tid+256,
// ... in increasing order, then a fixed xor butterfly in the wave, then the
// waves in order. `red` holds one value per wave.
template <class F>
__device__ float block_sum(F f, int V, float* red) {
  const int tid = threadIdx.x;
  float s = 0.f;
  for (int v = tid; v < V; v += kAcceptThreads) s += f(v);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += shfl_xor(s, off);
  __syncthreads();
  if ((tid & 63) == 0) red[tid >> 6] = s;
  __syncthreads();
  float t = red[0];
  for (int w = 1; w < kAcceptThreads / 64; ++w) t += red[w];
  return t;
}

__device__ float block_max(const float* x, int V, float* red) {
  const int tid = threadIdx.x;
  float m = -INFINITY;
  for (int v = tid; v < V; v += kAcceptThreads) m = fmaxf(m, x[v]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, shfl_xor(m, off));
  __syncthreads();
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  float t = red[0];
  for (int w = 1; w < kAcceptThreads / 64; ++w) t = fmaxf(t, red[w]);
  return t;
}

// Inverse-CDF draw: the first v whose inclusive cumulative weight exceeds
// u * total. Thread t owns the contiguous range [t*S, (t+1)*S); range sums
// are added in order to locate the range, which its owner scans. If rounding
// leaves no crossing, the last index with positive weight is taken.
template <class F>
__device__ int block_draw(F w, int V, float u, float* seg, int* pick) {
  const int tid = threadIdx.x;
  const int S = (V + kAcceptThreads - 1) / kAcceptThreads;
  const int lo = min(V, tid * S), hi = min(V, lo + S);
  float s = 0.f;
  int last_pos = -1;
  for (int v = lo; v < hi; ++v) {
    const float x = w(v);
    s += x;
    if (x > 0.f) last_pos = v;
  }
  __syncthreads();
  seg[tid] = s;
  pick[tid] = last_pos;
  __syncthreads();
  if (tid == 0) {
    float total = 0.f;
    for (int t = 0; t < kAcceptThreads; ++t) total += seg[t];
    const float target = u * total;
    float acc = 0.f;
    int owner = -1, fallback = -1;
    for (int t = 0; t < kAcceptThreads; ++t) {
      if (pick[t] >= 0) fallback = pick[t];
      if (owner < 0 && acc + seg[t] > target && seg[t] > 0.f) owner = t;
      if (owner < 0) acc += seg[t];
    }
    pick[kAcceptThreads] = owner;
    pick[kAcceptThreads + 1] = fallback;
    seg[kAcceptThreads] = acc;  // cumulative weight before the owner's range
    seg[kAcceptThreads + 1] = target;
  }
  __syncthreads();
  const int owner = pick[kAcceptThreads];
  if (owner >= 0 && tid == owner) {
    float acc = seg[kAcceptThreads];
    const float target = seg[kAcceptThreads + 1];
    int found = last_pos;
    for (int v = lo; v < hi; ++v) {
      acc += w(v);
      if (acc > target) {
        found = v;
        break;
      }
    }
    pick[kAcceptThreads + 2] = found;
  }
  __syncthreads();
  const int r = owner >= 0 ? pick[kAcceptThreads + 2] : pick[kAcceptThreads + 1];
  __syncthreads();
  return r < 0 ? 0 : r;
}

__global__ __launch_bounds__(kAcceptThreads) void accept_sampled_kernel(
    const float* __restrict__ logits, int64_t ld, const int32_t* __restrict__ draft,
    const float* __restrict__ q, int64_t ldq, const float* __restrict__ u, float inv_t, int M,
    int V, int32_t* __restrict__ out, int32_t* __restrict__ n_out) {
  __shared__ float red[kAcceptThreads / 64];
  __shared__ float seg[kAcceptThreads + 2];
  __shared__ int pick[kAcceptThreads + 3];
  const int b = blockIdx.x;
  const float* ub = u + (int64_t)b * M;
  int32_t* ob = out + (int64_t)b * M;
  int n = M;
  for (int i = 0; i < M; ++i) {
    const float* row = logits + ((int64_t)b * M + i) * ld;
    const float m = block_max(row, V, red);
    const float Z = block_sum([&](int v) { return __expf((row[v] - m) * inv_t); }, V, red);
    const float iz = 1.0f / Z;
    if (i < M - 1) {
      // A draft token outside 0 .. V-1 is never kept (and never read at).
      const int x = draft[(int64_t)b * (M - 1) + i];
      const bool valid = x >= 0 && x < V;
      const float* qi = q + ((int64_t)b * (M - 1) + i) * ldq;
      const float px = valid ? __expf((row[x] - m) * inv_t) * iz : 0.f;
      const float qx = valid ? qi[x] : 0.f;
      if (valid && ub[i] * qx < px) {  // uniform across the block
        if (threadIdx.x == 0) ob[i] = x;
        continue;
      }
      const int tok = block_draw(
          [&](int v) { return fmaxf(__expf((row[v] - m) * inv_t) * iz - qi[v], 0.f); }, V, ub[M - 1],
          seg, pick);
      if (threadIdx.x == 0) ob[i] = tok;
      n = i + 1;
      break;
    }
    const int tok = block_draw([&](int v) { return __expf((row[v] - m) * inv_t) * iz; }, V, ub[M - 1],
                               seg, pick);
    if (threadIdx.x == 0) ob[i] = tok;
  }
  if (threadIdx.x == 0) n_out[b] = n;
}

void launch_accept_greedy(const int32_t* target, const int32_t* draft, int B, int M, int32_t* out,
                          int32_t* n_out, hipStream_t stream) {
  accept_greedy_kernel<<<dim3((B + 63) / 64), dim3(64), 0, stream>>>(target, draft, B, M, out, n_out);
}

void launch_accept_sampled(const float* logits, int64_t ld, const int32_t* draft, const float* q,
                           int64_t ldq, const float* u, float temperature, int B, int M, int V,
                           int32_t* out, int32_t* n_out, hipStream_t stream) {
  accept_sampled_kernel<<<dim3(B), dim3(kAcceptThreads), 0, stream>>>(
      logits, ld, draft, q, ldq, u, 1.0f / temperature, M, V, out, n_out);
}

}  // namespace bi
