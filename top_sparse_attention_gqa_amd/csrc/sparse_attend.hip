// Attention over a given set of positions, and the merge of two partial
// outputs: the pieces of a decode step whose KV lives in two tiers
// (RetrievalAttention slides, frames "The GPU keeps 640 fixed positions":
// the static set W is attended from GPU memory, the retrieved set Omega
// from CPU memory, and "Two local softmax outputs need global weights":
// the two partials are merged by Eqs. (3)-(5)).
//
// sparse_attend: for each query head, softmax over the listed positions of
// z = q . k / sqrt(128) (Eq. (1)), times V (Eq. (2)), with the maximum
// subtracted; out and lse = m + ln Z. The pools may be GPU memory or
// pinned host memory mapped for the device (zero-copy reads over the
// host link). merge_partials: o = sum_S e^{lse_S - m} o_S / sum_S
// e^{lse_S - m}, lse = m + ln sum_S e^{lse_S - m}, m = max_S lse_S; an empty
// partial has lse = -inf and weight 0.
#include "ra_internal.h"

namespace ra {

// One block of 16 waves per query head. The kernel is bound by the latency
// of its dependent reads (index, page entry, K row; then V rows), most of
// all when the pools are in host memory: every wave keeps many rows in
// flight, and the scores take one position per thread.
constexpr int kSaThreads = 1024;
constexpr int kSaWaves = kSaThreads / 64;
constexpr int kSaRows = 8;  // V rows per wave in flight
constexpr float kScale = 0.08838834764831845f;  // 1 / sqrt(128)

__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__global__ __launch_bounds__(kSaThreads) void sparse_attend_kernel(SaParams p) {
  __shared__ float z[RA_SPARSE_MAX_K];
  __shared__ float red[kSaWaves];
  __shared__ float part[kSaWaves][kHeadDim];
  const int h = blockIdx.x;
  const int g = h / (p.H_q / p.H_kv);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t* idx = p.idx + size_t(h) * p.k;
  auto row = [&](const uint16_t* pool, int32_t n) {
    int32_t pg = p.block_table[n >> 6];
    pg = ((unsigned)pg < (unsigned)p.num_pages) ? pg : 0;
    return pool + ((size_t(pg) * p.H_kv + g) * kPage + (n & 63)) * kHeadDim;
  };

  // scores: q as bf16 pairs, dimensions 2 i then 2 i + 1
  uint32_t qw[kHeadDim / 2];
  {
    const uint4* qr = reinterpret_cast<const uint4*>(p.q + size_t(h) * kHeadDim);
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const uint4 x = qr[c];
      qw[4 * c] = x.x;
      qw[4 * c + 1] = x.y;
      qw[4 * c + 2] = x.z;
      qw[4 * c + 3] = x.w;
    }
  }
  float mx = -INFINITY;
  for (int i = tid; i < p.k; i += kSaThreads) {
    const int32_t n = idx[i];
    float s = -INFINITY;
    if (n >= 0 && n < p.N) {
      const uint4* kr = reinterpret_cast<const uint4*>(row(p.k_pool, n));
      float acc = 0.0f;
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const uint4 x = kr[c];
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t qq = qw[4 * c + j];
          acc = fmaf(__uint_as_float(qq << 16), __uint_as_float(w[j] << 16), acc);
          acc = fmaf(__uint_as_float(qq & 0xFFFF0000u), __uint_as_float(w[j] & 0xFFFF0000u), acc);
        }
      }
      s = acc * kScale;
    }
    z[i] = s;
    mx = fmaxf(mx, s);
  }
  mx = wave_max(mx);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int w = 1; w < kSaWaves; ++w) m = fmaxf(m, red[w]);
  __syncthreads();
  if (m == -INFINITY) {  // nothing listed: an empty partial (block-uniform)
    if (tid < kHeadDim) p.out[size_t(h) * kHeadDim + tid] = 0.0f;
    if (tid == 0) p.out_lse[h] = -INFINITY;
    return;
  }
  // weights and their sum
  float zs = 0.0f;
  for (int i = tid; i < p.k; i += kSaThreads) {
    const float w = z[i] == -INFINITY ? 0.0f : expf(z[i] - m);
    z[i] = w;
    zs += w;
  }
  zs = wave_sum_f(zs);
  if (lane == 0) red[wave] = zs;
  __syncthreads();
  float Z = 0.0f;
#pragma unroll
  for (int w = 0; w < kSaWaves; ++w) Z += red[w];
  // weighted V rows: wave w takes the positions i = w mod 16, lane l the
  // dimensions 2 l, 2 l + 1 (a row is 256 coalesced bytes); kSaRows rows
  // are in flight at a time
  float a0 = 0.0f, a1 = 0.0f;
  for (int i0 = wave; i0 < p.k; i0 += kSaRows * kSaWaves) {
    uint32_t v[kSaRows];
    float w[kSaRows];
#pragma unroll
    for (int r = 0; r < kSaRows; ++r) {
      const int i = i0 + r * kSaWaves;
      w[r] = i < p.k ? z[i] : 0.0f;
      v[r] = w[r] != 0.0f ? reinterpret_cast<const uint32_t*>(row(p.v_pool, idx[i]))[lane] : 0u;
    }
#pragma unroll
    for (int r = 0; r < kSaRows; ++r) {
      a0 = fmaf(w[r], __uint_as_float(v[r] << 16), a0);
      a1 = fmaf(w[r], __uint_as_float(v[r] & 0xFFFF0000u), a1);
    }
  }
  part[wave][2 * lane] = a0;
  part[wave][2 * lane + 1] = a1;
  __syncthreads();
  if (tid < kHeadDim) {
    float t = 0.0f;
#pragma unroll
    for (int w = 0; w < kSaWaves; ++w) t += part[w][tid];
    p.out[size_t(h) * kHeadDim + tid] = t / Z;
    if (tid == 0) p.out_lse[h] = m + logf(Z);
  }
}

__global__ __launch_bounds__(kHeadDim) void merge_partials_kernel(const float* oa, const float* la,
                                                                 const float* ob, const float* lb,
                                                                 float* out, float* lse) {
  const int h = blockIdx.x, d = threadIdx.x;
  const float a = la[h], b = lb[h];
  const float m = fmaxf(a, b);
  if (m == -INFINITY) {
    out[size_t(h) * kHeadDim + d] = 0.0f;
    if (d == 0) lse[h] = -INFINITY;
    return;
  }
  const float wa = a == -INFINITY ? 0.0f : expf(a - m);
  const float wb = b == -INFINITY ? 0.0f : expf(b - m);
  const size_t o = size_t(h) * kHeadDim + d;
  out[o] = (wa * oa[o] + wb * ob[o]) / (wa + wb);
  if (d == 0) lse[h] = m + logf(wa + wb);
}

hipError_t launch_sparse_attend(const SaParams& p, hipStream_t s) {
  hipLaunchKernelGGL(sparse_attend_kernel, dim3(p.H_q), dim3(kSaThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_merge_partials(const float* oa, const float* la, const float* ob,
                                 const float* lb, int32_t H, float* out, float* lse,
                                 hipStream_t s) {
  hipLaunchKernelGGL(merge_partials_kernel, dim3(H), dim3(kHeadDim), 0, s, oa, la, ob, lb, out, lse);
  return hipGetLastError();
}

}  // namespace ra
