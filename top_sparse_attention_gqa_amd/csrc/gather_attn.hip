// Softmax . V over W u Omega_h as split-K partials, then their log-sum-exp
// merge (RetrievalAttention slides, "Sparse attention renormalizes selected
// tokens", Eq. (2); "Two local softmax outputs need global weights",
// Eqs. (3)-(5); backup frame "the normalization identity": merging disjoint
// partials gives the exact softmax over their union).
//
// gather: one block per (sequence, KV head, tile of 8192 positions). The
//   block takes the union over the group's G query heads of their selected
//   positions in the tile plus the tile's static positions, in ascending
//   order, reads each V row (256 contiguous bytes) once, and accumulates for
//   every head that attends to it: m = max z, Z = sum e^{z - m},
//   N = sum e^{z - m} v. It also writes the tile's part of out_idx, whose
//   offset is the sum of the per-tile selection counts before it.
// merge: one block per (sequence, query head): m = max_t m_t,
//   out = sum_t e^{m_t - m} N_t / sum_t e^{m_t - m} Z_t, lse = m + ln(...),
//   and -1 padding of out_idx after k_eff.
#include "ra_internal.h"

namespace ra {

constexpr int kGathThreads = 256;
constexpr int kGathWaves = kGathThreads / 64;

__device__ __forceinline__ uint64_t range_mask(int nw, int a, int c) {
  const int s = max(a - nw, 0);
  const int e = min(c - nw, 64);
  if (e <= s) return 0ull;
  const uint64_t hi = e == 64 ? ~0ull : ((1ull << e) - 1ull);
  const uint64_t lo = (1ull << s) - 1ull;
  return hi & ~lo;
}

__device__ __forceinline__ float bf16lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }

template <int G>
__global__ __launch_bounds__(kGathThreads) void gather_kernel(Params p) {
  const int tile = blockIdx.x;
  const int bg = blockIdx.y;
  const int b = bg / p.H_kv;
  const int g = bg - b * p.H_kv;
  const SeqGeom sg = seq_geom(p, b);
  const int t0 = tile * kTile;
  if (t0 >= sg.N) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int row = lane >> 4;
  const int r = lane & 15;
  const size_t bh0 = size_t(b) * p.H_q + size_t(g) * G;
  const size_t words_row = size_t(p.n_cap / 64);
  const int wstart = max(sg.N - p.window, 0);  // W = [0, lo) u [wstart, N)

  __shared__ uint64_t bm[G][kWordsPerTile];
  __shared__ uint32_t wpre[kWordsPerTile];
  __shared__ int32_t upos[kTile];
  __shared__ uint8_t umem[kTile];
  __shared__ uint32_t s_off[G];
  __shared__ float s_m[G];
  __shared__ float s_part[kGathWaves][G];
  __shared__ float s_acc[kGathWaves][G][kHeadDim];
  __shared__ int64_t s_tmp[16];

  for (int i = tid; i < G * kWordsPerTile; i += kGathThreads) {
    const int hh = i / kWordsPerTile;
    const int w = i - hh * kWordsPerTile;
    bm[hh][w] = p.bitmap[(bh0 + hh) * words_row + size_t(tile) * kWordsPerTile + w];
  }
  for (int hh = wave; hh < G; hh += kGathWaves) {
    uint32_t s = 0;
    for (int t = lane; t < tile; t += 64) s += p.tile_cnt[(bh0 + hh) * p.n_tiles + t];
    s = wave_sum(s);
    if (lane == 0) s_off[hh] = s;
  }
  __syncthreads();

  // union of the group's selections and W, as an ordered position list
  uint64_t uw = 0, wm = 0;
  const int nw = t0 + tid * 64;
  if (tid < kWordsPerTile) {
    wm = range_mask(nw, 0, sg.lo) | range_mask(nw, wstart, sg.N);
    uw = wm;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) uw |= bm[hh][tid];
  }
  int64_t utotal;
  const int64_t ex = block_excl_scan(tid < kWordsPerTile ? __popcll(uw) : 0, s_tmp, &utotal);
  if (tid < kWordsPerTile) {
    int pos = int(ex);
    uint64_t x = uw;
    while (x) {
      const int bit = __ffsll((unsigned long long)x) - 1;
      x &= x - 1ull;
      uint32_t mem = 0;
      if ((wm >> bit) & 1ull) {
        mem = (1u << G) - 1u;
      } else {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) mem |= uint32_t((bm[hh][tid] >> bit) & 1ull) << hh;
      }
      upos[pos] = nw + bit;
      umem[pos] = uint8_t(mem);
      ++pos;
    }
  }

  // this tile's slice of out_idx, per head, ascending
  if (p.k_max > 0) {
#pragma unroll 1
    for (int hh = 0; hh < G; ++hh) {
      const uint64_t x0 = tid < kWordsPerTile ? bm[hh][tid] : 0ull;
      int64_t tot;
      const int64_t hx = block_excl_scan(__popcll(x0), s_tmp, &tot);
      uint32_t rank = s_off[hh] + uint32_t(hx);
      int32_t* dst = p.out_idx + (bh0 + hh) * p.k_max;
      uint64_t x = x0;
      while (x) {
        const int bit = __ffsll((unsigned long long)x) - 1;
        x &= x - 1ull;
        if (rank < uint32_t(p.k_max)) dst[rank] = nw + bit;
        ++rank;
      }
    }
  }
  __syncthreads();
  const int U = int(utotal);

  // per-head maximum over the attended positions of this tile
  float lm[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) lm[hh] = -INFINITY;
  for (int i = tid; i < U; i += kGathThreads) {
    const int n = upos[i];
    const uint32_t mem = umem[i];
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
      if ((mem >> hh) & 1u) lm[hh] = fmaxf(lm[hh], p.scores[(bh0 + hh) * p.n_cap + n]);
  }
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const float v = wave_max(lm[hh]);
    if (lane == 0) s_part[wave][hh] = v;
  }
  __syncthreads();
  if (tid < G) {
    float v = s_part[0][tid];
    for (int w = 1; w < kGathWaves; ++w) v = fmaxf(v, s_part[w][tid]);
    s_m[tid] = v;
  }
  __syncthreads();
  float mh[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) mh[hh] = s_m[hh];

  // accumulate: 4 positions per wave step, 16 lanes x 8 dims per V row
  float acc[G][8];
  float zs[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    zs[hh] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[hh][e] = 0.0f;
  }
  const size_t vstride_page = size_t(p.H_kv) * kPage * kHeadDim;
  for (int i = wave * 4 + row; i < U; i += kGathWaves * 4) {
    const int n = upos[i];
    const uint32_t mem = umem[i];
    const int pg = page_of(p, b, n >> 6);
    const uint4 v = *reinterpret_cast<const uint4*>(
        p.v_pool + size_t(pg) * vstride_page + (size_t(g) * kPage + (n & 63)) * kHeadDim + r * 8);
    const float vf[8] = {bf16lo(v.x), bf16hi(v.x), bf16lo(v.y), bf16hi(v.y),
                         bf16lo(v.z), bf16hi(v.z), bf16lo(v.w), bf16hi(v.w)};
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const bool on = (mem >> hh) & 1u;
      const float z = on ? p.scores[(bh0 + hh) * p.n_cap + n] : 0.0f;
      const float w = on ? expf(z - mh[hh]) : 0.0f;
      zs[hh] += w;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] += w * vf[e];
    }
  }
  // sum the 4 rows of each wave, then the waves
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    zs[hh] += __shfl_xor(zs[hh], 16);
    zs[hh] += __shfl_xor(zs[hh], 32);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[hh][e] += __shfl_xor(acc[hh][e], 16);
      acc[hh][e] += __shfl_xor(acc[hh][e], 32);
    }
  }
  if (row == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) s_acc[wave][hh][r * 8 + e] = acc[hh][e];
  }
  __syncthreads();  // s_part is reused below
  if (lane == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) s_part[wave][hh] = zs[hh];
  }
  __syncthreads();
  for (int i = tid; i < G * kHeadDim; i += kGathThreads) {
    const int hh = i / kHeadDim;
    const int d = i - hh * kHeadDim;
    float s = 0.0f;
    for (int w = 0; w < kGathWaves; ++w) s += s_acc[w][hh][d];
    p.part_n[((bh0 + hh) * p.n_tiles + tile) * kHeadDim + d] = s;
  }
  if (tid < G) {
    float z = 0.0f;
    for (int w = 0; w < kGathWaves; ++w) z += s_part[w][tid];
    float* mz = p.part_mz + ((bh0 + tid) * p.n_tiles + tile) * 2;
    mz[0] = s_m[tid];
    mz[1] = z;
  }
}

hipError_t launch_gather(const Params& p, hipStream_t s) {
  const unsigned tiles = unsigned((int64_t(p.max_seq_len) + kTile - 1) / kTile);
  const dim3 grid{tiles, unsigned(p.B * p.H_kv)}, block{unsigned(kGathThreads)};
  switch (p.G) {
    case 1: hipLaunchKernelGGL(gather_kernel<1>, grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL(gather_kernel<2>, grid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL(gather_kernel<4>, grid, block, 0, s, p); break;
    case 8: hipLaunchKernelGGL(gather_kernel<8>, grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- merge
__global__ __launch_bounds__(kHeadDim) void merge_kernel(Params p) {
  const int bh = blockIdx.x;
  const int b = bh / p.H_q;
  const SeqGeom sg = seq_geom(p, b);
  const int nt = (sg.N + kTile - 1) / kTile;
  const int d = threadIdx.x;
  const float* mz = p.part_mz + size_t(bh) * p.n_tiles * 2;
  float m = -INFINITY;
  for (int t = 0; t < nt; ++t)
    if (mz[2 * t + 1] > 0.0f) m = fmaxf(m, mz[2 * t]);
  float Z = 0.0f, acc = 0.0f;
  for (int t = 0; t < nt; ++t) {
    const float zt = mz[2 * t + 1];
    if (zt > 0.0f) {
      const float sc = expf(mz[2 * t] - m);
      Z += sc * zt;
      acc += sc * p.part_n[(size_t(bh) * p.n_tiles + t) * kHeadDim + d];
    }
  }
  p.out[size_t(bh) * kHeadDim + d] = Z > 0.0f ? acc / Z : 0.0f;
  if (d == 0 && p.lse) p.lse[bh] = Z > 0.0f ? m + logf(Z) : -INFINITY;
  if (p.k_max > 0) {
    int32_t* dst = p.out_idx + size_t(bh) * p.k_max;
    for (int i = sg.k_eff + d; i < p.k_max; i += kHeadDim) dst[i] = -1;
  }
}

hipError_t launch_merge(const Params& p, hipStream_t s) {
  hipLaunchKernelGGL(merge_kernel, dim3(unsigned(p.B * p.H_q)), dim3(kHeadDim), 0, s, p);
  return hipGetLastError();
}

}  // namespace ra
