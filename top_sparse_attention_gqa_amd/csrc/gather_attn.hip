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

// Exclusive prefix over the block of per-head popcounts packed four heads
// per 64-bit word (16-bit fields: a tile holds at most 8192 positions).
template <int G>
struct PackedCounts {
  static constexpr int kWords = (G + 3) / 4;
  int64_t v[kWords];
};

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
  __shared__ int32_t s_pg[kWordsPerTile];
  __shared__ int32_t upos[kTile];
  __shared__ uint8_t umem[kTile];
  __shared__ uint32_t s_off[G];
  __shared__ float s_zs[kGathWaves][G];
  __shared__ float s_acc[kGathWaves][G][kHeadDim];
  __shared__ int64_t s_tmp[16];

  for (int i = tid; i < G * kWordsPerTile; i += kGathThreads) {
    const int hh = i / kWordsPerTile;
    const int w = i - hh * kWordsPerTile;
    bm[hh][w] = p.bitmap[(bh0 + hh) * words_row + size_t(tile) * kWordsPerTile + w];
  }
  // a 64-bit word covers exactly one 64-token page
  if (tid < kWordsPerTile)
    s_pg[tid] = (t0 + tid * 64 < sg.N) ? page_of(p, b, (t0 >> 6) + tid) : 0;
  for (int hh = wave; hh < G; hh += kGathWaves) {
    uint32_t s = 0;
    for (int t = lane; t < tile; t += 64) s += p.tile_cnt[(bh0 + hh) * p.n_tiles + t];
    s = wave_sum(s);
    if (lane == 0) s_off[hh] = s;
  }
  float mref[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) mref[hh] = softmax_ref(p.state[bh0 + hh], sg.k_eff);
  __syncthreads();

  // union of the group's selections and W, as an ordered position list, and
  // each head's rank offsets for its out_idx slice
  uint64_t uw = 0, wm = 0;
  const int nw = t0 + tid * 64;
  PackedCounts<G> pc;
#pragma unroll
  for (int j = 0; j < PackedCounts<G>::kWords; ++j) pc.v[j] = 0;
  if (tid < kWordsPerTile) {
    wm = range_mask(nw, 0, sg.lo) | range_mask(nw, wstart, sg.N);
    uw = wm;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      uw |= bm[hh][tid];
      pc.v[hh >> 2] |= int64_t(__popcll(bm[hh][tid])) << (16 * (hh & 3));
    }
  }
  int64_t utotal, unused;
  const int64_t ex = block_excl_scan(__popcll(uw), s_tmp, &utotal);
  PackedCounts<G> px;
#pragma unroll
  for (int j = 0; j < PackedCounts<G>::kWords; ++j) px.v[j] = block_excl_scan(pc.v[j], s_tmp, &unused);
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
    if (p.k_max > 0) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        uint32_t rank = s_off[hh] + uint32_t((px.v[hh >> 2] >> (16 * (hh & 3))) & 0xFFFF);
        int32_t* dst = p.out_idx + (bh0 + hh) * p.k_max;
        uint64_t y = bm[hh][tid];
        while (y) {
          const int bit = __ffsll((unsigned long long)y) - 1;
          y &= y - 1ull;
          if (rank < uint32_t(p.k_max)) dst[rank] = nw + bit;
          ++rank;
        }
      }
    }
  }
  __syncthreads();
  const int U = int(utotal);

  // accumulate e^{z - m} v: 4 rows per wave step, 16 lanes x 8 dims per V
  // row, kUnroll rows per lane in flight
  constexpr int kUnroll = 4;
  float acc[G][8];
  float zs[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    zs[hh] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[hh][e] = 0.0f;
  }
  const size_t vpage = size_t(p.H_kv) * kPage * kHeadDim;
  const uint16_t* vbase = p.v_pool + size_t(g) * kPage * kHeadDim + r * 8;
  for (int i0 = wave * 4 + row; i0 < U; i0 += kGathWaves * 4 * kUnroll) {
    uint4 v[kUnroll];
    float z[kUnroll][G];
    uint32_t mem[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int i = i0 + u * kGathWaves * 4;
      const bool ok = i < U;
      const int n = ok ? upos[i] : t0;
      mem[u] = ok ? umem[i] : 0u;
      const int pg = s_pg[(n - t0) >> 6];
      v[u] = *reinterpret_cast<const uint4*>(vbase + size_t(pg) * vpage + size_t(n & 63) * kHeadDim);
#pragma unroll
      for (int hh = 0; hh < G; ++hh)
        z[u][hh] = ((mem[u] >> hh) & 1u) ? p.scores[(bh0 + hh) * p.n_cap + n] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float vf[8] = {bf16lo(v[u].x), bf16hi(v[u].x), bf16lo(v[u].y), bf16hi(v[u].y),
                           bf16lo(v[u].z), bf16hi(v[u].z), bf16lo(v[u].w), bf16hi(v[u].w)};
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float w = ((mem[u] >> hh) & 1u) ? expf(z[u][hh] - mref[hh]) : 0.0f;
        zs[hh] += w;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hh][e] += w * vf[e];
      }
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
  if (lane == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) s_zs[wave][hh] = zs[hh];
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
    for (int w = 0; w < kGathWaves; ++w) z += s_zs[w][tid];
    float* mz = p.part_mz + ((bh0 + tid) * p.n_tiles + tile) * 2;
    mz[0] = mref[tid];
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
  const float* pn = p.part_n + size_t(bh) * p.n_tiles * kHeadDim + d;
  float m = -INFINITY;
#pragma unroll 8
  for (int t = 0; t < nt; ++t) m = fmaxf(m, mz[2 * t + 1] > 0.0f ? mz[2 * t] : -INFINITY);
  float Z = 0.0f, acc = 0.0f;
  if (m > -INFINITY) {
#pragma unroll 8
    for (int t = 0; t < nt; ++t) {
      const float zt = mz[2 * t + 1];
      const float sc = zt > 0.0f ? expf(mz[2 * t] - m) : 0.0f;
      Z += sc * zt;
      acc += sc * pn[size_t(t) * kHeadDim];
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
