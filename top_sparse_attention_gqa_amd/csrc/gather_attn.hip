// Softmax . V over W u Omega_h as split-K partials, then their log-sum-exp
// merge (RetrievalAttention slides, "Sparse attention renormalizes selected
// tokens", Eq. (2); "Two local softmax outputs need global weights",
// Eqs. (3)-(5); backup frame "the normalization identity": merging disjoint
// partials gives the exact softmax over their union).
//
// One block per (sequence, KV head, tile of 8192 positions = two units). The
// block first takes each head's retrieved members of the tile: the entries
// of the tile's (head, unit) candidate lists at or above the head's exact
// threshold. It marks them in an LDS bitmap, stores their scores next to the
// scores of W that the scan left, and writes their positions, ascending, with
// their count, over the tile's consumed lists. It then walks
// the union over the group's G query heads of those positions and the
// tile's static positions in ascending order, reads each V row (256
// contiguous bytes) once, and accumulates for every head that attends to
// it: Z = sum e^{z - m}, N = sum e^{z - m} v, with m the head's largest
// score over W u Omega (the scan records it), so no partial can overflow.
//
// merge: per query head, one block combines the tile partials,
// out = sum_t e^{m_t - m} N_t / sum_t e^{m_t - m} Z_t, lse = m + ln(...),
// and pads out_idx with -1 after k_eff; further blocks each copy the
// retrieved positions of kMergeTiles tiles into out_idx at the offset the
// counts of the tiles before them give.
#include "ra_internal.h"

namespace ra {

constexpr int kGathThreads = 256;
constexpr int kGathWaves = kGathThreads / 64;
constexpr int kChunk = 1024;   // union positions listed in LDS at a time
constexpr int kWBatch = 8;     // (row, head) weights per lane in flight
constexpr int kListBatch = 8;  // list entries per lane in flight

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

// Per-head popcounts packed four heads per 64-bit word (16-bit fields: a
// tile holds at most 8192 positions), so one block scan ranks them all.
template <int G>
struct PackedCounts {
  static constexpr int kWords = (G + 3) / 4;
  int64_t v[kWords];
};

template <int G>
__global__ __launch_bounds__(kGathThreads) __attribute__((amdgpu_waves_per_eu(4))) void gather_kernel(Params p) {
  const int tile = blockIdx.x;
  const int bg = blockIdx.y;
  const int b = bg / p.H_kv;
  const int g = bg - b * p.H_kv;
  const SeqGeom sg = seq_geom(p, b);
  const size_t bh0 = size_t(b) * p.H_q + size_t(g) * G;
  const int t0 = tile * kTile;
  if (t0 >= sg.N) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int row = lane >> 4;
  const int r = lane & 15;
  const int wstart = max(sg.N - p.window, 0);  // W = [0, lo) u [wstart, N)
  constexpr int kVRows = G <= 4 ? 8 : 4;       // V rows per lane in flight
  constexpr int kCh = G <= 4 ? kChunk : kChunk / 2;  // union rows per chunk

  __shared__ uint64_t bm[G][kWordsPerTile];
  __shared__ int32_t s_pg[kWordsPerTile];
  __shared__ uint32_t ulist[kCh];           // offset in tile | heads << 13
  __shared__ float s_w[kCh][G];             // softmax weight of (row, head), 0 if absent
  __shared__ float s_zs[kGathWaves][G];
  __shared__ float s_acc[kGathWaves][G][kHeadDim];
  __shared__ int64_t s_tmp[16];
  __shared__ HeadState s_st[G];
  __shared__ uint32_t s_lc[2 * G];          // list j: head j / 2, unit 2 tile + j % 2
  __shared__ uint32_t s_lpre[2 * G + 1];

  // every small load of the block at once: page numbers, list lengths,
  // head states and the tile's out_idx offsets
  for (int i = tid; i < G * kWordsPerTile; i += kGathThreads) (&bm[0][0])[i] = 0ull;
  const int units_seq = (sg.N + kUnit - 1) / kUnit;
  if (tid < kWordsPerTile) {
    // a 64-bit word covers exactly one 64-token page
    s_pg[tid] = (t0 + tid * 64 < sg.N) ? page_of(p, b, (t0 >> 6) + tid) : 0;
  } else if (tid < kWordsPerTile + 2 * G) {
    const int j = tid - kWordsPerTile;
    const int unit = 2 * tile + (j & 1);
    s_lc[j] = unit < units_seq ? p.ucnt[(bh0 + (j >> 1)) * p.n_units + unit] : 0u;
  } else if (tid >= kWordsPerTile + 64 && tid < kWordsPerTile + 64 + G) {
    const int hh = tid - kWordsPerTile - 64;
    s_st[hh] = p.state[bh0 + hh];
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t run = 0;
    for (int j = 0; j < 2 * G; ++j) {
      s_lpre[j] = run;
      if (s_st[j >> 1].thr_shift < 64u) run += s_lc[j];
    }
    s_lpre[2 * G] = run;
  }
  float mref[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) mref[hh] = softmax_ref(s_st[hh], sg.k_eff);
  __syncthreads();

  // each head's retrieved members of this tile: the list entries whose
  // composite (key - lo) << 32 | ~n clears the head's threshold. The 2 G
  // lists are walked as one index space, kListBatch entries per lane in
  // flight.
  const uint32_t total = s_lpre[2 * G];
  for (uint32_t base = 0; base < total; base += kGathThreads * kListBatch) {
    uint64_t v[kListBatch];
    int jl[kListBatch];
#pragma unroll
    for (int u = 0; u < kListBatch; ++u) {
      const uint32_t i = base + u * kGathThreads + tid;
      v[u] = 0ull;
      jl[u] = -1;
      if (i < total) {
        int j = 0;
        while (j + 1 < 2 * G && s_lpre[j + 1] <= i) ++j;
        jl[u] = j;
        v[u] = p.cand[(bh0 + (j >> 1)) * p.n_cap + size_t(2 * tile + (j & 1)) * kUnit +
                      (i - s_lpre[j])];
      }
    }
#pragma unroll
    for (int u = 0; u < kListBatch; ++u) {
      if (jl[u] < 0) continue;
      const int hh = jl[u] >> 1;
      const uint32_t key = uint32_t(v[u] >> 32);
      const uint32_t n = uint32_t(v[u]);
      const uint64_t comp = (uint64_t(key - s_st[hh].lo_key) << 32) | uint32_t(~n);
      const uint64_t thr = (uint64_t(s_st[hh].thr_hi) << 32) | s_st[hh].thr_lo;
      if ((comp >> s_st[hh].thr_shift) >= thr) {
        atomicOr(reinterpret_cast<unsigned long long*>(&bm[hh][(int(n) - t0) >> 6]),
                 1ull << (n & 63u));
        p.scores[(bh0 + hh) * p.n_cap + n] = key2f(key);
      }
    }
  }
  __syncthreads();

  // union of the group's selections and W, and each head's ranks
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
  int64_t utotal;
  const int64_t ex = block_excl_scan(__popcll(uw), s_tmp, &utotal);
  PackedCounts<G> px, ptot;
#pragma unroll
  for (int j = 0; j < PackedCounts<G>::kWords; ++j)
    px.v[j] = block_excl_scan(pc.v[j], s_tmp, &ptot.v[j]);
  // the tile's retrieved positions, ascending, replace its consumed lists
  // (the merge concatenates the tiles into out_idx)
  if (tid < kWordsPerTile) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      uint64_t y = bm[hh][tid];
      uint32_t rank = uint32_t((px.v[hh >> 2] >> (16 * (hh & 3))) & 0xFFFF);
      int32_t* dst = reinterpret_cast<int32_t*>(p.cand + (bh0 + hh) * p.n_cap + size_t(t0));
      while (y) {
        const int bit = __ffsll((unsigned long long)y) - 1;
        y &= y - 1ull;
        dst[rank++] = nw + bit;
      }
    }
  }
  if (tid < G)
    p.scnt[(bh0 + tid) * p.n_tiles + tile] =
        uint32_t((ptot.v[tid >> 2] >> (16 * (tid & 3))) & 0xFFFF);
  const int U = int(utotal);

  // Two phases per chunk of the union: (A) the weights e^{z - m} of every
  // (row, head) pair into LDS, one head per lane (lane t serves head
  // t % G), all score loads in flight at once; (B) the V rows, kVRows per
  // lane in flight, accumulated with the weights from LDS.
  float acc[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[hh][e] = 0.0f;
  const int my_h = tid % G;
  float zsum = 0.0f;  // this lane's share of Z for head my_h
  float mref_h = mref[0];
#pragma unroll
  for (int hh = 1; hh < G; ++hh)
    if (my_h == hh) mref_h = mref[hh];
  const float* zrow = p.scores + (bh0 + my_h) * p.n_cap;
  const size_t vpage = size_t(p.H_kv) * kPage * kHeadDim;
  const uint16_t* vbase = p.v_pool + size_t(g) * kPage * kHeadDim + r * 8;
  for (int cb = 0; cb < U; cb += kCh) {
    // list this chunk of the union in LDS
    if (tid < kWordsPerTile) {
      int pos = int(ex) - cb;
      uint64_t x = uw;
      while (x && pos < kCh) {
        const int bit = __ffsll((unsigned long long)x) - 1;
        x &= x - 1ull;
        if (pos >= 0) {
          uint32_t mem = 0;
          if ((wm >> bit) & 1ull) {
            mem = (1u << G) - 1u;
          } else {
#pragma unroll
            for (int hh = 0; hh < G; ++hh) mem |= uint32_t((bm[hh][tid] >> bit) & 1ull) << hh;
          }
          ulist[pos] = uint32_t(tid * 64 + bit) | (mem << 13);
        }
        ++pos;
      }
    }
    __syncthreads();
    const int cnt = min(kCh, U - cb);
    // (A) pair q = i * G + h: row i, head h = my_h; kWBatch pairs per lane
    // in flight
    for (int q0 = 0; q0 < cnt * G; q0 += kGathThreads * kWBatch) {
      float z[kWBatch];
      bool in[kWBatch];
#pragma unroll
      for (int u = 0; u < kWBatch; ++u) {
        const int i = (q0 + u * kGathThreads + tid) / G;
        in[u] = false;
        z[u] = 0.0f;
        if (i < cnt) {
          const uint32_t e = ulist[i];
          in[u] = ((e >> (13 + my_h)) & 1u) != 0u;
          if (in[u]) z[u] = zrow[t0 + int(e & 8191u)];
        }
      }
#pragma unroll
      for (int u = 0; u < kWBatch; ++u) {
        const int i = (q0 + u * kGathThreads + tid) / G;
        const float w = in[u] ? expf(z[u] - mref_h) : 0.0f;
        zsum += w;
        if (i < cnt) s_w[i][my_h] = w;
      }
    }
    __syncthreads();
    // (B) 4 rows per wave step, 16 lanes x 8 dims per V row
    for (int i0 = wave * 4 + row; i0 < cnt; i0 += kGathWaves * 4 * kVRows) {
      uint4 v[kVRows];
#pragma unroll
      for (int u = 0; u < kVRows; ++u) {
        const int i = i0 + u * kGathWaves * 4;
        const int off = i < cnt ? int(ulist[i] & 8191u) : 0;
        const int pg = s_pg[off >> 6];
        v[u] = i < cnt ? *reinterpret_cast<const uint4*>(vbase + size_t(pg) * vpage +
                                                         size_t((t0 + off) & 63) * kHeadDim)
                       : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < kVRows; ++u) {
        const int i = i0 + u * kGathWaves * 4;
        if (i >= cnt) break;
        const float vf[8] = {bf16lo(v[u].x), bf16hi(v[u].x), bf16lo(v[u].y), bf16hi(v[u].y),
                             bf16lo(v[u].z), bf16hi(v[u].z), bf16lo(v[u].w), bf16hi(v[u].w)};
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const float w = s_w[i][hh];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[hh][e] += w * vf[e];
        }
      }
    }
    __syncthreads();
  }
  // Z per head: lanes with equal tid % G of each wave, then the waves
#pragma unroll
  for (int m = G; m < 64; m <<= 1) zsum += __shfl_xor(zsum, m);
  float zs[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) zs[hh] = __shfl(zsum, hh);
  // sum the 4 rows of each wave, then the waves
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
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

// ---------------------------------------------------------------- merge
// One block per (sequence, query head): 8 groups of 32 threads each take
// every 8th tile, 4 dims per thread (float4 loads issued kMergeUnroll deep),
// then the groups are summed in LDS in a fixed order.
constexpr int kMergeThreads = 256;
constexpr int kMergeGroups = kMergeThreads / 32;
constexpr int kMergeUnroll = 4;

constexpr int kMergeTiles = 8;  // tiles per out_idx copy block

// out_idx for tiles [c * kMergeTiles, (c + 1) * kMergeTiles) of head bh.
__device__ void copy_positions(const Params& p, int bh, int c, int nt) {
  const int tid = threadIdx.x;
  const int ta = c * kMergeTiles;
  if (ta >= nt) return;
  const int tb = min(nt, ta + kMergeTiles);
  __shared__ uint32_t s_pre[kMergeTiles + 1];
  __shared__ uint32_t s_part[kMergeThreads / 64];
  const uint32_t* sc = p.scnt + size_t(bh) * p.n_tiles;
  // offset: retrieved positions of the tiles before ta
  uint32_t before = 0;
  for (int t = tid; t < ta; t += kMergeThreads) before += sc[t];
  before = wave_sum(before);
  if ((tid & 63) == 0) s_part[tid >> 6] = before;
  if (tid == 0) {
    uint32_t run = 0;
    for (int t = ta; t < tb; ++t) {
      s_pre[t - ta] = run;
      run += sc[t];
    }
    s_pre[tb - ta] = run;
  }
  __syncthreads();
  uint32_t off = 0;
  for (int w = 0; w < kMergeThreads / 64; ++w) off += s_part[w];
  const uint32_t total = s_pre[tb - ta];
  int32_t* dst = p.out_idx + size_t(bh) * p.k_max;
  const int32_t* src = reinterpret_cast<const int32_t*>(p.cand + size_t(bh) * p.n_cap);
  for (uint32_t base = 0; base < total; base += kMergeThreads * kMergeUnroll) {
    int32_t v[kMergeUnroll];
    uint32_t at[kMergeUnroll];
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const uint32_t i = base + u * kMergeThreads + tid;
      int j = 0;
      while (j + 1 < tb - ta && s_pre[j + 1] <= i) ++j;
      at[u] = off + i;
      v[u] = i < total ? src[size_t(ta + j) * (2 * kTile) + (i - s_pre[j])] : 0;
    }
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const uint32_t i = base + u * kMergeThreads + tid;
      if (i < total && at[u] < uint32_t(p.k_max)) dst[at[u]] = v[u];
    }
  }
}

// Grid (1 + copy blocks, B * H_q): x == 0 merges the partials of head y,
// x > 0 copies positions.
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(Params p) {
  const int bh = blockIdx.y;
  const int b = bh / p.H_q;
  const SeqGeom sg = seq_geom(p, b);
  const int nt = (sg.N + kTile - 1) / kTile;
  if (blockIdx.x > 0) {
    if (p.k_max > 0 && sg.k_eff > 0) copy_positions(p, bh, int(blockIdx.x) - 1, nt);
    return;
  }
  const int tid = threadIdx.x;
  const int grp = tid >> 5;
  const int d0 = (tid & 31) * 4;
  const float* mz = p.part_mz + size_t(bh) * p.n_tiles * 2;
  const float* pn = p.part_n + size_t(bh) * p.n_tiles * kHeadDim + d0;
  __shared__ float s_red[kMergeGroups][kHeadDim + 4];
  __shared__ float s_m[kMergeThreads / 64];


  // m = max over tiles with a non-empty partial
  float m = -INFINITY;
  for (int t = tid; t < nt; t += kMergeThreads) m = fmaxf(m, mz[2 * t + 1] > 0.0f ? mz[2 * t] : -INFINITY);
  m = wave_max(m);
  if ((tid & 63) == 0) s_m[tid >> 6] = m;
  __syncthreads();
  m = s_m[0];
  for (int w = 1; w < kMergeThreads / 64; ++w) m = fmaxf(m, s_m[w]);

  float Z = 0.0f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (m > -INFINITY) {
    for (int t0 = grp; t0 < nt; t0 += kMergeGroups * kMergeUnroll) {
      float2 w2[kMergeUnroll];
      float4 v[kMergeUnroll];
#pragma unroll
      for (int u = 0; u < kMergeUnroll; ++u) {
        const int t = t0 + u * kMergeGroups;
        w2[u] = t < nt ? *reinterpret_cast<const float2*>(mz + 2 * t) : make_float2(0.f, 0.f);
        v[u] = t < nt ? *reinterpret_cast<const float4*>(pn + size_t(t) * kHeadDim)
                      : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < kMergeUnroll; ++u) {
        const float sc = w2[u].y > 0.0f ? expf(w2[u].x - m) : 0.0f;
        Z += sc * w2[u].y;
        acc.x += sc * v[u].x;
        acc.y += sc * v[u].y;
        acc.z += sc * v[u].z;
        acc.w += sc * v[u].w;
      }
    }
  }
  s_red[grp][d0 + 0] = acc.x;
  s_red[grp][d0 + 1] = acc.y;
  s_red[grp][d0 + 2] = acc.z;
  s_red[grp][d0 + 3] = acc.w;
  if ((tid & 31) == 0) s_red[grp][kHeadDim] = Z;
  __syncthreads();
  if (tid < kHeadDim) {
    float a = 0.0f, zz = 0.0f;
    for (int gI = 0; gI < kMergeGroups; ++gI) {
      a += s_red[gI][tid];
      zz += s_red[gI][kHeadDim];
    }
    p.out[size_t(bh) * kHeadDim + tid] = zz > 0.0f ? a / zz : 0.0f;
    if (tid == 0 && p.lse) p.lse[bh] = zz > 0.0f ? m + logf(zz) : -INFINITY;
  }
  if (p.k_max > 0) {
    int32_t* dst = p.out_idx + size_t(bh) * p.k_max;
    for (int i = sg.k_eff + tid; i < p.k_max; i += kMergeThreads) dst[i] = -1;
  }
}

hipError_t launch_merge(const Params& p, hipStream_t s) {
  const unsigned copies = p.k_max > 0 ? unsigned((p.n_tiles + kMergeTiles - 1) / kMergeTiles) : 0u;
  hipLaunchKernelGGL(merge_kernel, dim3(1 + copies, unsigned(p.B * p.H_q)), dim3(kMergeThreads), 0,
                     s, p);
  return hipGetLastError();
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

}  // namespace ra
