// Search of a query-aware key graph with decode queries (RetrievalAttention
// slides, frame "Prefill queries teach the key graph what matters", step 4:
// each new decode query searches the key-only graph projected from the
// prefill queries' top-k links). One block of kGsWaves waves per query head
// runs a best-first search: a result list R holds the ef best keys visited
// so far by (score, lower position); each round expands the kGsWaves best
// keys of R not yet expanded, one per wave; every neighbour not visited
// before is visited, scored and offered to R; the search ends when every
// key of R has been expanded.
//
// A score is q . k in fp32 with the bf16 products (exact in fp32) added one
// dimension after another, 0 to 127, each sum rounded (an fma chain): the
// search's decisions then follow from values both it and a reference can
// reproduce bit for bit. The factor 1/sqrt(d) is left out (it does not
// change the order).
//
// Lane i of a wave scores the i-th neighbour of its key (degree <= 64).
// The visited set is a bitmap in LDS (one bit per position, N <= 2^20);
// R is kept sorted in LDS, and the new keys of a round are merged into it
// by rank: an existing entry moves down by the number of new keys better
// than it, a new key lands after the entries and new keys better than it.
#include <climits>

#include "ra_internal.h"

namespace ra {

constexpr int kGsMaxEf = RA_GRAPH_MAX_EF;
constexpr int kGsWaves = kGsBatch;          // keys expanded per round, one per wave
constexpr int kGsThreads = kGsWaves * 64;
static_assert(kGsThreads >= kGsMaxEf, "one thread per entry of R");
// Rounds with more new keys than this sort them first (bitonic, in LDS), so
// that every rank is a binary search; fewer are ranked by counting.
constexpr int kGsSortMin = 128;

struct GsLds {
  float rs[2][kGsMaxEf];  // R, double-buffered: score, position, expanded
  int32_t rp[2][kGsMaxEf];
  int32_t rx[2][kGsMaxEf];
  // the keys new in this round, then padding to a multiple of 4 that ranks
  // below every key (read four at a time by the merge)
  __align__(16) float ns[kGsThreads];
  __align__(16) int32_t nu[kGsThreads];
  int32_t cand[kGsWaves]; // the keys expanded in this round
  int32_t cnt[kGsWaves];  // per wave: unexpanded entries, then new keys kept
  int32_t fcnt[kGsWaves]; // per wave: keys visited for the first time
};

// a ranks before b: larger score, then lower position
__device__ __forceinline__ bool gs_better(float sa, int32_t pa, float sb, int32_t pb) {
  return sa > sb || (sa == sb && pa < pb);
}

// bt: the block table's entries, already checked, in LDS; or null (read
// it from global memory).
__device__ __forceinline__ float gs_score(const GsParams& p, int g, const uint32_t (&qw)[64],
                                          int32_t u, const int32_t* bt) {
  int32_t pg;
  if (bt) {
    pg = bt[u >> 6];
  } else {
    pg = p.block_table[u >> 6];
    pg = ((unsigned)pg < (unsigned)p.num_pages) ? pg : 0;
  }
  const uint4* kr = reinterpret_cast<const uint4*>(
      p.k_pool + ((size_t(pg) * p.H_kv + g) * kPage + (u & 63)) * kHeadDim);
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const uint4 x = kr[c];
    const uint32_t kw[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t qq = qw[4 * c + i], kk = kw[i];
      // dimension 2 (4 c + i), then 2 (4 c + i) + 1: low half first
      s = fmaf(__uint_as_float(qq << 16), __uint_as_float(kk << 16), s);
      s = fmaf(__uint_as_float(qq & 0xFFFF0000u), __uint_as_float(kk & 0xFFFF0000u), s);
    }
  }
  return s;
}

// Sum of v over the waves before this one, and over all waves (v in LDS,
// one entry per wave, written before the last barrier).
__device__ __forceinline__ void gs_wave_prefix(const int32_t* v, int wave, int& before, int& total) {
  before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kGsWaves; ++w) {
    before += w < wave ? v[w] : 0;
    total += v[w];
  }
}

// BT_LDS: the block table's entries for [0, N) follow the bitmap in LDS.
template <bool BT_LDS>
__global__ __launch_bounds__(kGsThreads) void graph_search_kernel(GsParams p) {
  extern __shared__ uint32_t vis[];  // visited bitmap, p.vis_words words
  __shared__ GsLds sm;
  const int h = blockIdx.x;
  const int g = h / (p.H_q / p.H_kv);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = p.N, D = p.D, ef = p.ef;
  int32_t* out = p.out_idx + size_t(h) * p.k;

  for (int i = tid; i < p.vis_words; i += kGsThreads) vis[i] = 0u;
  int32_t* bt = nullptr;
  if constexpr (BT_LDS) {
    bt = reinterpret_cast<int32_t*>(vis + p.vis_words);
    for (int i = tid; i < (N + kPage - 1) / kPage; i += kGsThreads) {
      const int32_t pg = p.block_table[i];
      bt[i] = ((unsigned)pg < (unsigned)p.num_pages) ? pg : 0;
    }
  }
  const int32_t e = p.entry[h];
  if (e < 0 || e >= N) {  // block-uniform
    for (int i = tid; i < p.k; i += kGsThreads) out[i] = -1;
    if (tid == 0) p.out_visited[h] = 0;
    return;
  }
  uint32_t qw[64];
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
  const int32_t* nbr = p.nbr + size_t(h) * N * D;
  __syncthreads();
  if (tid == 0) {
    vis[e >> 5] |= 1u << (e & 31);
    sm.rs[0][0] = gs_score(p, g, qw, e, bt);
    sm.rp[0][0] = e;
    sm.rx[0][0] = 0;
  }
  int cur = 0, nr = 1;
  uint32_t visited = 1;
  __syncthreads();

  // every round expands at least one key of R and a key enters R once
  for (int iter = 0; iter <= N; ++iter) {
    // the kGsWaves best unexpanded entries of R (sorted), in order
    const bool un = tid < nr && !sm.rx[cur][tid];
    uint64_t bal = __ballot(un);
    if (lane == 0) sm.cnt[wave] = __popcll(bal);
    __syncthreads();
    int before, total;
    gs_wave_prefix(sm.cnt, wave, before, total);
    const int nb = min(total, kGsWaves);
    if (nb == 0) break;  // block-uniform
    if (un) {
      const int r = before + __popcll(bal & ((1ull << lane) - 1ull));
      if (r < kGsWaves) {
        sm.cand[r] = sm.rp[cur][tid];
        sm.rx[cur][tid] = 1;
      }
    }
    __syncthreads();

    // wave w expands the w-th of them; lane i takes its i-th neighbour
    bool fresh = false;
    int32_t u = -1;
    if (wave < nb && lane < D) {
      u = nbr[size_t(sm.cand[wave]) * D + lane];
      if (u >= 0 && u < N) {
        const uint32_t bit = 1u << (u & 31);
        fresh = (atomicOr(&vis[u >> 5], bit) & bit) == 0u;
      }
    }
    const float s = fresh ? gs_score(p, g, qw, u, bt) : 0.0f;
    // a key that ranks below the last entry of a full R can never enter it:
    // it counts as visited, and only the others are merged
    const bool full = nr >= ef;
    const bool keep = fresh && (!full || gs_better(s, u, sm.rs[cur][ef - 1], sm.rp[cur][ef - 1]));
    const uint64_t fb = __ballot(fresh);
    bal = __ballot(keep);
    __syncthreads();  // every wave has read sm.cnt
    if (lane == 0) {
      sm.cnt[wave] = __popcll(bal);
      sm.fcnt[wave] = __popcll(fb);
    }
    __syncthreads();
    int m, nf;
    gs_wave_prefix(sm.fcnt, wave, before, nf);
    gs_wave_prefix(sm.cnt, wave, before, m);
    visited += uint32_t(nf);
    if (keep) {
      const int slot = before + __popcll(bal & ((1ull << lane) - 1ull));
      sm.ns[slot] = s;
      sm.nu[slot] = u;
    }
    const int m4 = (m + 3) & ~3;
    if (tid >= m && tid < m4) {
      sm.ns[tid] = -INFINITY;
      sm.nu[tid] = INT_MAX;
    }
    __syncthreads();
    if (m == 0) continue;  // block-uniform

    // merge by rank into the other buffer, keeping the best ef
    const int nxt = cur ^ 1;
    const bool sorted = m > kGsSortMin;  // block-uniform
    if (sorted) {
      // best first over P = the power of two >= m (the padding, ranking
      // below every key, ends up behind them)
      int P = 4;
      while (P < m) P <<= 1;
      for (int i = m4 + tid; i < P; i += kGsThreads) {
        sm.ns[i] = -INFINITY;
        sm.nu[i] = INT_MAX;
      }
      __syncthreads();
      // Partners less than 64 apart are in the same wave: those steps run
      // in registers with shuffles, the others through LDS. P >= 256 is a
      // whole number of waves.
      const bool inP = tid < P;  // wave-uniform
      auto wave_steps = [&](int kb, int j) {
        float a = sm.ns[tid];
        int32_t ua = sm.nu[tid];
        for (; j > 0; j >>= 1) {
          const float b = __shfl_xor(a, j);
          const int32_t ub = __shfl_xor(ua, j);
          // the lower slot of an ascending pair, or the upper of a
          // descending one, takes the better key
          const bool want_better = ((tid & j) == 0) == ((tid & kb) == 0);
          const bool take = want_better ? gs_better(b, ub, a, ua) : gs_better(a, ua, b, ub);
          if (take) {
            a = b;
            ua = ub;
          }
        }
        sm.ns[tid] = a;
        sm.nu[tid] = ua;
      };
      if (inP) {
        for (int kb = 2; kb <= 64; kb <<= 1) wave_steps(kb, kb >> 1);
      }
      __syncthreads();
      for (int kb = 128; kb <= P; kb <<= 1) {
        for (int j = kb >> 1; j >= 64; j >>= 1) {
          const int l = tid ^ j;
          if (inP && l > tid) {
            const float a = sm.ns[tid], b = sm.ns[l];
            const int32_t ua = sm.nu[tid], ub = sm.nu[l];
            const bool sw = (tid & kb) == 0 ? gs_better(b, ub, a, ua) : gs_better(a, ua, b, ub);
            if (sw) {
              sm.ns[tid] = b;
              sm.ns[l] = a;
              sm.nu[tid] = ub;
              sm.nu[l] = ua;
            }
          }
          __syncthreads();
        }
        if (inP) wave_steps(kb, 32);
        __syncthreads();
      }
    }
    const float4* ns4 = reinterpret_cast<const float4*>(sm.ns);
    const int4* nu4 = reinterpret_cast<const int4*>(sm.nu);
    // how many of the new keys rank before (s, u)
    auto new_before = [&](float s, int32_t u) {
      int c = 0;
      if (sorted) {
        int hi = m;  // the new keys better than (s, u) are a prefix
        while (c < hi) {
          const int mid = (c + hi) >> 1;
          if (gs_better(sm.ns[mid], sm.nu[mid], s, u)) c = mid + 1; else hi = mid;
        }
        return c;
      }
      for (int j = 0; j < m4 / 4; ++j) {
        const float4 a = ns4[j];
        const int4 b = nu4[j];
        c += (gs_better(a.x, b.x, s, u) ? 1 : 0) + (gs_better(a.y, b.y, s, u) ? 1 : 0) +
             (gs_better(a.z, b.z, s, u) ? 1 : 0) + (gs_better(a.w, b.w, s, u) ? 1 : 0);
      }
      return c;
    };
    if (tid < nr) {
      const float si = sm.rs[cur][tid];
      const int32_t pi = sm.rp[cur][tid];
      const int shift = new_before(si, pi);
      const int pos = tid + shift;
      if (pos < ef) {
        sm.rs[nxt][pos] = si;
        sm.rp[nxt][pos] = pi;
        sm.rx[nxt][pos] = sm.rx[cur][tid];
      }
    }
    if (tid < m) {
      const float sx = sm.ns[tid];
      const int32_t ux = sm.nu[tid];
      int lo = 0, hi = nr;  // entries of R better than the new key
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (gs_better(sm.rs[cur][mid], sm.rp[cur][mid], sx, ux)) lo = mid + 1; else hi = mid;
      }
      const int pos = lo + new_before(sx, ux);
      if (pos < ef) {
        sm.rs[nxt][pos] = sx;
        sm.rp[nxt][pos] = ux;
        sm.rx[nxt][pos] = 0;
      }
    }
    __syncthreads();
    nr = min(ef, nr + m);
    cur = nxt;
  }

  // the best min(k, |R|) keys, ascending by position
  const int kk = min(p.k, nr);
  if (tid < kk) {
    const int32_t pi = sm.rp[cur][tid];
    int rank = 0;
    for (int j = 0; j < kk; ++j) rank += sm.rp[cur][j] < pi ? 1 : 0;
    out[rank] = pi;
  }
  for (int i = kk + tid; i < p.k; i += kGsThreads) out[i] = -1;
  if (tid == 0) p.out_visited[h] = int32_t(visited);
}

hipError_t launch_graph_search(const GsParams& p, hipStream_t s) {
  const size_t vis = size_t(p.vis_words) * sizeof(uint32_t);
  const size_t bt = size_t((p.N + kPage - 1) / kPage) * sizeof(int32_t);
  // the block table joins the bitmap in LDS when both fit a CU's 160 KB
  if (vis + bt + sizeof(GsLds) + 1024 <= 160 * 1024)
    hipLaunchKernelGGL(graph_search_kernel<true>, dim3(p.H_q), dim3(kGsThreads), vis + bt, s, p);
  else
    hipLaunchKernelGGL(graph_search_kernel<false>, dim3(p.H_q), dim3(kGsThreads), vis, s, p);
  return hipGetLastError();
}

}  // namespace ra
