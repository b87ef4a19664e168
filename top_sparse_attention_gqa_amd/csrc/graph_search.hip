// Search of a query-aware key graph with decode queries (RetrievalAttention
// slides, frame "Prefill queries teach the key graph what matters", step 4:
// each new decode query searches the key-only graph projected from the
// prefill queries' top-k links). One wave per query head runs a best-first
// search: a result list R holds the ef best keys visited so far by
// (score, lower position); the best key of R not yet expanded is expanded,
// every neighbour not visited before is visited, scored and offered to R;
// the search ends when every key of R has been expanded.
//
// A score is q . k in fp32 with the bf16 products (exact in fp32) added one
// dimension after another, 0 to 127, each sum rounded (an fma chain): the
// search's decisions then follow from values both it and a reference can
// reproduce bit for bit. The factor 1/sqrt(d) is left out (it does not
// change the order).
//
// Lane i scores the i-th neighbour of the expanded key (degree <= 64). The
// visited set is a bitmap in the workspace (one bit per position); R is
// kept sorted in LDS, and the new keys of an expansion are merged into it
// by rank: an existing entry moves down by the number of new keys better
// than it, a new key lands after the entries and new keys better than it.
#include <climits>

#include "ra_internal.h"

namespace ra {

constexpr int kGsMaxEf = RA_GRAPH_MAX_EF;

struct GsLds {
  float rs[2][kGsMaxEf];  // R, double-buffered: score, position, expanded
  int32_t rp[2][kGsMaxEf];
  int32_t rx[2][kGsMaxEf];
  float ns[64];           // the keys new in this expansion
  int32_t nu[64];
};

// a ranks before b: larger score, then lower position
__device__ __forceinline__ bool gs_better(float sa, int32_t pa, float sb, int32_t pb) {
  return sa > sb || (sa == sb && pa < pb);
}

__device__ __forceinline__ float gs_score(const GsParams& p, const uint32_t (&qw)[64], int32_t u) {
  const int jp = u >> 6;
  int32_t pg = p.block_table[jp];
  pg = ((unsigned)pg < (unsigned)p.num_pages) ? pg : 0;
  const uint4* kr = reinterpret_cast<const uint4*>(
      p.k_pool + ((size_t(pg) * p.H_kv + p.g) * kPage + (u & 63)) * kHeadDim);
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

__global__ __launch_bounds__(64) void graph_search_kernel(GsParams p0) {
  __shared__ GsLds sm;
  const int h = blockIdx.x;
  const int lane = threadIdx.x;
  GsParams p = p0;
  p.g = h / (p.H_q / p.H_kv);
  const int N = p.N, D = p.D, ef = p.ef;
  uint32_t* vis = p.visited + size_t(h) * p.vis_words;
  int32_t* out = p.out_idx + size_t(h) * p.k;

  for (int i = lane; i < p.vis_words; i += 64) vis[i] = 0u;
  __threadfence();
  __builtin_amdgcn_wave_barrier();

  const int32_t e = p.entry[h];
  if (e < 0 || e >= N) {
    for (int i = lane; i < p.k; i += 64) out[i] = -1;
    if (lane == 0) p.out_visited[h] = 0;
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

  int cur = 0, nr = 1;
  uint32_t visited = 1;
  if (lane == 0) {
    atomicOr(&vis[e >> 5], 1u << (e & 31));
    sm.rs[0][0] = gs_score(p, qw, e);
    sm.rp[0][0] = e;
    sm.rx[0][0] = 0;
  }
  __builtin_amdgcn_wave_barrier();

  // every pass expands one key of R and every key enters R at most once
  for (int iter = 0; iter <= N; ++iter) {
    // the best key of R not yet expanded (R is sorted)
    int best = INT_MAX;
    for (int i = lane; i < nr; i += 64)
      if (!sm.rx[cur][i]) best = min(best, i);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) best = min(best, __shfl_xor(best, off));
    if (best == INT_MAX) break;
    const int32_t c = sm.rp[cur][best];
    __builtin_amdgcn_wave_barrier();
    if (lane == 0) sm.rx[cur][best] = 1;

    int32_t u = lane < D ? nbr[size_t(c) * D + lane] : -1;
    bool fresh = false;
    if (u >= 0 && u < N) {
      const uint32_t bit = 1u << (u & 31);
      fresh = (atomicOr(&vis[u >> 5], bit) & bit) == 0u;
    }
    const float s = fresh ? gs_score(p, qw, u) : 0.0f;
    const uint64_t mask = __ballot(fresh);
    const int m = __popcll(mask);
    if (m == 0) continue;
    visited += uint32_t(m);
    if (fresh) {
      const int slot = __popcll(mask & ((1ull << lane) - 1ull));
      sm.ns[slot] = s;
      sm.nu[slot] = u;
    }
    __builtin_amdgcn_wave_barrier();

    // merge by rank into the other buffer, keeping the best ef
    const int nxt = cur ^ 1;
    for (int i = lane; i < nr; i += 64) {
      const float si = sm.rs[cur][i];
      const int32_t pi = sm.rp[cur][i];
      int shift = 0;
      for (int j = 0; j < m; ++j) shift += gs_better(sm.ns[j], sm.nu[j], si, pi) ? 1 : 0;
      const int pos = i + shift;
      if (pos < ef) {
        sm.rs[nxt][pos] = si;
        sm.rp[nxt][pos] = pi;
        sm.rx[nxt][pos] = sm.rx[cur][i];
      }
    }
    if (lane < m) {
      const float sx = sm.ns[lane];
      const int32_t ux = sm.nu[lane];
      int lo = 0, hi = nr;  // entries of R better than the new key
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (gs_better(sm.rs[cur][mid], sm.rp[cur][mid], sx, ux)) lo = mid + 1; else hi = mid;
      }
      int rn = 0;
      for (int j = 0; j < m; ++j) rn += gs_better(sm.ns[j], sm.nu[j], sx, ux) ? 1 : 0;
      const int pos = lo + rn;
      if (pos < ef) {
        sm.rs[nxt][pos] = sx;
        sm.rp[nxt][pos] = ux;
        sm.rx[nxt][pos] = 0;
      }
    }
    __builtin_amdgcn_wave_barrier();
    nr = min(ef, nr + m);
    cur = nxt;
  }

  // the best min(k, |R|) keys, ascending by position
  const int kk = min(p.k, nr);
  for (int i = lane; i < kk; i += 64) {
    const int32_t pi = sm.rp[cur][i];
    int rank = 0;
    for (int j = 0; j < kk; ++j) rank += sm.rp[cur][j] < pi ? 1 : 0;
    out[rank] = pi;
  }
  for (int i = kk + lane; i < p.k; i += 64) out[i] = -1;
  if (lane == 0) p.out_visited[h] = int32_t(visited);
}

hipError_t launch_graph_search(const GsParams& p, hipStream_t s) {
  hipLaunchKernelGGL(graph_search_kernel, dim3(p.H_q), dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace ra
