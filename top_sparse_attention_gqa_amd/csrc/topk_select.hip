// Exact top-k over the selection domain M = [lo, hi) of each query head,
// ties to the lower position: the fixed retrieval budget of the
// RetrievalAttention slides ("Sparse attention renormalizes selected tokens",
// and "The GPU keeps 640 fixed positions": W excluded, per-head indices).
//
// Scores are compared through an order-preserving uint32 key, and the
// choice among members is made on the composite  c = key' << 32 | ~n
// (key' = key minus a known lower bound): a larger composite is a larger
// score, then a lower position, and all composites are distinct, so "the
// k_eff largest composites" is the unique tie-broken top-k.
//
// select (one block per head): the scan left every member of M scoring at
// or above the head's sampled threshold in per-tile candidate lists. If they
// hold at least k_eff entries, the top-k of M is the top-k of the lists; a
// radix select on the composite finds the exact threshold (the bucket around
// the k-th entry is finished in LDS) and records it in the head state. The
// members are taken later, tile by tile, by the gather blocks. A head with
// too few candidates is flagged; the dense stage rescans its group with
// every member of M as a candidate and selects again.
#include "ra_internal.h"

namespace ra {

constexpr int kSelThreads = 1024;
constexpr int kWin = 2048;                 // tiles per LDS prefix window
constexpr int kSubCap = 4096;              // LDS list for one radix sub-bucket

// ---------------------------------------------------------------- sources
// Each source enumerates composites of members with (c, n).

// Entries loaded per thread before any is used, so that a pass over a list
// costs a few memory round trips rather than one per entry.
constexpr int kBatch = 8;

// A head's per-tile candidate lists (entries key << 32 | n; the list of
// tile t holds tcnt[t] entries from list + t * kTile), enumerated as
// composites c = (key - lo) << 32 | ~n. The list lengths of a window of
// kWin tiles are prefix-summed in LDS; entry i of the window is found by a
// binary search over that prefix. In dense mode the lengths follow from the
// geometry: every member of M is in its tile's list.
struct TileLists {
  const uint64_t* list;
  const uint32_t* tcnt;
  uint32_t* pre;      // LDS [kWin + 1]
  int32_t* s_w0;      // LDS: first tile of the window held in pre (-1: none)
  int64_t* tmp;       // LDS [16]
  int t_lo, t_hi;     // tiles that overlap M
  int m_lo, m_hi;     // M
  uint32_t lo;
  bool dense;

  __device__ __forceinline__ uint32_t tile_count(int t) const {
    if (!dense) return tcnt[t];
    const int a = max(t * kTile, m_lo), e = min((t + 1) * kTile, m_hi);
    return e > a ? uint32_t(e - a) : 0u;
  }

  // Prefix of the list lengths of tiles [w0, w0 + nw). Block-wide.
  __device__ void load(int w0, int nw) const {
    if (*s_w0 == w0) return;
    constexpr int per = kWin / kSelThreads;
    const int tid = threadIdx.x;
    uint32_t c[per];
    int64_t sum = 0;
#pragma unroll
    for (int u = 0; u < per; ++u) {
      const int i = tid * per + u;
      c[u] = i < nw ? tile_count(w0 + i) : 0u;
      sum += c[u];
    }
    int64_t total;
    int64_t run = block_excl_scan(sum, tmp, &total);
#pragma unroll
    for (int u = 0; u < per; ++u) {
      pre[tid * per + u] = uint32_t(run);
      run += c[u];
    }
    if (tid == 0) {
      pre[kWin] = uint32_t(total);
      *s_w0 = w0;
    }
    __syncthreads();
  }

  template <typename Fn>
  __device__ __forceinline__ void for_each(Fn&& fn) const {
    const uint32_t l = lo;
    for (int w0 = t_lo; w0 < t_hi; w0 += kWin) {
      const int nw = min(kWin, t_hi - w0);
      load(w0, nw);
      const uint32_t total = pre[kWin];
      const uint32_t step = blockDim.x * kBatch;
      for (uint32_t base = 0; base < total; base += step) {
        uint64_t v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const uint32_t i = base + u * blockDim.x + threadIdx.x;
          v[u] = 0ull;
          if (i < total) {
            int a = 0, e = nw - 1;
            while (a < e) {
              const int mid = (a + e + 1) >> 1;
              if (pre[mid] <= i) a = mid; else e = mid - 1;
            }
            v[u] = list[size_t(w0 + a) * kTile + (i - pre[a])];
          }
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          if (base + u * blockDim.x + threadIdx.x < total) {
            const uint32_t n = uint32_t(v[u]);
            fn((uint64_t(uint32_t(v[u] >> 32) - l) << 32) | uint32_t(~n), int(n));
          }
        }
      }
      if (t_hi - t_lo > kWin) __syncthreads();
    }
  }
};

// Composites already reduced to one sub-bucket, in LDS.
struct LdsSource {
  const uint64_t* c;
  uint32_t count;
  template <typename Fn>
  __device__ __forceinline__ void for_each(Fn&& fn) const {
    for (uint32_t i = threadIdx.x; i < count; i += blockDim.x) {
      const uint64_t v = c[i];
      fn(v, int(~uint32_t(v)));
    }
  }
};

struct Radix {
  uint32_t* hist;  // LDS [2048]
  uint32_t* s_d;   // LDS scalars: chosen digit, count above it, its count
  uint32_t* s_above;
  uint32_t* s_cnt;
};

// One radix pass: histogram the next w bits of the composites whose top
// plen bits equal prefix, then pick the digit where the running count from
// the top reaches need. Updates need/prefix/plen; returns the chosen digit's
// population (all block threads get the same values).
template <typename Src>
__device__ uint32_t radix_pass(const Src& src, const Radix& rx, int TB, uint32_t& need,
                               uint64_t& prefix, int& plen) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int w = min(11, TB - plen);
  const int shift = TB - plen - w;
  for (int i = tid; i < 2048; i += blockDim.x) rx.hist[i] = 0;
  __syncthreads();
  const int pl = plen;
  const uint64_t pf = prefix;
  const uint32_t dmask = (1u << w) - 1u;
  src.for_each([&](uint64_t c, int) {
    if (pl == 0 || (c >> (TB - pl)) == pf) atomicAdd(&rx.hist[uint32_t(c >> shift) & dmask], 1u);
  });
  __syncthreads();
  if (wave == 0) {
    uint32_t s = 0;
    for (int i = 0; i < 32; ++i) s += rx.hist[lane * 32 + i];
    const uint32_t suf = wave_suffix_sum(s);
    const uint64_t m = __ballot(suf >= need);
    const int L = m ? 63 - __clzll(m) : 0;
    if (lane == L) {
      uint32_t acc = suf - s;
      for (int i = 31; i >= 0; --i) {
        const uint32_t v = rx.hist[lane * 32 + i];
        if (acc + v >= need || i == 0) {
          *rx.s_d = uint32_t(lane * 32 + i);
          *rx.s_above = acc;
          *rx.s_cnt = v;
          break;
        }
        acc += v;
      }
    }
  }
  __syncthreads();
  need -= *rx.s_above;
  prefix = (prefix << w) | *rx.s_d;
  plen += w;
  const uint32_t cnt = *rx.s_cnt;
  __syncthreads();
  return cnt;
}

// Passes until the chosen digit's whole population is needed (or every bit
// is fixed, where the population is one).
template <typename Src>
__device__ void radix_finish(const Src& src, const Radix& rx, int TB, uint32_t& need,
                             uint64_t& prefix, int& plen) {
  while (plen < TB) {
    if (radix_pass(src, rx, TB, need, prefix, plen) == need) break;
  }
}

// Composite prefix (top plen of TB bits) of the need-th largest member of a
// source: one pass over it; if that does not settle it and the chosen
// sub-bucket fits LDS, the sub-bucket is copied there and finished in LDS.
// Members whose top plen bits are >= the returned prefix are exactly the
// need largest.
template <typename Src>
__device__ void find_threshold(const Src& src, const Radix& rx, int TB, uint32_t need,
                               uint64_t* sub, uint32_t* s_n, uint64_t& prefix, int& plen) {
  prefix = 0;
  plen = 0;
  const uint32_t cnt1 = radix_pass(src, rx, TB, need, prefix, plen);
  if (cnt1 == need || plen >= TB) return;
  if (cnt1 > uint32_t(kSubCap)) {
    radix_finish(src, rx, TB, need, prefix, plen);
    return;
  }
  if (threadIdx.x == 0) *s_n = 0;
  __syncthreads();
  const uint64_t pf = prefix;
  const int pl = plen;
  src.for_each([&](uint64_t c, int) {
    if ((c >> (TB - pl)) == pf) sub[atomicAdd(s_n, 1u)] = c;
  });
  __syncthreads();
  const LdsSource lds{sub, *s_n};
  radix_finish(lds, rx, TB, need, prefix, plen);
}

// ---------------------------------------------------------------- select
__device__ __forceinline__ int bit_length(uint32_t x) { return 32 - __clz(x); }

// Exact threshold of head bh over its lists; writes it into the head state.
__device__ void decide(const Params& p, int bh, const SeqGeom& sg, uint32_t lo, uint32_t max_m,
                       bool dense) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t s_d, s_above, s_cnt, s_n;
  __shared__ uint64_t sub[kSubCap];
  __shared__ uint32_t pre[kWin + 1];
  __shared__ int32_t s_w0;
  __shared__ int64_t tmp[16];
  if (threadIdx.x == 0) s_w0 = -1;
  __syncthreads();
  const uint32_t span = max_m > lo ? max_m - lo : 1u;
  const int TB = 32 + bit_length(span);
  const TileLists src{p.cand + size_t(bh) * p.n_cap, p.tcnt + size_t(bh) * p.n_tiles, pre, &s_w0,
                      tmp, sg.lo / kTile, (sg.hi - 1) / kTile + 1, sg.lo, sg.hi, lo, dense};
  const Radix rx{hist, &s_d, &s_above, &s_cnt};
  uint64_t prefix;
  int plen;
  find_threshold(src, rx, TB, uint32_t(sg.k_eff), sub, &s_n, prefix, plen);
  if (threadIdx.x == 0) {
    HeadState& w = p.state[bh];
    w.lo_key = lo;
    w.thr_shift = uint32_t(TB - plen);
    w.thr_lo = uint32_t(prefix);
    w.thr_hi = uint32_t(prefix >> 32);
  }
}

// One block per head: count the candidates; decide the threshold, or flag
// the head (and its group) for the rescan when there are fewer than k_eff.
__global__ __launch_bounds__(kSelThreads) void select_kernel(Params p) {
  const int bh = blockIdx.x;
  const int b = bh / p.H_q;
  const int g = (bh - b * p.H_q) / p.G;
  const SeqGeom sg = seq_geom(p, b);
  if (sg.k_eff == 0) return;  // the unset threshold takes nothing
  __shared__ int64_t tmp[16];
  const int t_lo = sg.lo / kTile, t_hi = (sg.hi - 1) / kTile + 1;
  const uint32_t* tc = p.tcnt + size_t(bh) * p.n_tiles;
  int64_t c = 0;
  for (int t = t_lo + int(threadIdx.x); t < t_hi; t += kSelThreads) c += tc[t];
  int64_t m;
  block_excl_scan(c, tmp, &m);
  const HeadState st = p.state[bh];
  if (m < sg.k_eff) {
    if (threadIdx.x == 0) {
      p.state[bh].dense = 1u;
      atomicOr(&p.gflag[size_t(b) * p.H_kv + g], 1u);
      atomicAdd(p.any_dense, 1u);
    }
    return;
  }
  decide(p, bh, sg, st.lo_key, st.max_m, false);
}

hipError_t launch_select(const Params& p, hipStream_t s) {
  hipLaunchKernelGGL(select_kernel, dim3(unsigned(p.B * p.H_q)), dim3(kSelThreads), 0, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------- dense
// After the rescan: the flagged heads select over every member of M (their
// lists now hold all of it, so the candidate counts are the tile sizes).
__global__ __launch_bounds__(kSelThreads) void reselect_kernel(Params p) {
  if (*p.any_dense == 0u) return;
  const int bh = blockIdx.x;
  const HeadState st = p.state[bh];
  if (!st.dense) return;
  const SeqGeom sg = seq_geom(p, bh / p.H_q);
  const int t_lo = sg.lo / kTile, t_hi = (sg.hi - 1) / kTile + 1;
  uint32_t* tc = p.tcnt + size_t(bh) * p.n_tiles;
  for (int t = t_lo + int(threadIdx.x); t < t_hi; t += kSelThreads) {
    const int a = max(t * kTile, sg.lo), e = min((t + 1) * kTile, sg.hi);
    tc[t] = uint32_t(e - a);
  }
  decide(p, bh, sg, 0u, st.max_m, true);
}

hipError_t launch_dense_scan(const Params& p, hipStream_t s);  // score_scan.hip

hipError_t launch_dense(const Params& p, hipStream_t s) {
  hipError_t e = launch_dense_scan(p, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(reselect_kernel, dim3(unsigned(p.B * p.H_q)), dim3(kSelThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace ra
