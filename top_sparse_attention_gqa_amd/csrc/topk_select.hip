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
// threshold (one block per head, before the scan): from the keys of the
// sampled positions, a key at or just below the R-th largest sampled member
// (its top 22 bits), with R a conservative stand-in for the rank of the k-th
// largest member of M in the sample. Members at or above it are the head's
// candidates.
//
// select (one block per head, after the scan): if the per-unit candidate
// lists hold at least k_eff entries, the top-k of M is the top-k of the
// lists; a radix select on the composite finds the exact threshold (the
// bucket around the k-th entry is finished in LDS). The lists are read once
// into registers when they fit. A head with too few candidates is flagged;
// the dense stage rescans its group with every member of M as a candidate
// and selects again.
#include "ra_internal.h"

namespace ra {

constexpr int kSelThreads = 512;
constexpr int kSubCap = 2048;     // LDS list for one radix sub-bucket
constexpr uint32_t kRankMax = 256; // sub-buckets up to this size are finished by ranking
constexpr int kBatch = 8;         // global entries per lane in flight per pass
constexpr int kRegEntries = 64;   // candidate entries per lane kept in registers
constexpr int kRegKeys = 32;      // sampled keys per lane kept in registers

// ---------------------------------------------------------------- wave helpers
// Every lane of the wave must call these.

// Append v to an LDS list (capacity cap) for every lane with `flag`: one
// atomic per wave.
__device__ __forceinline__ void wave_append(uint64_t* list, uint32_t* n, uint32_t cap, uint64_t v,
                                            bool flag) {
  const uint64_t m = __ballot(flag);
  if (!m) return;
  const int lane = lane_id();
  const int leader = __ffsll((unsigned long long)m) - 1;
  uint32_t base = 0;
  if (lane == leader) base = atomicAdd(n, uint32_t(__popcll(m)));
  base = __shfl(base, leader);
  if (flag) {
    const uint32_t i = base + uint32_t(__popcll(m & ((1ull << lane) - 1ull)));
    if (i < cap) list[i] = v;
  }
}

// ---------------------------------------------------------------- sources
// A source enumerates composites: for_each(fn) calls fn(c, n, valid) in
// lockstep over the wave (valid is false for padding slots).

// A head's per-unit candidate lists in global memory (entries key << 32 | n;
// the list of unit u holds cnt(u) entries from list + u * kUnit), enumerated
// as composites c = (key - lo) << 32 | ~n. The list lengths of the units that
// overlap M are prefix-summed in LDS; entry i is found by a branch-free
// binary search over that prefix whose kBatch lookups proceed in lockstep.
struct UnitLists {
  const uint64_t* list;
  const uint32_t* pre;  // LDS [nu + 1]
  int u_lo, nu;         // units u_lo .. u_lo + nu - 1 overlap M
  uint32_t lo;

  __device__ __forceinline__ void locate(const uint32_t (&idx)[kBatch], int (&a)[kBatch]) const {
    const int top = nu > 1 ? 1 << (31 - __clz(nu - 1)) : 0;  // largest power of two < nu
#pragma unroll
    for (int u = 0; u < kBatch; ++u) a[u] = 0;
    for (int step = top; step > 0; step >>= 1) {
      uint32_t pv[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) pv[u] = pre[min(a[u] + step, nu - 1)];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) a[u] += (a[u] + step < nu && pv[u] <= idx[u]) ? step : 0;
    }
  }

  // Entries [first, total) of the lists.
  template <typename Fn>
  __device__ __forceinline__ void for_each_from(uint32_t first, Fn&& fn) const {
    const uint32_t l = lo;
    const uint32_t total = pre[nu];
    for (uint32_t base = first; base < total; base += blockDim.x * kBatch) {
      uint32_t idx[kBatch];
      int a[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) idx[u] = base + u * blockDim.x + threadIdx.x;
      locate(idx, a);
      uint64_t v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        v[u] = idx[u] < total ? list[size_t(u_lo + a[u]) * kUnit + (idx[u] - pre[a[u]])] : 0ull;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const uint32_t n = uint32_t(v[u]);
        fn((uint64_t(uint32_t(v[u] >> 32) - l) << 32) | uint32_t(~n), int(n), idx[u] < total);
      }
    }
  }

  template <typename Fn>
  __device__ __forceinline__ void for_each(Fn&& fn) const {
    for_each_from(0u, fn);
  }
};

// The same lists with their first NR * blockDim entries read once into
// registers (entry r * blockDim + t in slot r of thread t); entries past
// those are streamed from global memory on every pass.
template <int NR>
struct RegLists {
  uint64_t c[NR];
  uint32_t total;  // entries held in registers
  UnitLists rest;

  // start: LDS scratch of NR * blockDim / 64 entries. Entry q gets the unit
  // of list entry 64 q (one search per thread); the lanes of a wave, which
  // hold 64 consecutive entries, then step forward from their first unit.
  __device__ __forceinline__ void load(const UnitLists& src, uint16_t* start) {
    rest = src;
    total = min(src.pre[src.nu], uint32_t(NR) * blockDim.x);
    const uint32_t l = src.lo;
    const uint32_t nq = (total + 63u) / 64u;
    for (uint32_t q = threadIdx.x; q < nq; q += blockDim.x) {
      uint32_t idx[kBatch];
      int a[kBatch];
      idx[0] = q * 64u;
#pragma unroll
      for (int u = 1; u < kBatch; ++u) idx[u] = idx[0];
      src.locate(idx, a);
      start[q] = uint16_t(a[0]);
    }
    __syncthreads();
    const int wave = threadIdx.x >> 6;
    const int waves = blockDim.x >> 6;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      if (uint32_t(r) * blockDim.x >= total) break;  // uniform
      const uint32_t i = r * blockDim.x + threadIdx.x;
      uint64_t v = 0ull;
      if (i < total) {
        int a = start[r * waves + wave];
        while (a + 1 < src.nu && src.pre[a + 1] <= i) ++a;
        v = src.list[size_t(src.u_lo + a) * kUnit + (i - src.pre[a])];
      }
      c[r] = v;
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const uint32_t n = uint32_t(c[r]);
      c[r] = (uint64_t(uint32_t(c[r] >> 32) - l) << 32) | uint32_t(~n);
    }
  }

  template <typename Fn>
  __device__ __forceinline__ void for_each(Fn&& fn) const {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      if (uint32_t(r) * blockDim.x >= total) break;  // uniform
      const uint32_t i = r * blockDim.x + threadIdx.x;
      fn(c[r], int(~uint32_t(c[r])), i < total);
    }
    rest.for_each_from(uint32_t(NR) * blockDim.x, fn);
  }
};

// Keys of a head's sampled positions in global memory; 0 marks a position
// outside M (and is skipped).
struct SampleKeys {
  const uint32_t* keys;
  uint32_t count;
  template <typename Fn>
  __device__ __forceinline__ void for_each(Fn&& fn) const {
    for (uint32_t base = 0; base < count; base += blockDim.x * kBatch) {
      uint32_t v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const uint32_t i = base + u * blockDim.x + threadIdx.x;
        v[u] = i < count ? keys[i] : 0u;
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) fn(uint64_t(v[u]), 0, v[u] != 0u);
    }
  }
};

// The same keys read once into registers.
template <int NR>
struct RegKeys {
  uint32_t k[NR];
  uint32_t count;
  __device__ __forceinline__ void load(const uint32_t* keys, uint32_t n) {
    count = n;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const uint32_t i = r * blockDim.x + threadIdx.x;
      k[r] = i < count ? keys[i] : 0u;
    }
  }
  template <typename Fn>
  __device__ __forceinline__ void for_each(Fn&& fn) const {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      if (uint32_t(r) * blockDim.x >= count) break;  // uniform
      fn(uint64_t(k[r]), 0, k[r] != 0u);
    }
  }
};

// Composites already reduced to one sub-bucket, in LDS.
struct LdsSource {
  const uint64_t* c;
  uint32_t count;
  template <typename Fn>
  __device__ __forceinline__ void for_each(Fn&& fn) const {
    for (uint32_t base = 0; base < count; base += blockDim.x) {
      const uint32_t i = base + threadIdx.x;
      const uint64_t v = i < count ? c[i] : 0ull;
      fn(v, int(~uint32_t(v)), i < count);
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
__device__ __forceinline__ uint32_t radix_pass(const Src& src, const Radix& rx, int TB, uint32_t& need,
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
  src.for_each([&](uint64_t c, int, bool valid) {
    if (valid && (pl == 0 || (c >> (TB - pl)) == pf))
      atomicAdd(&rx.hist[uint32_t(c >> shift) & dmask], 1u);
  });
  __syncthreads();
  if (wave == 0) {
    // lane l sums bins 32 l .. 32 l + 31; the lane where the count from the
    // top reaches need owns the digit, found among its 32 bins in parallel
    uint32_t s = 0;
    for (int i = 0; i < 32; ++i) s += rx.hist[lane * 32 + i];
    const uint32_t suf = wave_suffix_sum(s);
    const uint64_t m = __ballot(suf >= need);
    const int L = m ? 63 - __clzll(m) : 0;
    const uint32_t above_l = __shfl(suf - s, L);
    const uint32_t v = lane < 32 ? rx.hist[L * 32 + lane] : 0u;
    const uint32_t fsuf = wave_suffix_sum(v) + above_l;
    const uint64_t mf = __ballot(lane < 32 && fsuf >= need);
    const int F = mf ? 63 - __clzll(mf) : 0;
    if (lane == F) {
      *rx.s_d = uint32_t(L * 32 + F);
      *rx.s_above = fsuf - v;
      *rx.s_cnt = v;
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
__device__ __forceinline__ void radix_finish(const Src& src, const Radix& rx, int TB, uint32_t& need,
                             uint64_t& prefix, int& plen) {
  while (plen < TB) {
    if (radix_pass(src, rx, TB, need, prefix, plen) == need) break;
  }
}

// The need-th largest of n <= blockDim values in LDS, ties allowed: the
// value v with #(x > v) < need <= #(x >= v), found by letting each entry
// count the entries above it (one broadcast pass over LDS instead of
// several radix passes, for the small buckets left after the first pass).
__device__ __forceinline__ uint64_t rank_select(const uint64_t* sub, uint32_t n, uint32_t need) {
  __shared__ uint64_t s_val;
  const uint32_t t = threadIdx.x;
  if (t < n) {
    const uint64_t c = sub[t];
    uint32_t gt = 0, eq = 0;
#pragma unroll 8
    for (uint32_t j = 0; j < n; ++j) {
      const uint64_t x = sub[j];
      gt += x > c ? 1u : 0u;
      eq += x == c ? 1u : 0u;
    }
    if (gt < need && gt + eq >= need) s_val = c;
  }
  __syncthreads();
  const uint64_t v = s_val;
  __syncthreads();
  return v;
}

// Composite prefix (top plen of TB bits) of the need-th largest member of a
// source: one pass over it; if that does not settle it and the chosen
// sub-bucket fits LDS, the sub-bucket is copied there and finished in LDS
// (by ranking when it is small, else by more radix passes).
// Members whose top plen bits are >= the returned prefix are exactly the
// need largest (all of them when every bit is fixed and values tie).
template <typename Src>
__device__ __forceinline__ void find_threshold(const Src& src, const Radix& rx, int TB, uint32_t need,
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
  src.for_each([&](uint64_t c, int, bool valid) {
    wave_append(sub, s_n, kSubCap, c, valid && (c >> (TB - pl)) == pf);
  });
  __syncthreads();
  const uint32_t n = *s_n;
  if (n <= kRankMax) {
    prefix = rank_select(sub, n, need);
    plen = TB;
    return;
  }
  const LdsSource lds{sub, n};
  radix_finish(lds, rx, TB, need, prefix, plen);
}

// ---------------------------------------------------------------- threshold
__device__ __forceinline__ int bit_length(uint32_t x) { return 32 - __clz(x); }

// One block per head. Also resets the per-call state the later stages
// accumulate into (head state, group flags, the rescan counter) and writes
// the unit prefix the scan distributes its work by.
__global__ __launch_bounds__(kSelThreads) void threshold_kernel(Params p) {
  const int bh = blockIdx.x;
  const int b = bh / p.H_q;
  const int hq = bh - b * p.H_q;
  const int tid = threadIdx.x;
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t s_d, s_above, s_cnt;
  __shared__ int64_t tmp[16];

  if (bh == 0) {
    // unit prefix over the batch
    const int per = (p.B + kSelThreads - 1) / kSelThreads;
    int64_t sum = 0;
    for (int i = 0; i < per; ++i) {
      const int bb = tid * per + i;
      if (bb < p.B) {
        const int P = (seq_geom(p, bb).N + kPage - 1) / kPage;
        sum += int64_t(p.H_kv) * ((P + kUnitPages - 1) / kUnitPages);
      }
    }
    int64_t total;
    int64_t run = block_excl_scan(sum, tmp, &total);
    for (int i = 0; i < per; ++i) {
      const int bb = tid * per + i;
      if (bb < p.B) {
        const int P = (seq_geom(p, bb).N + kPage - 1) / kPage;
        p.unit_off[bb] = run;
        run += int64_t(p.H_kv) * ((P + kUnitPages - 1) / kUnitPages);
      }
    }
    if (tid == 0) {
      p.unit_off[p.B] = total;
      *p.any_dense = 0u;
    }
  }
  if (tid == 0 && hq % p.G == 0) p.gflag[size_t(b) * p.H_kv + hq / p.G] = 0u;

  const SeqGeom sg = seq_geom(p, b);
  uint32_t lo = 0xFFFFFFFFu;  // k_eff == 0: no candidates
  if (sg.k_eff > 0) {
    const int P = (sg.N + kPage - 1) / kPage;
    const int ns = sampled_pages(P);
    const int S = 1 << sample_log2(P);
    const uint32_t* keys = p.samp + size_t(bh) * p.samp_cap;
    const uint32_t count = uint32_t(ns * kPage);
    RegKeys<kRegKeys> rk;
    const bool in_regs = count <= uint32_t(kRegKeys * kSelThreads);
    if (in_regs) rk.load(keys, count);  // in flight while the count below runs
    // sampled members of M: overlap of every sampled page with [lo, hi)
    int64_t c = 0;
    for (int t = tid; t < ns; t += kSelThreads) {
      const int j = (S >> 1) + t * S;
      const int a = max(j * kPage, sg.lo), e = min(j * kPage + kPage, sg.hi);
      c += e > a ? e - a : 0;
    }
    int64_t m_s;
    block_excl_scan(c, tmp, &m_s);
    const int64_t m_all = sg.hi - sg.lo;
    uint32_t R;
    if (m_s >= m_all) {
      R = uint32_t(sg.k_eff);  // the sample is all of M: exact
    } else {
      const float kr = float(sg.k_eff) * float(m_s) / float(m_all);
      R = uint32_t(ceilf(1.05f * kr + 5.0f * sqrtf(kr) + 8.0f));
    }
    if (m_s == 0 || int64_t(R) >= m_s) {
      lo = 0u;  // keep every member of M
    } else {
      // the bound need not be exact, only at or below the R-th largest
      // sampled key: two radix passes fix its top 22 bits
      const Radix rx{hist, &s_d, &s_above, &s_cnt};
      uint64_t prefix = 0;
      int plen = 0;
      uint32_t need = R;
      if (in_regs) {
        radix_pass(rk, rx, 32, need, prefix, plen);
        radix_pass(rk, rx, 32, need, prefix, plen);
      } else {
        const SampleKeys sk{keys, count};
        radix_pass(sk, rx, 32, need, prefix, plen);
        radix_pass(sk, rx, 32, need, prefix, plen);
      }
      lo = uint32_t(prefix << (32 - plen));
    }
  }
  if (tid == 0) {
    HeadState st;
    st.lo_key = lo;
    st.max_w = 0u;
    st.max_m = 0u;
    st.dense = 0u;
    st.thr_shift = 64u;  // nothing passes until select decides
    st.thr_lo = 0xFFFFFFFFu;
    st.thr_hi = 0xFFFFFFFFu;
    st.pad = 0u;
    p.state[bh] = st;
  }
}

hipError_t launch_threshold(const Params& p, hipStream_t s) {
  hipLaunchKernelGGL(threshold_kernel, dim3(unsigned(p.B * p.H_q)), dim3(kSelThreads), 0, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------- select
struct SelLds {
  uint16_t start[kRegEntries * kSelThreads / 64];  // unit of every 64th entry
  uint32_t pre[kMaxUnits + 1];  // prefix of the list lengths
  uint32_t hist[2048];
  uint64_t sub[kSubCap];
  uint32_t s_d, s_above, s_cnt, s_n;
  int64_t tmp[16];
};

// Prefix of the list lengths of units u_lo .. u_lo + nu - 1 into L.pre;
// returns the total. Block-wide.
__device__ uint32_t unit_prefix(const Params& p, int bh, const SeqGeom& sg, int u_lo, int nu,
                                bool dense, SelLds& L) {
  constexpr int per = kMaxUnits / kSelThreads;
  const int tid = threadIdx.x;
  const uint32_t* uc = p.ucnt + size_t(bh) * p.n_units;
  uint32_t c[per];
  int64_t sum = 0;
#pragma unroll
  for (int u = 0; u < per; ++u) {
    const int i = tid * per + u;
    c[u] = 0u;
    if (i < nu) {
      if (dense) {
        const int v = u_lo + i;
        c[u] = uint32_t(min((v + 1) * kUnit, sg.hi) - max(v * kUnit, sg.lo));
      } else {
        c[u] = uc[u_lo + i];
      }
    }
    sum += c[u];
  }
  int64_t total;
  int64_t run = block_excl_scan(sum, L.tmp, &total);
#pragma unroll
  for (int u = 0; u < per; ++u) {
    L.pre[tid * per + u] = uint32_t(run);
    run += c[u];
  }
  if (tid == 0) L.pre[kMaxUnits] = uint32_t(total);
  __syncthreads();
  return uint32_t(total);
}

// Exact threshold of head bh over its candidates (source src), written
// into the head state.
template <typename Src>
__device__ __forceinline__ void decide(const Params& p, int bh, const SeqGeom& sg, const Src& src,
                                       int TB, uint32_t lo, SelLds& L) {
  const Radix rx{L.hist, &L.s_d, &L.s_above, &L.s_cnt};
  uint64_t prefix;
  int plen;
  find_threshold(src, rx, TB, uint32_t(sg.k_eff), L.sub, &L.s_n, prefix, plen);
  if (threadIdx.x == 0) {
    HeadState& w = p.state[bh];
    w.lo_key = lo;
    w.thr_shift = uint32_t(TB - plen);
    w.thr_lo = uint32_t(prefix);
    w.thr_hi = uint32_t(prefix >> 32);
  }
}

// Select over the lists of head bh (whose prefix is in L.pre), from
// registers when they fit.
__device__ __forceinline__ void select_head(const Params& p, int bh, const SeqGeom& sg, int u_lo, int nu,
                            uint32_t lo, uint32_t max_m, SelLds& L) {
  const uint32_t span = max_m > lo ? max_m - lo : 1u;
  const int TB = 32 + bit_length(span);
  const UnitLists gl{p.cand + size_t(bh) * p.n_cap, L.pre, u_lo, nu, lo};
  RegLists<kRegEntries> rl;
  rl.load(gl, L.start);
  decide(p, bh, sg, rl, TB, lo, L);
}

// One block per head: count the candidates; decide the threshold, or flag
// the head (and its group) for the rescan when there are fewer than k_eff.
__global__ __launch_bounds__(kSelThreads) void select_kernel(Params p) {
  const int bh = blockIdx.x;
  const int b = bh / p.H_q;
  const int g = (bh - b * p.H_q) / p.G;
  const SeqGeom sg = seq_geom(p, b);
  if (sg.k_eff == 0) return;  // the unset threshold takes nothing
  __shared__ SelLds L;
  const int u_lo = sg.lo / kUnit, nu = (sg.hi - 1) / kUnit + 1 - u_lo;
  const uint32_t m = unit_prefix(p, bh, sg, u_lo, nu, false, L);
  const HeadState st = p.state[bh];
  if (m < uint32_t(sg.k_eff)) {
    if (threadIdx.x == 0) {
      p.state[bh].dense = 1u;
      atomicOr(&p.gflag[size_t(b) * p.H_kv + g], 1u);
      atomicAdd(p.any_dense, 1u);
    }
    return;
  }
  select_head(p, bh, sg, u_lo, nu, st.lo_key, st.max_m, L);
}

hipError_t launch_select(const Params& p, hipStream_t s) {
  hipLaunchKernelGGL(select_kernel, dim3(unsigned(p.B * p.H_q)), dim3(kSelThreads), 0, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------- dense
// After the rescan: the flagged heads select over every member of M (their
// lists now hold all of it, so the list lengths are the units' overlaps).
__global__ __launch_bounds__(kSelThreads) void reselect_kernel(Params p) {
  if (*p.any_dense == 0u) return;
  const int bh = blockIdx.x;
  const HeadState st = p.state[bh];
  if (!st.dense) return;
  const SeqGeom sg = seq_geom(p, bh / p.H_q);
  __shared__ SelLds L;
  const int u_lo = sg.lo / kUnit, nu = (sg.hi - 1) / kUnit + 1 - u_lo;
  unit_prefix(p, bh, sg, u_lo, nu, true, L);
  uint32_t* uc = p.ucnt + size_t(bh) * p.n_units;
  for (int i = threadIdx.x; i < nu; i += kSelThreads) uc[u_lo + i] = L.pre[i + 1] - L.pre[i];
  select_head(p, bh, sg, u_lo, nu, 0u, st.max_m, L);
}

hipError_t launch_dense_scan(const Params& p, hipStream_t s);  // score_scan.hip

hipError_t launch_dense(const Params& p, hipStream_t s) {
  hipError_t e = launch_dense_scan(p, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(reselect_kernel, dim3(unsigned(p.B * p.H_q)), dim3(kSelThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace ra
