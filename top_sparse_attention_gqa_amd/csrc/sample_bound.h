// The candidate bound of a head, from the keys of its sampled positions:
// a key at or just below the R-th largest sampled member of M (its top 22
// bits), R a conservative stand-in for the rank of the k_eff-th largest
// member of M in the sample (RetrievalAttention slides, "The GPU keeps 640
// fixed positions": a fixed budget per query head). Members at or above it
// are the head's candidates; the selection checks that at least k_eff of
// them exist, so the bound only has to be good, not exact.
//
// The bound is a deterministic function of the sampled keys, so any block
// may compute it and every block gets the same value. It is published in
// the head state as one 64-bit word (bound | 1 << 32), with no other field
// in that word, so a reader needs no fence: an agent-scope atomic load sees
// either "not yet" or the bound.
#pragma once

#include "ra_internal.h"

namespace ra {

constexpr int kBatch = 8;     // global entries per lane in flight per pass
constexpr int kRegKeys = 32;  // sampled keys per lane kept in registers

// Which sampled positions are members of M: slot i of a head's sample row
// holds position (S / 2 + (i / 64) * S) * 64 + i % 64 (the row also keeps
// the keys of W, which the scan uses).
struct SampledM {
  int sh, lo, hi;  // S = 1 << sh; M = [lo, hi)
  __device__ __forceinline__ bool has(uint32_t i) const {
    const int pos = (((1 << sh) >> 1) + int(i >> 6) * (1 << sh)) * kPage + int(i & 63u);
    return pos >= lo && pos < hi;
  }
};

// Keys of a head's sampled positions in global memory.
struct SampleKeys {
  const uint32_t* keys;
  uint32_t count;
  SampledM m;
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
      for (int u = 0; u < kBatch; ++u) {
        const uint32_t i = base + u * blockDim.x + threadIdx.x;
        fn(uint64_t(v[u]), 0, i < count && m.has(i));
      }
    }
  }
};

// The same keys read once into registers.
template <int NR>
struct RegKeys {
  uint32_t k[NR];
  uint32_t count;
  SampledM m;
  __device__ __forceinline__ void load(const uint32_t* keys, uint32_t n, SampledM mm) {
    count = n;
    m = mm;
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
      const uint32_t i = r * blockDim.x + threadIdx.x;
      fn(uint64_t(k[r]), 0, i < count && m.has(i));
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
    // lane l sums bins 32 l .. 32 l + 31 (starting at a lane-dependent bin,
    // so that the lanes read different LDS banks); the lane where the count
    // from the top reaches need owns the digit, found among its 32 bins in
    // parallel
    uint32_t s = 0;
    for (int i = 0; i < 32; ++i) s += rx.hist[lane * 32 + ((i + lane) & 31)];
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

// The bound of head bh, returned to every thread. Every thread of the block
// calls it; it uses rx and tmp (16 int64) of LDS.
__device__ __forceinline__ uint32_t head_bound(const Params& p, int bh, const Radix& rx,
                                               int64_t* tmp) {
  const int tid = threadIdx.x;
  const int b = bh / p.H_q;
  const SeqGeom sg = seq_geom(p, b);
  if (sg.k_eff <= 0) return 0xFFFFFFFFu;  // no candidates
  const int P = (sg.N + kPage - 1) / kPage;
  const int ns = sampled_pages(P);
  const int S = 1 << sample_log2(P);
  const uint32_t* keys = p.samp + size_t(bh) * p.samp_cap;
  const uint32_t count = uint32_t(ns * kPage);
  const SampledM sm{sample_log2(P), sg.lo, sg.hi};
  RegKeys<kRegKeys> rk;
  const bool in_regs = count <= uint32_t(kRegKeys) * blockDim.x;
  if (in_regs) rk.load(keys, count, sm);  // in flight while the count below runs
  // sampled members of M: overlap of every sampled page with [lo, hi)
  int64_t c = 0;
  for (int t = tid; t < ns; t += blockDim.x) {
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
  if (m_s == 0 || int64_t(R) >= m_s) return 0u;  // keep every member of M
  // the bound need not be exact, only at or below the R-th largest sampled
  // key: two radix passes fix its top 22 bits
  uint64_t prefix = 0;
  int plen = 0;
  uint32_t need = R;
  if (in_regs) {
    radix_pass(rk, rx, 32, need, prefix, plen);
    radix_pass(rk, rx, 32, need, prefix, plen);
  } else {
    const SampleKeys sk{keys, count, sm};
    radix_pass(sk, rx, 32, need, prefix, plen);
    radix_pass(sk, rx, 32, need, prefix, plen);
  }
  return uint32_t(prefix << (32 - plen));
}

__device__ __forceinline__ uint64_t* bound_slot(const Params& p, size_t bh) {
  return reinterpret_cast<uint64_t*>(&p.state[bh].lo_key);
}

// One thread.
__device__ __forceinline__ void publish_bound(const Params& p, size_t bh, uint32_t lo) {
  __hip_atomic_store(bound_slot(p, bh), (uint64_t(1) << 32) | lo, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// One thread: true and *lo = the bound once it is published.
__device__ __forceinline__ bool read_bound(const Params& p, size_t bh, uint32_t* lo) {
  const uint64_t v = __hip_atomic_load(bound_slot(p, bh), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  *lo = uint32_t(v);
  return (v >> 32) != 0u;
}

}  // namespace ra
