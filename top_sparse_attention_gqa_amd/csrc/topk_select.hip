// Exact top-k over the selection domain M = [lo, hi) of each query head,
// ties to the lower position: the fixed retrieval budget of the
// RetrievalAttention slides ("Sparse attention renormalizes selected tokens",
// and "The GPU keeps 640 fixed positions": W excluded, per-head indices).
//
// Scores are compared through an order-preserving uint32 key, and the
// choice among members is made on the composite  c = key' << 32 | ~n
// (key' = key relative to a known lower bound): a larger composite is a
// larger score, then a lower position, and all composites are distinct, so
// "the need largest composites" is the unique tie-broken top-k.
//
// select (common path, one block per head): the scan left every member of M
// scoring at or above the head's sampled threshold in a candidate list. If
// the list holds at least k_eff entries and did not overflow, the top-k of M
// is the top-k of the list; a radix select on the composite finds it (the
// bucket around the k-th entry is finished in LDS). The block writes the
// head's selection bitmap, per-tile counts and the selected scores.
// Otherwise the head is flagged for the dense path:
//  dense scan   - every score stored, exact histogram of M;
//  dense filter - threshold bucket from the histogram; keys above it go
//                 straight into the bitmap, keys inside it to a list;
//  dense resolve- the same radix select inside the bucket (or over the row
//                 if the bucket overflowed the list).
#include "ra_internal.h"

namespace ra {

constexpr int kFiltThreads = 256;  // 4 waves x 2048 positions = one tile
constexpr int kFiltIters = kTile / kFiltThreads;  // 32 positions per lane
constexpr int kSelThreads = 1024;
constexpr int kSubCap = 4096;              // LDS list for one radix sub-bucket
constexpr int kMaxTiles = RA_MAX_SEQ_LEN / kTile;

// ---------------------------------------------------------------- sources
// Each source enumerates composites of members with (c, n).

// Sparse candidate list: c = (key - lo) << 32 | ~n.
struct CandSource {
  const uint64_t* c;
  uint32_t count;
  uint32_t lo;
  template <typename Fn>
  __device__ __forceinline__ void for_each(Fn&& fn) const {
    for (uint32_t i = threadIdx.x; i < count; i += blockDim.x) {
      const uint64_t v = c[i];
      const uint32_t notn = uint32_t(v);
      fn((uint64_t(uint32_t(v >> 32) - lo) << 32) | notn, int(~notn));
    }
  }
};

// Dense-path bucket list: c = (key & low_mask) << 32 | ~n.
struct BucketList {
  const uint64_t* c;
  uint32_t count;
  uint64_t low_mask;
  template <typename Fn>
  __device__ __forceinline__ void for_each(Fn&& fn) const {
    for (uint32_t i = threadIdx.x; i < count; i += blockDim.x) {
      const uint64_t v = c[i];
      const uint32_t notn = uint32_t(v);
      fn((uint64_t(uint32_t(v >> 32)) & low_mask) << 32 | notn, int(~notn));
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

// A head's whole score row filtered to one bucket (dense path, when the
// bucket overflowed its list).
struct RowSource {
  const float* row;
  int lo, hi;
  uint32_t b1;
  int shift;
  uint64_t low_mask;
  template <typename Fn>
  __device__ __forceinline__ void for_each(Fn&& fn) const {
    for (int n = lo + int(threadIdx.x); n < hi; n += int(blockDim.x)) {
      const uint32_t key = f2key(row[n]);
      if ((key >> shift) != b1) continue;
      fn((uint64_t(key) & low_mask) << 32 | uint32_t(~uint32_t(n)), n);
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

// Take every composite whose top plen bits are >= prefix.
template <typename Src, typename Take>
__device__ void take_from(const Src& src, int TB, uint64_t prefix, int plen, Take&& take) {
  src.for_each([&](uint64_t c, int n) {
    if ((c >> (TB - plen)) >= prefix) take(c, n);
  });
}

// The need largest composites of a source: one pass over it; if that does not
// settle it and the chosen sub-bucket fits LDS, members above it are taken
// at once and the sub-bucket is finished in LDS.
template <typename Src, typename Take>
__device__ void select_top(const Src& src, const Radix& rx, int TB, uint32_t need,
                           uint64_t* sub, uint32_t* s_n, Take&& take) {
  uint64_t prefix = 0;
  int plen = 0;
  const uint32_t cnt1 = radix_pass(src, rx, TB, need, prefix, plen);
  if (cnt1 == need || plen >= TB) {
    take_from(src, TB, prefix, plen, take);
    return;
  }
  if (cnt1 > uint32_t(kSubCap)) {
    radix_finish(src, rx, TB, need, prefix, plen);
    take_from(src, TB, prefix, plen, take);
    return;
  }
  if (threadIdx.x == 0) *s_n = 0;
  __syncthreads();
  const uint64_t pf = prefix;
  const int pl = plen;
  src.for_each([&](uint64_t c, int n) {
    const uint64_t top = c >> (TB - pl);
    if (top > pf) {
      take(c, n);
    } else if (top == pf) {
      sub[atomicAdd(s_n, 1u)] = c;
    }
  });
  __syncthreads();
  const LdsSource lds{sub, *s_n};
  radix_finish(lds, rx, TB, need, prefix, plen);
  take_from(lds, TB, prefix, plen, take);
}

// ---------------------------------------------------------------- select
__global__ __launch_bounds__(kSelThreads) void select_kernel(Params p) {
  const int bh = blockIdx.x;
  const int b = bh / p.H_q;
  const int g = (bh - b * p.H_q) / p.G;
  const SeqGeom sg = seq_geom(p, b);
  const int nt = (sg.N + kTile - 1) / kTile;
  const int tid = threadIdx.x;

  __shared__ uint32_t hist[2048];
  __shared__ uint32_t s_d, s_above, s_cnt, s_n;
  __shared__ uint64_t sub[kSubCap];
  __shared__ uint32_t tcnt[kMaxTiles];

  const HeadState st = p.state[bh];
  const uint32_t m = st.cand_count;
  if (sg.k_eff > 0 && (m < uint32_t(sg.k_eff) || m > uint32_t(p.cap))) {
    // the sample's margin did not hold: decide this head on the dense path
    if (tid == 0) {
      p.state[bh].dense = 1u;
      atomicOr(&p.gflag[size_t(b) * p.H_kv + g], 1u);
    }
    return;
  }

  uint64_t* bm = p.bitmap + size_t(bh) * (p.n_cap / 64);
  for (int i = tid; i < nt * kWordsPerTile; i += kSelThreads) bm[i] = 0ull;
  for (int i = tid; i < nt; i += kSelThreads) tcnt[i] = 0u;
  __syncthreads();

  if (sg.k_eff > 0) {
    const uint32_t lo = st.lo_key;
    const uint32_t span = st.max_m > lo ? st.max_m - lo : 1u;
    const int TB = 32 + (32 - __clz(span));
    const CandSource src{p.cand + size_t(bh) * p.cap, m, lo};
    const Radix rx{hist, &s_d, &s_above, &s_cnt};
    float* srow = p.scores + size_t(bh) * p.n_cap;
    select_top(src, rx, TB, uint32_t(sg.k_eff), sub, &s_n, [&](uint64_t c, int n) {
      atomicOr(reinterpret_cast<unsigned long long*>(&bm[n >> 6]), 1ull << (n & 63));
      atomicAdd(&tcnt[n / kTile], 1u);
      srow[n] = key2f(uint32_t(c >> 32) + lo);
    });
  }
  __syncthreads();
  for (int i = tid; i < nt; i += kSelThreads) p.tile_cnt[size_t(bh) * p.n_tiles + i] = tcnt[i];
}

hipError_t launch_select(const Params& p, hipStream_t s) {
  hipLaunchKernelGGL(select_kernel, dim3(unsigned(p.B * p.H_q)), dim3(kSelThreads), 0, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------- dense
__global__ __launch_bounds__(kFiltThreads) void dense_filter_kernel(Params p) {
  const int tile = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / p.H_q;
  const SeqGeom sg = seq_geom(p, b);
  const int t0 = tile * kTile;
  if (t0 >= sg.N || !p.state[bh].dense) return;

  const int HB = hist_bits(p.G);
  const int SHIFT = 32 - HB;
  const int NC = 1 << (HB - 6);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  __shared__ uint32_t s_b1, s_mode, s_cbase;
  __shared__ uint32_t s_cnt[kFiltThreads / 64], s_cc[kFiltThreads / 64];

  // issue every score load of this lane before anything waits
  const float* row = p.scores + size_t(bh) * p.n_cap;
  const int wbase = t0 + wave * (kTile / 4);
  float z[kFiltIters];
#pragma unroll
  for (int it = 0; it < kFiltIters; ++it) z[it] = row[wbase + it * 64 + lane];

  if (wave == 0) {
    uint32_t b1 = 0xFFFFFFFFu, mode = 0, above = 0, need = 0;
    if (sg.k_eff > 0) {
      const uint32_t* gh = p.dhist + size_t(bh) * kHistStride;
      const uint32_t k = uint32_t(sg.k_eff);
      // coarse bucket holding the k-th largest (from the top)
      const uint32_t c = lane < NC ? gh[kFineBins + lane] : 0u;
      const uint32_t suf = wave_suffix_sum(c);
      const uint64_t mc = __ballot(suf >= k);
      const int cs = mc ? 63 - __clzll(mc) : 0;
      const uint32_t above_c = __shfl(suf - c, cs);
      // fine bucket inside it
      const uint32_t f = gh[cs * 64 + lane];
      const uint32_t fsuf = wave_suffix_sum(f) + above_c;
      const uint64_t mf = __ballot(fsuf >= k);
      const int fl = mf ? 63 - __clzll(mf) : 0;
      b1 = uint32_t(cs * 64 + fl);
      above = __shfl(fsuf - f, fl);
      const uint32_t cnt = __shfl(f, fl);
      need = k - above;
      mode = cnt <= uint32_t(p.dcap) ? kModeCand : kModeRescan;
    }
    if (lane == 0) {
      s_b1 = b1;
      s_mode = mode;
      if (tile == 0) {
        HeadState& st = p.state[bh];
        st.b1 = b1;
        st.above1 = above;
        st.need1 = need;
        st.mode = mode;
      }
    }
  }
  __syncthreads();
  const uint32_t b1 = s_b1;
  const bool cand_mode = s_mode == kModeCand;

  // above-bucket members become bitmap words (lane it keeps word it)
  uint64_t myword = 0;
  uint32_t cnt = 0, ccnt = 0;
#pragma unroll
  for (int it = 0; it < kFiltIters; ++it) {
    const int n = wbase + it * 64 + lane;
    const bool valid = n >= sg.lo && n < sg.hi;
    const uint32_t dg = f2key(z[it]) >> SHIFT;
    const uint64_t m = __ballot(valid && dg > b1);
    if (lane == it) myword = m;
    cnt += uint32_t(__popcll(m));
    ccnt += uint32_t(__popcll(__ballot(cand_mode && valid && dg == b1)));
  }
  if (lane < kFiltIters) p.bitmap[size_t(bh) * (p.n_cap / 64) + (wbase >> 6) + lane] = myword;
  if (lane == 0) {
    s_cnt[wave] = cnt;
    s_cc[wave] = ccnt;
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t t = 0, c = 0;
    for (int w = 0; w < kFiltThreads / 64; ++w) {
      t += s_cnt[w];
      c += s_cc[w];
    }
    p.tile_cnt[size_t(bh) * p.n_tiles + tile] = t;
    // one reservation per block in the head's bucket list
    s_cbase = c ? atomicAdd(&p.state[bh].dcand_count, c) : 0u;
  }
  __syncthreads();
  if (cand_mode && ccnt) {
    uint32_t base = s_cbase;
    for (int w = 0; w < wave; ++w) base += s_cc[w];
    uint64_t* cl = p.dcand + size_t(bh) * p.dcap;
#pragma unroll
    for (int it = 0; it < kFiltIters; ++it) {
      const int n = wbase + it * 64 + lane;
      const bool valid = n >= sg.lo && n < sg.hi;
      const uint32_t key = f2key(z[it]);
      const bool cd = valid && (key >> SHIFT) == b1;
      const uint64_t cm = __ballot(cd);
      if (cd) {
        const uint32_t idx = base + uint32_t(__popcll(cm & ((1ull << lane) - 1ull)));
        if (idx < uint32_t(p.dcap)) cl[idx] = (uint64_t(key) << 32) | uint32_t(~uint32_t(n));
      }
      base += uint32_t(__popcll(cm));
    }
  }
}

__global__ __launch_bounds__(kSelThreads) void dense_resolve_kernel(Params p) {
  const int bh = blockIdx.x;
  const int b = bh / p.H_q;
  const SeqGeom sg = seq_geom(p, b);
  if (sg.k_eff == 0) return;
  const HeadState st = p.state[bh];
  if (!st.dense || st.mode == 0) return;

  const int HB = hist_bits(p.G);
  const int TB = 64 - HB;
  const uint64_t low_mask = (1ull << (32 - HB)) - 1ull;

  __shared__ uint32_t hist[2048];
  __shared__ uint32_t s_d, s_above, s_cnt, s_n;
  __shared__ uint64_t sub[kSubCap];
  const Radix rx{hist, &s_d, &s_above, &s_cnt};
  uint64_t* bm = p.bitmap + size_t(bh) * (p.n_cap / 64);
  auto take = [&](uint64_t, int n) {
    atomicOr(reinterpret_cast<unsigned long long*>(&bm[n >> 6]), 1ull << (n & 63));
    atomicAdd(&p.tile_cnt[size_t(bh) * p.n_tiles + n / kTile], 1u);
  };
  if (st.mode == kModeRescan) {
    const RowSource src{p.scores + size_t(bh) * p.n_cap, sg.lo, sg.hi, st.b1, 32 - HB, low_mask};
    uint32_t need = st.need1;
    uint64_t prefix = 0;
    int plen = 0;
    radix_finish(src, rx, TB, need, prefix, plen);
    take_from(src, TB, prefix, plen, take);
    return;
  }
  const BucketList src{p.dcand + size_t(bh) * p.dcap, min(st.dcand_count, uint32_t(p.dcap)), low_mask};
  select_top(src, rx, TB, st.need1, sub, &s_n, take);
}

hipError_t launch_dense_scan(const Params& p, hipStream_t s);  // score_scan.hip

hipError_t launch_dense(const Params& p, hipStream_t s) {
  hipError_t e = launch_dense_scan(p, s);
  if (e != hipSuccess) return e;
  const unsigned tiles = unsigned((int64_t(p.max_seq_len) + kTile - 1) / kTile);
  hipLaunchKernelGGL(dense_filter_kernel, dim3(tiles, unsigned(p.B * p.H_q)),
                     dim3(kFiltThreads), 0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dense_resolve_kernel, dim3(unsigned(p.B * p.H_q)), dim3(kSelThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace ra
