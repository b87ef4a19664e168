// Exact top-k over the selection domain M = [lo, hi) of each query head's
// score row, ties to the lower position: the fixed retrieval budget of the
// RetrievalAttention slides ("Sparse attention renormalizes selected tokens",
// and "The GPU keeps 640 fixed positions": W excluded, per-head indices).
//
// Scores are compared through an order-preserving uint32 key. The scan left a
// per-head histogram of the key's top 12 (or 11) bits over M. From it:
//  filter  - every tile block finds the bucket b1 holding the k_eff-th largest
//            key; keys above b1 are selected outright (written as a bitmap of
//            M, plus a per-tile count); keys in b1 are appended to a small
//            per-head candidate list when the bucket fits it.
//  resolve - one block per head picks exactly `need` members of bucket b1 by
//            a radix select on the composite (low key bits, ~position): larger
//            score first, then lower position, so the choice is unique. If the
//            bucket did not fit the list, the block re-reads the head's row.
#include "ra_internal.h"

namespace ra {

constexpr int kFiltThreads = 256;  // 4 waves x 2048 positions = one tile
constexpr int kResThreads = 1024;

__global__ __launch_bounds__(kFiltThreads) void filter_kernel(Params p) {
  const int tile = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / p.H_q;
  const SeqGeom sg = seq_geom(p, b);
  const int t0 = tile * kTile;
  if (t0 >= sg.N) return;

  const int HB = hist_bits(p.G);
  const int SHIFT = 32 - HB;
  const int NC = 1 << (HB - 6);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  __shared__ uint32_t s_b1, s_mode, s_cnt[kFiltThreads / 64];

  if (wave == 0) {
    uint32_t b1 = 0xFFFFFFFFu, mode = 0, above = 0, need = 0;
    if (sg.k_eff > 0) {
      const uint32_t* gh = p.hist + size_t(bh) * kHistStride;
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
      mode = cnt <= uint32_t(p.cap) ? kModeCand : kModeRescan;
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

  const float* row = p.scores + size_t(bh) * p.n_cap;
  const int wbase = t0 + wave * (kTile / 4);
  uint64_t myword = 0;
  uint32_t cnt = 0;
#pragma unroll 8
  for (int it = 0; it < 32; ++it) {
    const int n = wbase + it * 64 + lane;
    const float z = row[n];
    const bool valid = n >= sg.lo && n < sg.hi;
    const uint32_t key = f2key(z);
    const uint32_t dg = key >> SHIFT;
    const uint64_t m = __ballot(valid && dg > b1);
    if (lane == it) myword = m;
    cnt += uint32_t(__popcll(m));
    const bool cd = cand_mode && valid && dg == b1;
    const uint64_t cm = __ballot(cd);
    if (cm) {
      const int leader = __ffsll((unsigned long long)cm) - 1;
      uint32_t base = 0;
      if (lane == leader) base = atomicAdd(&p.state[bh].cand_count, uint32_t(__popcll(cm)));
      base = __shfl(base, leader);
      if (cd) {
        const uint32_t idx = base + uint32_t(__popcll(cm & ((1ull << lane) - 1ull)));
        if (idx < uint32_t(p.cap))
          p.cand[size_t(bh) * p.cap + idx] = (uint64_t(key) << 32) | uint32_t(~uint32_t(n));
      }
    }
  }
  if (lane < 32) p.bitmap[size_t(bh) * (p.n_cap / 64) + (wbase >> 6) + lane] = myword;
  if (lane == 0) s_cnt[wave] = cnt;
  __syncthreads();
  if (tid == 0) {
    uint32_t t = 0;
    for (int w = 0; w < kFiltThreads / 64; ++w) t += s_cnt[w];
    p.tile_cnt[size_t(bh) * p.n_tiles + tile] = t;
  }
}

hipError_t launch_filter(const Params& p, hipStream_t s) {
  const unsigned tiles = unsigned((int64_t(p.max_seq_len) + kTile - 1) / kTile);
  hipLaunchKernelGGL(filter_kernel, dim3(tiles, unsigned(p.B * p.H_q)),
                     dim3(kFiltThreads), 0, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------- resolve
// Members of bucket b1 as composite values: (key & low_mask) << 32 | ~n.
// A larger composite is a larger score, then a lower position; all distinct.
struct BucketSource {
  const Params* p;
  int bh;
  bool from_list;
  uint32_t count;   // list length
  int lo, hi;       // row range when rescanning
  uint32_t b1;
  int shift;        // 32 - HB
  uint64_t low_mask;

  template <typename Fn>
  __device__ __forceinline__ void for_each(Fn&& fn) const {
    if (from_list) {
      const uint64_t* c = p->cand + size_t(bh) * p->cap;
      for (uint32_t i = threadIdx.x; i < count; i += blockDim.x) {
        const uint64_t v = c[i];
        const uint32_t key = uint32_t(v >> 32);
        const uint32_t notn = uint32_t(v);
        fn((uint64_t(key) & low_mask) << 32 | notn, int(~notn));
      }
    } else {
      const float* row = p->scores + size_t(bh) * p->n_cap;
      for (int n = lo + int(threadIdx.x); n < hi; n += int(blockDim.x)) {
        const uint32_t key = f2key(row[n]);
        if ((key >> shift) != b1) continue;
        fn((uint64_t(key) & low_mask) << 32 | uint32_t(~uint32_t(n)), n);
      }
    }
  }
};

__global__ __launch_bounds__(kResThreads) void resolve_kernel(Params p) {
  const int bh = blockIdx.x;
  const int b = bh / p.H_q;
  const SeqGeom sg = seq_geom(p, b);
  if (sg.k_eff == 0) return;
  const HeadState st = p.state[bh];
  if (st.mode == 0) return;

  const int HB = hist_bits(p.G);
  const int TB = 64 - HB;  // composite bits: (32 - HB) key bits + 32 position bits
  BucketSource src;
  src.p = &p;
  src.bh = bh;
  src.from_list = st.mode == kModeCand;
  src.count = min(st.cand_count, uint32_t(p.cap));
  src.lo = sg.lo;
  src.hi = sg.hi;
  src.b1 = st.b1;
  src.shift = 32 - HB;
  src.low_mask = (1ull << (32 - HB)) - 1ull;

  __shared__ uint32_t hist[2048];
  __shared__ uint32_t s_d, s_above, s_cnt;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  uint32_t need = st.need1;
  uint64_t prefix = 0;
  int plen = 0;
  while (true) {
    const int w = min(11, TB - plen);
    const int shift = TB - plen - w;
    for (int i = tid; i < 2048; i += kResThreads) hist[i] = 0;
    __syncthreads();
    const int pl = plen;
    const uint64_t pf = prefix;
    const uint32_t dmask = (1u << w) - 1u;
    src.for_each([&](uint64_t c, int) {
      if (pl == 0 || (c >> (TB - pl)) == pf)
        atomicAdd(&hist[uint32_t(c >> shift) & dmask], 1u);
    });
    __syncthreads();
    if (wave == 0) {
      uint32_t s = 0;
      for (int i = 0; i < 32; ++i) s += hist[lane * 32 + i];
      const uint32_t suf = wave_suffix_sum(s);
      const uint64_t m = __ballot(suf >= need);
      const int L = m ? 63 - __clzll(m) : 0;
      if (lane == L) {
        uint32_t acc = suf - s;
        for (int i = 31; i >= 0; --i) {
          const uint32_t v = hist[lane * 32 + i];
          if (acc + v >= need || i == 0) {
            s_d = uint32_t(lane * 32 + i);
            s_above = acc;
            s_cnt = v;
            break;
          }
          acc += v;
        }
      }
    }
    __syncthreads();
    need -= s_above;
    prefix = (prefix << w) | s_d;
    plen += w;
    const uint32_t cnt = s_cnt;
    __syncthreads();
    if (cnt == need || plen >= TB) break;
  }

  // take every bucket member whose top plen composite bits are >= prefix
  const size_t words = size_t(p.n_cap / 64);
  const int pl = plen;
  const uint64_t pf = prefix;
  src.for_each([&](uint64_t c, int n) {
    if ((c >> (TB - pl)) >= pf) {
      atomicOr(reinterpret_cast<unsigned long long*>(&p.bitmap[size_t(bh) * words + (n >> 6)]),
               1ull << (n & 63));
      atomicAdd(&p.tile_cnt[size_t(bh) * p.n_tiles + n / kTile], 1u);
    }
  });
}

hipError_t launch_resolve(const Params& p, hipStream_t s) {
  hipLaunchKernelGGL(resolve_kernel, dim3(unsigned(p.B * p.H_q)),
                     dim3(kResThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace ra
