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
// threshold (one block per head, before the scan, when the scan does not
// run in the same call): the head's candidate bound from its sampled keys
// (sample_bound.h).
//
// select (one block per head, after the scan): if the per-unit candidate
// lists hold at least k_eff entries, the top-k of M is the top-k of the
// lists; a radix select on the composite finds the exact threshold (the
// bucket around the k-th entry is finished in LDS). The lists are read once
// into registers when they fit. A head with too few candidates is flagged;
// the dense stage rescans its group with every member of M as a candidate
// and selects again.
#include "page_scores.h"
#include "sample_bound.h"

namespace ra {

constexpr int kSelThreads = 512;
constexpr int kSubCap = 2048;     // LDS list for one radix sub-bucket
constexpr uint32_t kRankMax = 256; // sub-buckets up to this size are finished by ranking
constexpr int kRegEntries = 64;   // candidate entries per lane kept in registers (wide select)
constexpr int kStartRows = 4096;  // rows of 64 list entries whose first unit is tabled (wide)
static_assert(kRegEntries * kSelThreads / 64 <= kStartRows, "register rows must be tabled");
// The narrow select (select_kernel_narrow) holds 24 entries per lane and
// tables their 192 rows, so its registers and LDS leave room for two blocks
// per CU: when a batch has more heads than CUs they select in one round
// instead of two. It serves budgets up to kNarrowKMax, whose candidates
// (about 1.5 to 1.7 times k_eff under the sampled bound) fit its 12288
// register slots; more would be streamed, correctly but slower.
constexpr int kNarrowEntries = 24;
constexpr int kNarrowRows = kNarrowEntries * kSelThreads / 64;
constexpr int kNarrowKMax = 6144;

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
// as composites c = (key - lo) << 32 | ~n. In LDS: the non-empty units in
// order (ne) with the index of their first entry (pb), and for every row of
// 64 entries the non-empty unit holding its first entry (rowk) and a mask
// of the lanes where another one starts (rmask). The 64 lanes of a wave hold
// one row, so a lane finds its unit with a popcount. Rows past the table
// fall back to a binary search over pb.
struct UnitLists {
  const uint64_t* list;
  const uint16_t* ne;     // LDS [n_ne]
  const uint32_t* pb;     // LDS [n_ne + 1]
  const uint16_t* rowk;   // LDS [rows]
  const uint64_t* rmask;  // LDS [rows]
  int u_lo, n_ne;         // units u_lo .. overlap M; n_ne of them non-empty
  uint32_t rows;          // tabled rows
  uint32_t lo;

  __device__ __forceinline__ const uint64_t* at(int k, uint32_t i) const {
    return list + size_t(u_lo + ne[k]) * kUnit + (i - pb[k]);
  }

  // Entry i of row q (q wave-uniform, < rows).
  __device__ __forceinline__ const uint64_t* row_entry(uint32_t q, uint32_t i) const {
    const uint64_t below = (2ull << (i & 63u)) - 1ull;  // lanes 0 .. i % 64
    return at(int(rowk[q]) + __popcll(rmask[q] & below), i);
  }

  // Entry i anywhere: the last non-empty unit whose list begins at or
  // before i.
  __device__ __forceinline__ const uint64_t* search_entry(uint32_t i) const {
    int k = 0;
    for (int step = n_ne > 1 ? 1 << (31 - __clz(n_ne - 1)) : 0; step > 0; step >>= 1)
      k += (k + step < n_ne && pb[k + step] <= i) ? step : 0;
    return at(k, i);
  }

  // Entries [first, total) of the lists; first is a multiple of 64.
  template <typename Fn>
  __device__ __forceinline__ void for_each_from(uint32_t first, Fn&& fn) const {
    const uint32_t l = lo;
    const uint32_t total = pb[n_ne];
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    for (uint32_t base = first; base < total; base += blockDim.x * kBatch) {
      uint64_t v[kBatch];
      if ((min(base + blockDim.x * kBatch, total) + 63u) / 64u <= rows) {  // uniform: all tabled
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const uint32_t i = base + u * blockDim.x + threadIdx.x;
          const uint64_t* e = row_entry(min((base + u * blockDim.x) / 64u + wave, rows - 1u), i);
          v[u] = *(i < total ? e : list);
        }
      } else {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const uint32_t i = base + u * blockDim.x + threadIdx.x;
          v[u] = i < total ? *search_entry(i) : 0ull;
        }
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const uint32_t i = base + u * blockDim.x + threadIdx.x;
        const uint32_t n = uint32_t(v[u]);
        fn((uint64_t(uint32_t(v[u] >> 32) - l) << 32) | uint32_t(~n), int(n), i < total);
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

  // Straight-line groups of kBatch slots (no branch inside a group), so the
  // LDS lookups of a group overlap; lanes past the end load the list's
  // first entry, which is never used.
  __device__ __forceinline__ void load(const UnitLists& src) {
    static_assert(NR % kBatch == 0, "slots come in groups of kBatch");
    rest = src;
    total = min(src.pb[src.n_ne], uint32_t(NR) * blockDim.x);
    const uint32_t l = src.lo;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t waves = blockDim.x >> 6;
    const uint32_t qmax = src.rows > 0 ? src.rows - 1 : 0;
#pragma unroll
    for (int r0 = 0; r0 < NR; r0 += kBatch) {
      if (uint32_t(r0) * blockDim.x >= total) break;  // uniform
#pragma unroll
      for (int r = r0; r < r0 + kBatch; ++r) {
        const uint32_t i = r * blockDim.x + threadIdx.x;
        // rows below total / 64 are tabled (the table covers NR * blockDim)
        const uint64_t* e = src.row_entry(min(r * waves + wave, qmax), i);
        c[r] = *(i < total ? e : src.list);
      }
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

// One block per head: the head's candidate bound, published in its state.
// Left out when the scan runs in the same call: then the scan's blocks
// compute the bounds themselves (score_scan.hip).
__global__ __launch_bounds__(kSelThreads) void threshold_kernel(Params p) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t s_d, s_above, s_cnt;
  __shared__ int64_t tmp[16];
  const Radix rx{hist, &s_d, &s_above, &s_cnt};
  const uint32_t lo = head_bound(p, blockIdx.x, rx, tmp);
  if (threadIdx.x == 0) publish_bound(p, blockIdx.x, lo);
}

hipError_t launch_threshold(const Params& p, hipStream_t s) {
  hipLaunchKernelGGL(threshold_kernel, dim3(unsigned(p.B * p.H_q)), dim3(kSelThreads), 0, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------- select state
template <int ROWS>
struct SelLds {
  uint16_t ne[kMaxUnits];         // non-empty units (relative to u_lo), ascending
  uint32_t pb[kMaxUnits + 1];     // index of the first entry of each; the total
  uint16_t rowk[ROWS];            // non-empty unit holding entry 64 q (index into ne)
  uint64_t rmask[ROWS];           // bit l (l > 0): entry 64 q + l starts a unit
  uint32_t hist[2048];
  uint64_t sub[kSubCap];
  uint32_t s_d, s_above, s_cnt, s_n;
  int64_t tmp[16];
};

// List lengths of units u_lo .. u_lo + nu - 1 (their overlaps with M when
// dense), laid out as the non-empty units and their entry ranges, with the
// row table. Returns the list view. Block-wide.
template <int ROWS>
__device__ __forceinline__ UnitLists unit_prefix(const Params& p, int bh, const SeqGeom& sg, int u_lo, int nu,
                                 bool dense, uint32_t lo, SelLds<ROWS>& L) {
  constexpr int per = kMaxUnits / kSelThreads;
  const int tid = threadIdx.x;
  const uint32_t* uc = p.ucnt + size_t(bh) * p.n_units;
  for (int q = tid; q < ROWS; q += kSelThreads) L.rmask[q] = 0ull;
  uint32_t c[per];
  int64_t v = 0;  // entries << 13 | non-empty units (at most kMaxUnits < 2^13)
#pragma unroll
  for (int u = 0; u < per; ++u) {
    const int i = tid * per + u;
    c[u] = 0u;
    if (i < nu) {
      if (dense) {
        const int x = u_lo + i;
        c[u] = uint32_t(min((x + 1) * kUnit, sg.hi) - max(x * kUnit, sg.lo));
      } else {
        c[u] = uc[u_lo + i];
      }
    }
    v += (int64_t(c[u]) << 13) + (c[u] > 0u ? 1 : 0);
  }
  int64_t tot;
  const int64_t run = block_excl_scan(v, L.tmp, &tot);
  const uint32_t total = uint32_t(tot >> 13);
  const int n_ne = int(tot & 8191);
  const uint32_t rows = min(uint32_t(ROWS), (total + 63u) / 64u);
  uint32_t e = uint32_t(run >> 13);
  int k = int(run & 8191);
#pragma unroll
  for (int u = 0; u < per; ++u) {
    if (c[u] > 0u) {
      L.ne[k] = uint16_t(tid * per + u);
      L.pb[k] = e;
      const uint32_t q1 = min((e + c[u] + 63u) / 64u, rows);
      for (uint32_t q = (e + 63u) / 64u; q < q1; ++q) L.rowk[q] = uint16_t(k);
      if ((e & 63u) != 0u && e / 64u < rows)
        atomicOr(reinterpret_cast<unsigned long long*>(&L.rmask[e / 64u]), 1ull << (e & 63u));
      ++k;
      e += c[u];
    }
  }
  if (tid == 0) L.pb[n_ne] = total;
  __syncthreads();
  return UnitLists{p.cand + size_t(bh) * p.n_cap, L.ne, L.pb, L.rowk, L.rmask, u_lo, n_ne, rows, lo};
}

// Exact threshold of head bh over its candidates (source src), written
// into the head state.
template <typename Src, int ROWS>
__device__ __forceinline__ void decide(const Params& p, int bh, const SeqGeom& sg, const Src& src,
                                       int TB, uint32_t lo, SelLds<ROWS>& L) {
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

// Select over the lists of head bh, from registers when they fit (NR
// entries per lane).
template <int NR, int ROWS>
__device__ __forceinline__ void select_head(const Params& p, int bh, const SeqGeom& sg,
                                            const UnitLists& gl, uint32_t max_m, SelLds<ROWS>& L) {
  static_assert(NR * kSelThreads / 64 <= ROWS, "register rows must be tabled");
  const uint32_t span = max_m > gl.lo ? max_m - gl.lo : 1u;
  const int TB = 32 + bit_length(span);
  RegLists<NR> rl;
  rl.load(gl);
  decide(p, bh, sg, rl, TB, gl.lo, L);
}

// ---------------------------------------------------------------- select
// One launch, two kinds of blocks. The first B * H_q blocks select, one per
// head: with at least k_eff candidates the top-k of M is the top-k of the
// head's lists, whose exact threshold is decided here; a head with fewer
// is "short" and left to the rescan. The other blocks rescan: they walk the
// units like the scan, and in a group with a short head every member of M
// of the short heads becomes a candidate, written at its place in its
// unit's list (the list of unit u holds positions max(u * kUnit, lo) .. in
// order). A block decides shortness from the list lengths itself, so the
// two kinds never wait for each other; without short heads the rescan
// blocks only read the lengths. Finished units are counted per group, and
// the block that finishes a group's last unit selects again, over every
// member of M, for the group's short heads (their lists now hold all of M,
// so the list lengths are the units' overlaps with it). Nothing in this
// launch rewrites the counts the select blocks read, so it does not matter
// in which order the two kinds of blocks run.
static_assert(kScanThreads == kSelThreads, "the rescan blocks also select");

template <int NR, int ROWS>
__device__ __forceinline__ void select_block(const Params& p, int bh, SelLds<ROWS>& L) {
  const int b = bh / p.H_q;
  const SeqGeom sg = seq_geom(p, b);
  if (sg.k_eff == 0) return;  // the unset threshold takes nothing
  const HeadState st = p.state[bh];
  const int u_lo = sg.lo / kUnit, nu = (sg.hi - 1) / kUnit + 1 - u_lo;
  const UnitLists gl = unit_prefix(p, bh, sg, u_lo, nu, false, st.lo_key, L);
  if (gl.pb[gl.n_ne] < uint32_t(sg.k_eff)) {
    if (threadIdx.x == 0) {
      p.state[bh].dense = 1u;
      atomicAdd(p.any_dense, 1u);  // the count of rescanned heads
    }
    return;
  }
  select_head<NR>(p, bh, sg, gl, st.max_m, L);
}

// Bit hh set: head hh of group (b, g) has fewer than k_eff candidates.
// Wave hh sums the head's list lengths. Block-wide.
template <int G>
__device__ __forceinline__ uint32_t short_heads(const Params& p, int b, int g, uint32_t* s_mask) {
  const SeqGeom sg = seq_geom(p, b);
  const int wave = threadIdx.x >> 6;
  if (threadIdx.x == 0) *s_mask = 0u;
  __syncthreads();
  if (wave < G && sg.k_eff > 0) {
    const size_t bh = size_t(b) * p.H_q + size_t(g) * G + wave;
    const uint32_t* uc = p.ucnt + bh * p.n_units;
    const int u_lo = sg.lo / kUnit, u_hi = (sg.hi - 1) / kUnit + 1;
    uint32_t m = 0;
    for (int u = u_lo + lane_id(); u < u_hi; u += 64) m += uc[u];
    m = wave_sum(m);
    if (lane_id() == 0 && m < uint32_t(sg.k_eff)) atomicOr(s_mask, 1u << wave);
  }
  __syncthreads();
  return *s_mask;
}

template <int ROWS>
__device__ __forceinline__ void reselect_head(const Params& p, int bh, SelLds<ROWS>& L) {
  const HeadState st = p.state[bh];
  const SeqGeom sg = seq_geom(p, bh / p.H_q);
  const int u_lo = sg.lo / kUnit, nu = (sg.hi - 1) / kUnit + 1 - u_lo;
  // the lists hold every member of M now, so their lengths are the units'
  // overlaps with M; the candidate counts stay as the scan wrote them (the
  // select blocks of this launch read them, and the gather derives a
  // rescanned head's lengths from its dense flag instead)
  const UnitLists gl = unit_prefix(p, bh, sg, u_lo, nu, true, 0u, L);
  // all of M: far more than registers hold, so streamed on every pass
  const uint32_t span = st.max_m > 0u ? st.max_m : 1u;
  decide(p, bh, sg, gl, 32 + bit_length(span), 0u, L);
}

// Rescan of one unit for a group with short heads (mask), and the
// reselect when it is the group's last.
template <int G, int ROWS>
__device__ __forceinline__ void rescan_unit(const Params& p, UnitRef ur, uint32_t mask,
                                                      SelLds<ROWS>& S) {
  __shared__ uint32_t s_last;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const Lane<G> L;
  const int b = ur.b, g = ur.g;
  const int bg = b * p.H_kv + g;
  const SeqGeom sg = seq_geom(p, b);
  const size_t bh = size_t(b) * p.H_q + size_t(g) * G + L.F;
  const bool mine = (mask >> L.F) & 1u;
  uint4 qreg[G];
  load_q<G>(p, b, g, L, qreg);
  const int u0 = ur.u * kUnit;
  uint64_t* crow = p.cand + bh * p.n_cap + size_t(u0);
  const int first = max(u0, sg.lo);
  for (int jj = wave; jj < ur.npages; jj += kScanWaves) {
    const int j = ur.u * kUnitPages + jj;
    float z[G];
    page_scores<G>(p, page_of(p, b, j), g, L, qreg, z);
#pragma unroll
    for (int s = 0; s < G; ++s) {
      const int n = j * kPage + L.tok(s);
      if (mine && n >= sg.lo && n < sg.hi && RA_IN(n - first < kUnit, p, 4))
        crow[n - first] = (uint64_t(f2key(z[s])) << 32) | uint32_t(n);
    }
  }
  // this unit's lists are complete: make them visible, then count it
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int units = ((sg.N + kPage - 1) / kPage + kUnitPages - 1) / kUnitPages;
    s_last = atomicAdd(&p.gdone[bg], 1u) == uint32_t(units - 1) ? 1u : 0u;
  }
  __syncthreads();
  if (s_last) {
    __threadfence();  // see the lists the other blocks wrote
    for (int hh = 0; hh < G; ++hh)
      if ((mask >> hh) & 1u) reselect_head(p, b * p.H_q + g * G + hh, S);
  }
}

template <int G, int ROWS>
__device__ __forceinline__ void rescan_block(const Params& p, int blk, int nblk, SelLds<ROWS>& S) {
  __shared__ uint32_t s_mask;
  const int64_t T = p.unit_off[p.B];
  const int64_t X0 = T * blk / nblk;
  const int64_t X1 = T * (blk + 1) / nblk;
  int cur = -1;          // group whose mask is known
  uint32_t mask = 0u;
  for (int64_t x = X0; x < X1; ++x) {
    const UnitRef ur = unit_at(p, x);
    const int bg = ur.b * p.H_kv + ur.g;
    if (bg != cur) {  // block-uniform
      mask = short_heads<G>(p, ur.b, ur.g, &s_mask);
      cur = bg;
    }
    if (mask != 0u) rescan_unit<G>(p, ur, mask, S);
  }
}

// SELECT: blocks 0 .. B * H_q - 1 select; RESCAN: the rest (all blocks
// when not SELECT) rescan.
template <int G, int NR, int ROWS, bool SELECT, bool RESCAN>
__device__ __forceinline__ void select_body(const Params& p, SelLds<ROWS>& S) {
  const int heads = SELECT ? p.B * p.H_q : 0;
  if (SELECT && int(blockIdx.x) < heads) {
    select_block<NR>(p, blockIdx.x, S);
  } else if (RESCAN) {
    // after a select launch of its own, whose blocks counted the short
    // heads: with none, there is nothing to rescan
    if (!SELECT && *p.any_dense == 0u) return;  // block-uniform
    rescan_block<G>(p, int(blockIdx.x) - heads, int(gridDim.x) - heads, S);
  }
}

// both kinds of blocks in one launch
template <int G>
__global__ __launch_bounds__(kSelThreads) void select_kernel(Params p) {
  __shared__ SelLds<kStartRows> S;
  select_body<G, kRegEntries, kStartRows, true, true>(p, S);
}

// For batches with more heads than CUs and budgets up to kNarrowKMax: the
// select blocks alone, at most 128 registers per lane and 51 KB of LDS, two
// per CU; the rescan follows in its own launch (its registers would not fit
// beside them).
template <int G>
__global__ __launch_bounds__(kSelThreads) __attribute__((amdgpu_waves_per_eu(4)))
void select_kernel_narrow(Params p) {
  __shared__ SelLds<kNarrowRows> S;
  select_body<G, kNarrowEntries, kNarrowRows, true, false>(p, S);
}

template <int G>
__global__ __launch_bounds__(kSelThreads) void rescan_kernel(Params p) {
  __shared__ SelLds<kStartRows> S;
  select_body<G, kRegEntries, kStartRows, false, true>(p, S);
}

template <int G>
static void launch_select_g(const Params& p, hipStream_t s) {
  const unsigned heads = unsigned(p.B * p.H_q);
  const dim3 block{unsigned(kSelThreads)};
  const int cus = p.num_cus > 0 ? p.num_cus : 256;
  if (p.k_max <= kNarrowKMax && int64_t(heads) > cus) {
    hipLaunchKernelGGL(select_kernel_narrow<G>, dim3(heads), block, 0, s, p);
    hipLaunchKernelGGL(rescan_kernel<G>, dim3(scan_blocks(p)), block, 0, s, p);
  } else {
    hipLaunchKernelGGL(select_kernel<G>, dim3(heads + scan_blocks(p)), block, 0, s, p);
  }
}

hipError_t launch_select(const Params& p, hipStream_t s) {
  switch (p.G) {
    case 1: launch_select_g<1>(p, s); break;
    case 2: launch_select_g<2>(p, s); break;
    case 4: launch_select_g<4>(p, s); break;
    case 8: launch_select_g<8>(p, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ra
