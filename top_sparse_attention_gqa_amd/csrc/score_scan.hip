// Exact scores of every cached key for every query head of its GQA group,
// z = q . k / sqrt(128) (RetrievalAttention slides, "Sparse attention
// renormalizes selected tokens", Eq. (1)), streamed once from HBM; one wave
// scores one (page, KV head) block at a time (page_scores.h).
//
// HBM writes interleaved with this read stream cost far more than their
// bytes, so the scan does not store the score rows. A sampling pass first
// scores one page in S; from the sample every head gets a conservative
// threshold such that, with a wide statistical margin, at least k_eff
// members of M score at or above it. The scan then keeps only those
// candidates, staged in LDS over one or several units of 64 pages and
// written in one burst to per-(head, unit) lists, plus the scores of the
// static set W. The
// selection checks the margin exactly (it needs at least k_eff candidates);
// heads that fail it are rescanned with every member of M as a candidate.
//
// The thresholds are computed by the scan's own blocks (sample_bound.h):
// block i first computes those of heads i, i + grid, ... and publishes
// them, then streams; a block whose group's thresholds are not yet out when
// it starts holds its first pages' keys in LDS, and decides their
// candidates once they are (or computes a missing one itself after a
// bounded wait). Every block computes the same value for a head, so the
// result does not depend on which one did.
#include "page_scores.h"
#include "sample_bound.h"

namespace ra {

constexpr int kStage = 8192;       // LDS candidate staging entries per block
constexpr int kDeferUnits = 16;    // units whose candidates one burst may write
// sampled pages per sample block, one per wave: at 95 VGPRs five such
// blocks fit a CU, against two of eight waves
constexpr int kSampleWaves = 4;
constexpr int kSampleThreads = kSampleWaves * 64;

// ---------------------------------------------------------------- sample
// Resets of the per-call state of group (b, g), by block (b * H_kv + g, 0)
// of the sample launch: the group's head states, its rescan counter and the
// per-unit candidate counts (the scan may reserve list slots with atomics),
// and the step's new token when there is one (lanes 0..15 write its K row,
// 16..31 its V row, 16 bytes each). Writing the token here, while other
// blocks of the launch may read its page, is safe: it is the last position,
// inside the recent window whenever window > 0, whose keys the sample does
// not keep, and otherwise a stale sampled key only loosens the bound; the
// scan and everything after it read the row after this launch.
template <int G>
__device__ __forceinline__ void group_reset(const Params& p, int b, int g, int P) {
  const int tid = threadIdx.x;
  const size_t bh0 = size_t(b) * p.H_q + size_t(g) * G;
  if (p.app_pos != nullptr && tid < 32) {
    const int ps = p.app_pos[b];
    if (ps >= 0 && ps < p.max_pages * kPage) {
      const int pg = p.block_table[size_t(b) * p.max_pages + ps / kPage];
      if ((unsigned)pg < (unsigned)p.num_pages) {
        const int part = tid >> 4, c = tid & 15;
        const uint16_t* src = (part ? p.app_v : p.app_k) + (size_t(b) * p.H_kv + g) * kHeadDim + c * 8;
        uint16_t* dst = const_cast<uint16_t*>(part ? p.v_pool : p.k_pool) +
                        ((size_t(pg) * p.H_kv + g) * kPage + (ps & (kPage - 1))) * kHeadDim + c * 8;
        *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
      }
    }
  }
  if (tid < G) {
    HeadState st;
    st.lo_key = 0u;
    st.lo_set = 0u;  // published later by the threshold launch or the scan
    st.max_w = 0u;
    st.max_m = 0u;
    st.dense = 0u;
    st.thr_shift = 64u;  // nothing passes until select decides
    st.thr_lo = 0xFFFFFFFFu;
    st.thr_hi = 0xFFFFFFFFu;
    p.state[bh0 + tid] = st;
  }
  if (tid == 0) p.gdone[size_t(b) * p.H_kv + g] = 0u;
  const int nu = (P + kUnitPages - 1) / kUnitPages;
  for (int i = tid; i < G * nu; i += blockDim.x)
    p.ucnt[(bh0 + size_t(i / nu)) * p.n_units + size_t(i % nu)] = 0u;
}

// The unit prefix over the batch, which the scan and rescan distribute
// their work by, and the rescan counter. Every thread of the block.
__device__ __forceinline__ void batch_reset(const Params& p, int64_t* tmp) {
  const int tid = threadIdx.x;
  const int per = (p.B + int(blockDim.x) - 1) / int(blockDim.x);
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

// Grid (B * H_kv, chunks + 1): block (bg, c < chunks) scores the sampled
// pages c * kSampleWaves .. of group bg, one page per wave, and stores the
// keys of the sampled positions per head (0 past the sequence's end; the
// scan takes these pages' scores from here instead of reading them again);
// block
// (bg, chunks) resets the group's per-call state, and (0, chunks) also the
// batch's, so that the sampling blocks do nothing else.
template <int G>
__global__ __launch_bounds__(kSampleThreads) void sample_kernel(Params p) {
  __shared__ int64_t tmp[16];
  const int bg = blockIdx.x;
  const int b = bg / p.H_kv;
  const int g = bg - b * p.H_kv;
  const SeqGeom sg = seq_geom(p, b);
  const int P = (sg.N + kPage - 1) / kPage;
  if (blockIdx.y == gridDim.y - 1) {  // block-uniform
    if (bg == 0) batch_reset(p, tmp);
    group_reset<G>(p, b, g, P);
    return;
  }
  const int ns = sampled_pages(P);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = blockIdx.y * kSampleWaves + wave;
  if (t >= ns) return;
  const Lane<G> L;
  const int S = 1 << sample_log2(P);
  const int j = (S >> 1) + t * S;
  uint4 qreg[G];
  load_q<G>(p, b, g, L, qreg);
  float z[G];
  page_scores<G>(p, page_of(p, b, j), g, L, qreg, z);
  uint32_t* row = p.samp + (size_t(b) * p.H_q + size_t(g) * G + L.F) * p.samp_cap + size_t(t) * kPage;
#pragma unroll
  for (int s = 0; s < G; ++s) {
    const int pos = j * kPage + L.tok(s);
    if (RA_IN(size_t(t) * kPage + L.tok(s) < size_t(p.samp_cap), p, 3))
      row[L.tok(s)] = pos < sg.N ? f2key(z[s]) : 0u;
  }
}

#if defined(RA_DEBUG)
// the failed-check word starts each step at zero, before any kernel can set it
__global__ void dbg_reset_kernel(uint32_t* w) { *w = 0u; }
#endif

hipError_t launch_sample(const Params& p, hipStream_t s) {
#if defined(RA_DEBUG)
  hipLaunchKernelGGL(dbg_reset_kernel, dim3(1), dim3(1), 0, s, p.dbg);
#endif
  const int ns_max = p.samp_cap / kPage;
  const unsigned chunks = unsigned(ns_max > 0 ? (ns_max + kSampleWaves - 1) / kSampleWaves : 1);
  const dim3 grid{unsigned(p.B * p.H_kv), chunks + 1}, block{unsigned(kSampleThreads)};
  switch (p.G) {
    case 1: hipLaunchKernelGGL(sample_kernel<1>, grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL(sample_kernel<2>, grid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL(sample_kernel<4>, grid, block, 0, s, p); break;
    case 8: hipLaunchKernelGGL(sample_kernel<8>, grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- scan
// Pages of a unit whose keys a block can hold in LDS while it waits for the
// group's candidate bounds (a multiple of kScanWaves). 32 pages are four per
// wave, past the time a bound takes, and fewer held keys to decide once the
// bounds are out measured faster than a whole unit (64 pages: C3_1 scan
// 1-1.5 us, C2 1.4 us more).
template <int G>
struct RawCfg {
  static constexpr int pages = G >= 4 ? 32 : kUnitPages;
  static constexpr int words = pages * kPage * G;
  static_assert(pages % kScanWaves == 0, "whole rounds of the block's waves");
};

// How often a block polls for a bound another block computes before it
// computes the bound itself (the value is the same either way). In a
// debug build it does not wait, and the blocks leave the bounds of odd
// heads to the blocks that need them, so that both ways run.
#if defined(RA_DEBUG)
constexpr int kBoundPolls = 0;
constexpr bool kHelpOddHeads = false;
#else
constexpr int kBoundPolls = 32;
constexpr bool kHelpOddHeads = true;
#endif

// Persistent over the linear unit index (sequence, KV head, unit of 64
// pages): each block takes a contiguous range of units. The candidates
// (members of M scoring at or above the head's threshold) are staged in LDS
// over one or several units of a group and written in one burst to the
// (head, unit) lists with their counts; the block owns those units, so no
// global atomics are needed (in a split scan, where two blocks may share a
// unit, each unit's slots are reserved with them).
// W scores go straight to the score rows. Running maxima over W and M per
// head are folded into the head state whenever the block moves to another
// (sequence, KV head) and at its end.
template <int G>
__global__ __launch_bounds__(kScanThreads) void scan_kernel(Params p) {
  __shared__ uint32_t st_key[kStage];
  __shared__ uint32_t st_nh[kStage];  // position | head << 27
  __shared__ uint32_t raw[RawCfg<G>::words];  // keys of pages held for the bounds
  __shared__ uint32_t s_fill;
  __shared__ uint32_t s_lo[G];
  __shared__ uint32_t s_set[G];   // 1: s_lo holds the head's bound
  __shared__ uint32_t s_cnt[G];
  __shared__ uint32_t s_ucnt[G][kDeferUnits];  // list slots taken per (head, staged unit)
  __shared__ uint32_t s_base[G];  // first slot the burst reserved in each head's list (page split)
  __shared__ uint32_t lmax[G][2];     // max key over W, over M
  __shared__ uint32_t r_d, r_above, r_cnt, s_flag;
  __shared__ int64_t tmp[16];
  // the bound computation borrows the staging keys as its histogram: the
  // staging is empty whenever it runs (before the first unit, and before a
  // unit's first candidate is staged)
  const Radix rx{st_key, &r_d, &r_above, &r_cnt};

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const Lane<G> L;

  // the bounds this block computes up front (already published ones, by a
  // threshold launch in an earlier call, are skipped)
  const int H = p.scan_bounds ? p.B * p.H_q : 0;
  for (int bh = blockIdx.x; bh < H; bh += gridDim.x) {
    if (!kHelpOddHeads && (bh & 1)) continue;
    if (tid == 0) {
      uint32_t lo;
      s_flag = read_bound(p, bh, &lo) ? 1u : 0u;
    }
    __syncthreads();
    const bool known = s_flag != 0u;  // block-uniform
    __syncthreads();
    if (!known) {
      const uint32_t lo = head_bound(p, bh, rx, tmp);
      if (tid == 0) publish_bound(p, bh, lo);
    }
  }
  __syncthreads();
  if (tid == 0) s_fill = 0;
  if (tid < G) s_cnt[tid] = 0;
  for (int i = tid; i < G * kDeferUnits; i += kScanThreads) (&s_ucnt[0][0])[i] = 0u;
  if (tid < 2 * G) lmax[tid >> 1][tid & 1] = 0u;

  // Units split evenly over the blocks. For one sequence whose units do
  // not divide evenly (a length just past a multiple of 64 pages leaves a
  // short last unit per KV head, and some block would take it on top of
  // full ones) the pages are split instead, and a unit two blocks share
  // has its list slots reserved with global atomics (3 us less scan at
  // N = 2^20 + 1000; for ragged batches the unit split measured better).
  const int64_t T = p.unit_off[p.B];
  const int64_t NB = gridDim.x;
  const bool split = p.B == 1 && T % NB != 0;  // block-uniform
  const int64_t TP = T * kUnitPages;
  const int64_t X0p = split ? TP * blockIdx.x / NB : (T * blockIdx.x / NB) * kUnitPages;
  const int64_t X1p = split ? TP * (blockIdx.x + 1) / NB : (T * (blockIdx.x + 1) / NB) * kUnitPages;
  const int64_t X0 = X0p / kUnitPages, X1 = (X1p + kUnitPages - 1) / kUnitPages;
  uint32_t mw = 0u, mm = 0u;  // running max keys of head F over W and M
  int u_first = 0, nu_st = 0;  // staged units: u_first .. u_first + nu_st - 1 of one group
  bool sync_top = true;        // LDS state changed since the last barrier
  int cur_b = -1, cur_g = -1;
  uint4 qreg[G];
  for (int64_t x = X0; x < X1; ++x) {
    const UnitRef ur = unit_at(p, x);
    const int b = ur.b, g = ur.g;
    const SeqGeom sg = seq_geom(p, b);
    const size_t bh0 = size_t(b) * p.H_q + size_t(g) * G;
    if (nu_st == 0) u_first = ur.u;
    const int lu = nu_st;  // this unit among the staged ones (0 in a split scan)
    if (b != cur_b || g != cur_g) {
      if (cur_b >= 0) {
        // fold the maxima of the previous group
        const size_t pbh0 = size_t(cur_b) * p.H_q + size_t(cur_g) * G;
#pragma unroll
        for (int m = 1; m < ScanCfg<G>::D; m <<= 1) {
          mw = max(mw, uint32_t(__shfl_xor(int(mw), m)));
          mm = max(mm, uint32_t(__shfl_xor(int(mm), m)));
        }
        mw = max(mw, uint32_t(__shfl_xor(int(mw), 16)));
        mm = max(mm, uint32_t(__shfl_xor(int(mm), 16)));
        mw = max(mw, uint32_t(__shfl_xor(int(mw), 32)));
        mm = max(mm, uint32_t(__shfl_xor(int(mm), 32)));
        if (L.row == 0 && L.qsel == 0) {
          if (mw) atomicMax(&lmax[L.F][0], mw);
          if (mm) atomicMax(&lmax[L.F][1], mm);
        }
        __syncthreads();
        if (tid < 2 * G) {
          const int hh = tid >> 1;
          const uint32_t v = lmax[hh][tid & 1];
          if (v) atomicMax((tid & 1) ? &p.state[pbh0 + hh].max_m : &p.state[pbh0 + hh].max_w, v);
          lmax[hh][tid & 1] = 0u;
        }
        mw = mm = 0u;
      }
      cur_b = b;
      cur_g = g;
      if (tid < G) {
        uint32_t lo;
        s_set[tid] = read_bound(p, bh0 + tid, &lo) ? 1u : 0u;
        s_lo[tid] = lo;
      }
      load_q<G>(p, b, g, L, qreg);
      sync_top = true;
    }
    // between two units of a group whose candidates stay staged, the
    // waves run on without meeting
    if (sync_top) __syncthreads();
    sync_top = false;
    bool ready = true;  // block-uniform: every bound of the group is known
#pragma unroll
    for (int hh = 0; hh < G; ++hh) ready = ready && s_set[hh] != 0u;
    uint32_t lo_f = s_lo[L.F];
    float* srow = p.scores + (bh0 + L.F) * p.n_cap;
    const size_t ubase = size_t(ur.u) * kUnit;
    uint64_t* crow = p.cand + (bh0 + L.F) * p.n_cap + ubase;
    // this block's pages of the unit
    const int pa = int(max<int64_t>(X0p - x * kUnitPages, 0));
    const int pe = int(min<int64_t>(min<int64_t>(X1p - x * kUnitPages, kUnitPages), ur.npages));
    // pages [pa, pr) are scored before the bounds are known, their keys held
    const int pr = ready ? pa : min(pe, pa + RawCfg<G>::pages);
    // the physical pages of this wave's pages of the unit, read up front
    // (lane k holds the page of the wave's k-th page)
    const int my_pg = L.lane < kUnitPages / kScanWaves && pa + wave + kScanWaves * L.lane < pe
                          ? page_of(p, b, ur.u * kUnitPages + pa + wave + kScanWaves * L.lane)
                          : 0;

    // Scores of page jj of the unit: a sampled page's come from its keys in
    // the sample rows (the same function of the same K and q, so the same
    // values), except the page of a token appended in this call, whose row
    // the sample launch may have read before it was written
    const int ssh = sample_log2((sg.N + kPage - 1) / kPage);
    const int app_ps = p.app_pos != nullptr ? p.app_pos[b] : -1;
    const int app_page = app_ps >= 0 ? app_ps / kPage : -1;
    const uint32_t* krow = p.samp + (bh0 + L.F) * size_t(p.samp_cap);
    auto scores = [&](int jj, int j, float (&z)[G]) {
      if ((j & ((1 << ssh) - 1)) == ((1 << ssh) >> 1) && j != app_page) {  // wave-uniform
        const size_t t = size_t(j >> ssh) * kPage;
#pragma unroll
        for (int s = 0; s < G; ++s)
          z[s] = RA_IN(t + L.tok(s) < size_t(p.samp_cap), p, 3) ? key2f(krow[t + L.tok(s)]) : 0.0f;
      } else {
        page_scores<G>(p, __shfl(my_pg, (jj - pa - wave) / kScanWaves), g, L, qreg, z);
      }
    };
    // W score and running maxima of one scored position; true if it is a
    // member of M
    // (the maxima as value selects: conditional updates of the two were
    // merged into one store through a selected address, which put both in
    // scratch memory)
    auto account = [&](int n, uint32_t key, float zs) {
      const bool in_m = n >= sg.lo && n < sg.hi;
      const bool in_w = !in_m && n < sg.N;
      if (in_w && RA_IN(n < p.n_cap, p, 2)) srow[n] = zs;
      mw = max(mw, in_w ? key : 0u);
      mm = max(mm, in_m ? key : 0u);
      return in_m;
    };
    // stage the candidates of one round of the wave (cand per lane)
    auto stage = [&](bool cand, uint32_t key, int n) {
      const uint64_t cm = __ballot(cand);
      if (!cm) return;
      const int leader = __ffsll((unsigned long long)cm) - 1;
      uint32_t base = 0;
      if (L.lane == leader) base = atomicAdd(&s_fill, uint32_t(__popcll(cm)));
      base = __shfl(base, leader);
      if (cand) {
        const uint32_t idx = base + uint32_t(__popcll(cm & ((1ull << L.lane) - 1ull)));
        if (idx < uint32_t(kStage)) {
          st_key[idx] = key;
          st_nh[idx] = uint32_t(n) | (uint32_t(L.F) << 27);
          if (split) atomicAdd(&s_cnt[L.F], 1u);
        } else {
          // staging full: take a slot of the list at once
          const uint32_t slot = split ? atomicAdd(&p.ucnt[(bh0 + L.F) * p.n_units + ur.u], 1u)
                                      : atomicAdd(&s_ucnt[L.F][lu], 1u);
          if (RA_IN(slot < uint32_t(kUnit), p, 1))
            crow[slot] = (uint64_t(key) << 32) | uint32_t(n);
        }
      }
    };

    if (!ready) {  // block-uniform
      for (int jj = pa + wave; jj < pr; jj += kScanWaves) {
        const int j = ur.u * kUnitPages + jj;
        // lanes 0 .. G-1 look for the bounds while the page is in flight
        // (the load is issued first and its value used last)
        uint64_t bw = 0u;
        if (L.lane < G)
          bw = __hip_atomic_load(bound_slot(p, bh0 + L.lane), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
        float z[G];
        scores(jj, j, z);
#pragma unroll
        for (int s = 0; s < G; ++s) {
          const int n = j * kPage + L.tok(s);
          const uint32_t key = f2key(z[s]);
          account(n, key, z[s]);
          raw[((jj - pa) * G + s) * kPage + L.lane] = key;
        }
        if (L.lane < G && (bw >> 32) != 0u) {
          s_lo[L.lane] = uint32_t(bw);  // the same value from every lane that sees it
          s_set[L.lane] = 1u;
        }
      }
      __syncthreads();
      // the bounds still missing: a bounded wait, in parallel over the heads
      if (tid < G && s_set[tid] == 0u) {
        uint32_t lo = 0u;
        bool ok = read_bound(p, bh0 + tid, &lo);
        for (int i = 0; i < kBoundPolls && !ok; ++i) {
          __builtin_amdgcn_s_sleep(8);
          ok = read_bound(p, bh0 + tid, &lo);
        }
        if (ok) {
          s_lo[tid] = lo;
          s_set[tid] = 1u;
        }
      }
      // and what is still missing after it, computed here
      for (int hh = 0; hh < G; ++hh) {
        __syncthreads();
        if (s_set[hh] == 0u) {  // block-uniform
          const uint32_t lo = head_bound(p, int(bh0) + hh, rx, tmp);
          __syncthreads();  // every thread has read s_set[hh]
          if (tid == 0) {
            publish_bound(p, bh0 + hh, lo);
            s_lo[hh] = lo;
            s_set[hh] = 1u;
          }
        }
      }
      __syncthreads();
      lo_f = s_lo[L.F];
      // the held pages' candidates (each lane reads back its own keys): a
      // count per lane, one reservation per wave, then the stores
      uint32_t mine = 0u;
      for (int jj = pa + wave; jj < pr; jj += kScanWaves) {
        const int j = ur.u * kUnitPages + jj;
#pragma unroll
        for (int s = 0; s < G; ++s) {
          const int n = j * kPage + L.tok(s);
          const uint32_t key = raw[((jj - pa) * G + s) * kPage + L.lane];
          mine += (n >= sg.lo && n < sg.hi && key >= lo_f) ? 1u : 0u;
        }
      }
      uint32_t incl = mine;  // inclusive prefix over the wave's lanes
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t t = __shfl_up(incl, off);
        if (L.lane >= off) incl += t;
      }
      const uint32_t wtot = __shfl(incl, 63);
      uint32_t wbase = 0u;
      if (L.lane == 0 && wtot) wbase = atomicAdd(&s_fill, wtot);
      uint32_t idx = __shfl(wbase, 0) + incl - mine;
      if (mine) {  // lane-divergent: no wave operation inside
        for (int jj = pa + wave; jj < pr; jj += kScanWaves) {
          const int j = ur.u * kUnitPages + jj;
#pragma unroll
          for (int s = 0; s < G; ++s) {
            const int n = j * kPage + L.tok(s);
            const uint32_t key = raw[((jj - pa) * G + s) * kPage + L.lane];
            if (n >= sg.lo && n < sg.hi && key >= lo_f) {
              if (idx < uint32_t(kStage)) {
                st_key[idx] = key;
                st_nh[idx] = uint32_t(n) | (uint32_t(L.F) << 27);
                if (split) atomicAdd(&s_cnt[L.F], 1u);
              } else {
                // staging full: take a slot of the list at once
                const uint32_t slot = split ? atomicAdd(&p.ucnt[(bh0 + L.F) * p.n_units + ur.u], 1u)
                                            : atomicAdd(&s_ucnt[L.F][lu], 1u);
                if (RA_IN(slot < uint32_t(kUnit), p, 1))
                  crow[slot] = (uint64_t(key) << 32) | uint32_t(n);
              }
              ++idx;
            }
          }
        }
      }
    }
    for (int jj = pr + wave; jj < pe; jj += kScanWaves) {
      const int j = ur.u * kUnitPages + jj;
      float z[G];
      scores(jj, j, z);
#pragma unroll
      for (int s = 0; s < G; ++s) {
        const int n = j * kPage + L.tok(s);
        const uint32_t key = f2key(z[s]);
        const bool in_m = account(n, key, z[s]);
        stage(in_m && key >= lo_f, key, n);
      }
    }
    // burst the staged candidates into the (head, unit) lists; streaming
    // stores, since cached writes interleaved with the K stream cost it
    // about twice as much time
    if (split) {
      // a split scan reserves the list slots of each unit with global
      // atomics (two blocks may share it) and writes one burst per unit
      // (kept over several units, its bursts measured slower: 335 against
      // 325 us per scan for the 32-layer workload at 2^20 + 1000 tokens)
      __syncthreads();
      const uint32_t nst = min(s_fill, uint32_t(kStage));
      if (tid < G) {
        s_base[tid] = s_cnt[tid] ? atomicAdd(&p.ucnt[(bh0 + tid) * p.n_units + ur.u], s_cnt[tid]) : 0u;
        s_cnt[tid] = 0;
      }
      __syncthreads();
      for (uint32_t i = tid; i < nst; i += kScanThreads) {
        const uint32_t nh = st_nh[i];
        const uint32_t hh = nh >> 27;
        const uint32_t slot = s_base[hh] + atomicAdd(&s_cnt[hh], 1u);
        if (RA_IN(slot < uint32_t(kUnit), p, 0))
          __builtin_nontemporal_store((uint64_t(st_key[i]) << 32) | (nh & ((1u << 27) - 1u)),
                                      &p.cand[(bh0 + hh) * p.n_cap + ubase + slot]);
      }
      __syncthreads();
      if (tid < G) s_cnt[tid] = 0;
      if (tid == 0) s_fill = 0;
      sync_top = true;
      continue;
    }
    // Otherwise the block owns its units: their candidates stay staged over
    // several units of the group and are written in one burst when the
    // group ends, the block is done, or as many units are staged as the
    // staging holds at 1.6 k_eff candidates per head (the sampled bound
    // passes about 1.5 k_eff; a unit that passes more sends the excess
    // straight to its list). Each burst stops the block's waves at two
    // barriers; between bursts they do not meet.
    ++nu_st;
    const int np_seq = (sg.N + kPage - 1) / kPage;
    const int np_next = min(kUnitPages, np_seq - (ur.u + 1) * kUnitPages);
    const bool next_here = x + 1 < X1 && np_next > 0;
    const int64_t per_unit =
        int64_t(G) * 8 * sg.k_eff / (5 * ((np_seq + kUnitPages - 1) / kUnitPages)) + 64;
    const int n_defer = int(max<int64_t>(1, min<int64_t>(kDeferUnits, kStage / per_unit)));
    if (next_here && nu_st < n_defer) continue;  // block-uniform
    __syncthreads();
    const uint32_t nst = min(s_fill, uint32_t(kStage));
    for (uint32_t i = tid; i < nst; i += kScanThreads) {
      const uint32_t nh = st_nh[i];
      const uint32_t hh = nh >> 27;
      const uint32_t n = nh & ((1u << 27) - 1u);
      const int su = int(n / uint32_t(kUnit)) - u_first;  // staged unit of the entry
      if (RA_IN(su >= 0 && su < nu_st, p, 0)) {
        const uint32_t slot = atomicAdd(&s_ucnt[hh][su], 1u);
        if (RA_IN(slot < uint32_t(kUnit), p, 0))
          __builtin_nontemporal_store((uint64_t(st_key[i]) << 32) | n,
                                      &p.cand[(bh0 + hh) * p.n_cap +
                                              size_t(u_first + su) * kUnit + slot]);
      }
    }
    __syncthreads();
    for (int i = tid; i < G * nu_st; i += kScanThreads) {
      const int hh = i / nu_st, su = i - hh * nu_st;
      p.ucnt[(bh0 + hh) * p.n_units + u_first + su] = s_ucnt[hh][su];
      s_ucnt[hh][su] = 0u;
    }
    nu_st = 0;
    if (tid == 0) s_fill = 0;
    sync_top = true;
  }
  if (cur_b >= 0) {
    const size_t pbh0 = size_t(cur_b) * p.H_q + size_t(cur_g) * G;
#pragma unroll
    for (int m = 1; m < ScanCfg<G>::D; m <<= 1) {
      mw = max(mw, uint32_t(__shfl_xor(int(mw), m)));
      mm = max(mm, uint32_t(__shfl_xor(int(mm), m)));
    }
    mw = max(mw, uint32_t(__shfl_xor(int(mw), 16)));
    mm = max(mm, uint32_t(__shfl_xor(int(mm), 16)));
    mw = max(mw, uint32_t(__shfl_xor(int(mw), 32)));
    mm = max(mm, uint32_t(__shfl_xor(int(mm), 32)));
    if (L.row == 0 && L.qsel == 0) {
      if (mw) atomicMax(&lmax[L.F][0], mw);
      if (mm) atomicMax(&lmax[L.F][1], mm);
    }
    __syncthreads();
    if (tid < 2 * G) {
      const int hh = tid >> 1;
      const uint32_t v = lmax[hh][tid & 1];
      if (v) atomicMax((tid & 1) ? &p.state[pbh0 + hh].max_m : &p.state[pbh0 + hh].max_w, v);
    }
  }
}

// One persistent block per CU: the scan block's registers leave room for
// one 8-wave block per CU, so a larger grid would only run in two rounds.
unsigned scan_blocks(const Params& p) {
  const int64_t units_max = int64_t(p.B) * p.H_kv *
      ((int64_t(p.max_seq_len) + kUnit - 1) / kUnit);
  const int64_t cap = p.num_cus > 0 ? p.num_cus : 256;
  int64_t blocks = units_max < cap ? units_max : cap;
  if (blocks < 1) blocks = 1;
  return unsigned(blocks);
}

// With at most one head per scan block the bounds cost the scan less than
// a launch of their own (measured: 3.4 us less per step for one 1M-token
// Llama-3-8B layer, 2.4 us at 128K); with two per block (16 sequences of
// 32 heads) every block starts streaming late and the threshold launch is
// the faster one. The sample must also fit the registers of one block
// (16,384 keys per head, lengths up to about 2^20 + 4,000): a bound over a
// larger sample is streamed and takes longer than the blocks hold their
// first pages.
bool scan_computes_bounds(const Params& p) {
  return int64_t(p.B) * p.H_q <= int64_t(scan_blocks(p)) &&
         int64_t(p.samp_cap) <= int64_t(kRegKeys) * kScanThreads;
}

hipError_t launch_scan(const Params& p, hipStream_t s) {
  const dim3 grid{scan_blocks(p)}, block{unsigned(kScanThreads)};
  switch (p.G) {
    case 1: hipLaunchKernelGGL(scan_kernel<1>, grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL(scan_kernel<2>, grid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL(scan_kernel<4>, grid, block, 0, s, p); break;
    case 8: hipLaunchKernelGGL(scan_kernel<8>, grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ra
