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
// candidates, staged in LDS and written in one burst per unit of 64 pages
// to per-(head, unit) lists, plus the scores of the static set W. The
// selection checks the margin exactly (it needs at least k_eff candidates);
// heads that fail it are rescanned with every member of M as a candidate.
#include "page_scores.h"

namespace ra {

constexpr int kStage = 6144;       // LDS candidate staging entries per block
constexpr int kSampleWaves = 8;    // sampled pages per sample block (one per wave)
constexpr int kSampleThreads = kSampleWaves * 64;

// ---------------------------------------------------------------- sample
// Grid (B * H_kv, chunks): block (bg, c) scores the sampled pages
// c * kSampleWaves .. of group bg, one page per wave, and stores the keys of
// the sampled positions per head (0 for positions outside M).
template <int G>
__global__ __launch_bounds__(kSampleThreads) void sample_kernel(Params p) {
  const int bg = blockIdx.x;
  const int b = bg / p.H_kv;
  const int g = bg - b * p.H_kv;
  const SeqGeom sg = seq_geom(p, b);
  const int P = (sg.N + kPage - 1) / kPage;
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
      row[L.tok(s)] = (pos >= sg.lo && pos < sg.hi) ? f2key(z[s]) : 0u;
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
  const dim3 grid{unsigned(p.B * p.H_kv), chunks}, block{unsigned(kSampleThreads)};
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
// Persistent over the linear unit index (sequence, KV head, unit of 64
// pages): each block takes a contiguous range of units. Per unit, the
// candidates (members of M scoring at or above the head's threshold) are
// staged in LDS and written after the unit to the (head, unit) lists with
// their counts; the block owns the unit, so no global atomics are needed.
// W scores go straight to the score rows. Running maxima over W and M per
// head are folded into the head state whenever the block moves to another
// (sequence, KV head) and at its end.
template <int G>
__global__ __launch_bounds__(kScanThreads) void scan_kernel(Params p) {
  __shared__ uint32_t st_key[kStage];
  __shared__ uint32_t st_nh[kStage];  // position | head << 27
  __shared__ uint32_t s_fill;
  __shared__ uint32_t s_lo[G];
  __shared__ uint32_t s_cnt[G];
  __shared__ uint32_t s_base[G];  // first slot the burst reserved in each head's list (page split)
  __shared__ uint32_t lmax[G][2];     // max key over W, over M

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const Lane<G> L;
  if (tid == 0) s_fill = 0;
  if (tid < G) s_cnt[tid] = 0;
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
  int cur_b = -1, cur_g = -1;
  uint4 qreg[G];
  for (int64_t x = X0; x < X1; ++x) {
    const UnitRef ur = unit_at(p, x);
    const int b = ur.b, g = ur.g;
    const SeqGeom sg = seq_geom(p, b);
    const size_t bh0 = size_t(b) * p.H_q + size_t(g) * G;
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
      if (tid < G) s_lo[tid] = p.state[bh0 + tid].lo_key;
      load_q<G>(p, b, g, L, qreg);
    }
    __syncthreads();
    const uint32_t lo_f = s_lo[L.F];
    float* srow = p.scores + (bh0 + L.F) * p.n_cap;
    const size_t ubase = size_t(ur.u) * kUnit;
    uint64_t* crow = p.cand + (bh0 + L.F) * p.n_cap + ubase;
    // this block's pages of the unit
    const int pa = int(max<int64_t>(X0p - x * kUnitPages, 0));
    const int pe = int(min<int64_t>(min<int64_t>(X1p - x * kUnitPages, kUnitPages), ur.npages));
    // the physical pages of this wave's pages of the unit, read up front
    // (lane k holds the page of the wave's k-th page)
    const int my_pg = L.lane < kUnitPages / kScanWaves && pa + wave + kScanWaves * L.lane < pe
                          ? page_of(p, b, ur.u * kUnitPages + pa + wave + kScanWaves * L.lane)
                          : 0;
    for (int jj = pa + wave; jj < pe; jj += kScanWaves) {
      const int j = ur.u * kUnitPages + jj;
      float z[G];
      page_scores<G>(p, __shfl(my_pg, (jj - pa - wave) / kScanWaves), g, L, qreg, z);
#pragma unroll
      for (int s = 0; s < G; ++s) {
        const int n = j * kPage + L.tok(s);
        const uint32_t key = f2key(z[s]);
        const bool in_m = n >= sg.lo && n < sg.hi;
        const bool in_w = !in_m && n < sg.N;
        if (in_w) {
          if (RA_IN(n < p.n_cap, p, 2)) srow[n] = z[s];
          mw = max(mw, key);
        }
        if (in_m) mm = max(mm, key);
        const bool cand = in_m && key >= lo_f;
        const uint64_t cm = __ballot(cand);
        if (cm) {
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
                                          : atomicAdd(&s_cnt[L.F], 1u);
              if (RA_IN(slot < uint32_t(kUnit), p, 1))
                crow[slot] = (uint64_t(key) << 32) | uint32_t(n);
            }
          }
        }
      }
    }
    __syncthreads();
    // burst the staged candidates into the (head, unit) lists; streaming
    // stores, since cached writes interleaved with the K stream cost it
    // about twice as much time
    const uint32_t nst = min(s_fill, uint32_t(kStage));
    if (split) {
      if (tid < G) {
        s_base[tid] = s_cnt[tid] ? atomicAdd(&p.ucnt[(bh0 + tid) * p.n_units + ur.u], s_cnt[tid]) : 0u;
        s_cnt[tid] = 0;
      }
      __syncthreads();
    }
    for (uint32_t i = tid; i < nst; i += kScanThreads) {
      const uint32_t nh = st_nh[i];
      const uint32_t hh = nh >> 27;
      const uint32_t slot = (split ? s_base[hh] : 0u) + atomicAdd(&s_cnt[hh], 1u);
      if (RA_IN(slot < uint32_t(kUnit), p, 0))
        __builtin_nontemporal_store((uint64_t(st_key[i]) << 32) | (nh & ((1u << 27) - 1u)),
                                    &p.cand[(bh0 + hh) * p.n_cap + ubase + slot]);
    }
    __syncthreads();
    if (tid < G) {
      if (!split) p.ucnt[(bh0 + tid) * p.n_units + ur.u] = s_cnt[tid];
      s_cnt[tid] = 0;
    }
    if (tid == 0) s_fill = 0;
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
