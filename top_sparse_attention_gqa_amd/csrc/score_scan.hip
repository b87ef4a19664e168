// Exact scores of every cached key for every query head of its GQA group,
// z = q . k / sqrt(128) (RetrievalAttention slides, "Sparse attention
// renormalizes selected tokens", Eq. (1)), streamed once from HBM.
//
// Mapping on gfx950 (wave64): a wave reads a (page, KV head) block of 64 keys
// as 16 fully coalesced 1 KiB loads; in each load lane l holds 16 bytes
// (8 dims) of key (l / 16). Each lane keeps the same 8 dims of all G query
// heads of the group in registers and forms 8-term partial dot products with
// v_dot2_f32_bf16 (bf16 products are exact in fp32, fp32 accumulation). The
// 16 partials of a key are then summed across the 16-lane row with a
// reduce-scatter over DPP row permutations (mirror, half-mirror, two quad
// swaps): every step halves the number of heads a lane carries, so G heads
// cost G - 1 + 4 - log2(G) DPP adds instead of 4 G. The query slots are
// loaded in a lane-dependent order so that no selects are needed.
//
// HBM writes interleaved with this read stream cost far more than their
// bytes, so the scan does not store the score rows. A sampling pass first
// scores one page in S and histograms the sample; from it every head gets a
// conservative threshold such that, with a wide statistical margin, more
// than k_eff members of M score at or above it. The scan then keeps only
// those candidates, staged in LDS and written in bursts (every <= 64 pages)
// to per-(head, tile) lists, plus the scores of the static set W. The
// selection checks the margin exactly (it needs at least k_eff candidates);
// heads that fail it are rescanned with every member of M as a candidate.
#include "ra_internal.h"

namespace ra {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kScanThreads = 512;
constexpr int kScanWaves = kScanThreads / 64;
constexpr int kStage = 6144;       // LDS candidate staging entries per block
constexpr int kFlushPages = 64;    // pages between flushes: at most 2 tiles
constexpr float kInvSqrtD = 0.08838834764831845f;  // 1 / sqrt(128)

template <int G>
struct ScanCfg {
  static constexpr int HB = G <= 4 ? 12 : 11;  // histogram digit bits
  static constexpr int SHIFT = 32 - HB;
  static constexpr int NC = 1 << (HB - 6);     // coarse bins of 64 fine bins
  static constexpr int D = 16 / G;             // lanes of a row sharing a head
};

// Head whose full dot product lane r (0..15 within its row) holds after the
// reduce-scatter. F is linear over GF(2) with F(15) = G/2, F(7) = G/4,
// F(3) = G/8, F(1) = G/16 (0 where fractional): exactly what makes the
// partner of every step carry the same head in the slot being added.
template <int G>
__device__ __forceinline__ int head_of_lane(int r) {
  if constexpr (G == 1) {
    return 0;
  } else if constexpr (G == 2) {
    return (r >> 3) & 1;
  } else if constexpr (G == 4) {
    return ((r >> 2) & 1) ^ (((r >> 3) & 1) * 3);
  } else {
    return ((r >> 1) & 1) ^ (((r >> 2) & 1) * 3) ^ (((r >> 3) & 1) * 6);
  }
}

// DPP row permutations used by the reduce-scatter (partner lane r ^ mask).
constexpr int kDppMirror = 0x140;      // r ^ 15
constexpr int kDppHalfMirror = 0x141;  // r ^ 7
constexpr int kDppQuadXor3 = 0x1B;     // quad_perm [3,2,1,0]: r ^ 3
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]: r ^ 1

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                         0xF, 0xF, false));
}

// v[s] holds this lane's partial for head s ^ F(r). Returns the full sum
// over the 16 lanes of the row for head F(r).
template <int G>
__device__ __forceinline__ float reduce16(float (&v)[G]) {
  if constexpr (G >= 2) {
#pragma unroll
    for (int j = 0; j < G / 2; ++j) v[j] += dpp<kDppMirror>(v[G / 2 + j]);
  } else {
    v[0] += dpp<kDppMirror>(v[0]);
  }
  if constexpr (G >= 4) {
#pragma unroll
    for (int j = 0; j < G / 4; ++j) v[j] += dpp<kDppHalfMirror>(v[G / 4 + j]);
  } else {
    v[0] += dpp<kDppHalfMirror>(v[0]);
  }
  if constexpr (G >= 8) {
    v[0] += dpp<kDppQuadXor3>(v[1]);
  } else {
    v[0] += dpp<kDppQuadXor3>(v[0]);
  }
  v[0] += dpp<kDppQuadXor1>(v[0]);
  return v[0];
}

__device__ __forceinline__ float dot8(const uint4& k, const uint4& q) {
  float acc = __builtin_amdgcn_fdot2_f32_bf16(
      __builtin_bit_cast(bf16x2_t, k.x), __builtin_bit_cast(bf16x2_t, q.x),
      0.0f, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.y),
                                        __builtin_bit_cast(bf16x2_t, q.y), acc,
                                        false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.z),
                                        __builtin_bit_cast(bf16x2_t, q.z), acc,
                                        false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.w),
                                        __builtin_bit_cast(bf16x2_t, q.w), acc,
                                        false);
  return acc;
}

// The lane's view of one scan: row/lane position, its head F and its turn
// among the D lanes that carry the same head.
template <int G>
struct Lane {
  int lane, row, r, F, qsel;
  __device__ __forceinline__ Lane() {
    lane = lane_id();
    row = lane >> 4;
    r = lane & 15;
    F = head_of_lane<G>(r);
    qsel = r & (ScanCfg<G>::D - 1);
  }
  // position within the page of slot s
  __device__ __forceinline__ int tok(int s) const {
    return 4 * (s * ScanCfg<G>::D + qsel) + row;
  }
};

// This lane's 8 dims of the group's G query heads, slot s = head s ^ F.
template <int G>
__device__ __forceinline__ void load_q(const Params& p, int b, int g, const Lane<G>& L,
                                       uint4 (&qreg)[G]) {
  const uint16_t* qb = p.q + (size_t(b) * p.H_q + size_t(g) * G) * kHeadDim;
#pragma unroll
  for (int s = 0; s < G; ++s)
    qreg[s] = *reinterpret_cast<const uint4*>(qb + size_t(s ^ L.F) * kHeadDim + L.r * 8);
}

// Scores of one (page, KV head) block: after the call z[s] is the score of
// head F at position L.tok(s) of the page. K is streamed (nontemporal).
template <int G>
__device__ __forceinline__ void page_scores(const Params& p, int pg, int g, const Lane<G>& L,
                                            const uint4 (&qreg)[G], float (&z)[G]) {
  const uint4* kb = reinterpret_cast<const uint4*>(
      p.k_pool + (size_t(pg) * p.H_kv + g) * (kPage * kHeadDim));
  uint4 kd[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const u32x4_t t = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4_t*>(kb + (i * 4 + L.row) * 16 + L.r));
    kd[i] = make_uint4(t.x, t.y, t.z, t.w);
  }
#pragma unroll
  for (int s = 0; s < G; ++s) z[s] = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float v[G];
#pragma unroll
    for (int s = 0; s < G; ++s) v[s] = dot8(kd[i], qreg[s]);
    const float x = reduce16<G>(v);
    // after load i, lane (row, r) holds key 4 i + row for head F; the D
    // lanes sharing F take turns keeping it
    if ((i % ScanCfg<G>::D) == L.qsel) z[i / ScanCfg<G>::D] = x * kInvSqrtD;
  }
}

// A run of pages of one (sequence, KV head) inside a block's range of the
// linear page index L over (b, g, page), page fastest.
struct Segment {
  int b, g, j0, npages;
  int64_t end;
};

__device__ __forceinline__ Segment segment_at(const Params& p, int64_t L, int64_t L1) {
  // the largest b with seq_off[b] <= L (it has at least one page)
  int blo = 0, bhi = p.B - 1;
  while (blo < bhi) {
    const int mid = (blo + bhi + 1) >> 1;
    if (p.seq_off[mid] <= L) blo = mid; else bhi = mid - 1;
  }
  Segment s;
  s.b = blo;
  const int P = (seq_geom(p, blo).N + kPage - 1) / kPage;
  const int64_t rel = L - p.seq_off[blo];
  s.g = int(rel / P);
  s.j0 = int(rel - int64_t(s.g) * P);
  s.end = min(L1, p.seq_off[blo] + int64_t(s.g + 1) * P);
  s.npages = int(s.end - L);
  return s;
}

// Flush an LDS histogram [G][NC][65] into the global per-head histograms of
// group (b, g), one atomic per non-empty bin, and clear it.
template <int G>
__device__ __forceinline__ void flush_hist(uint32_t* lhist, uint32_t* gbase, const Params& p,
                                           int b, int g) {
  using C = ScanCfg<G>;
  const int tid = threadIdx.x;
  if (tid < G * C::NC) {
    const int hh = tid / C::NC;
    const int c = tid - hh * C::NC;
    uint32_t* rowp = lhist + (hh * C::NC + c) * 65;
    uint32_t* gh = gbase + (size_t(b) * p.H_q + size_t(g) * G + hh) * kHistStride;
    uint32_t sum = 0;
    for (int i = 0; i < 64; ++i) {
      const uint32_t v = rowp[i];
      if (v) {
        atomicAdd(&gh[c * 64 + i], v);
        sum += v;
        rowp[i] = 0;
      }
    }
    if (sum) atomicAdd(&gh[kFineBins + c], sum);
  }
}

// ---------------------------------------------------------------- sample stride
// Sample stride S = 2^s: at least kSampleMinPages pages of a (b, g) are
// scored, at most one in 2^kSampleMaxLog2. Short sequences are scored whole,
// which makes their threshold exact. Page j is sampled iff j % S == S / 2.
__device__ __forceinline__ int sample_log2(int P) {
  int s = 0;
  while (s < kSampleMaxLog2 && (P >> (s + 1)) >= kSampleMinPages) ++s;
  return s;
}

__device__ __forceinline__ int sampled_pages(int P) {
  const int S = 1 << sample_log2(P);
  const int half = S >> 1;
  return P > half ? (P - half + S - 1) / S : 0;
}

// ---------------------------------------------------------------- prep
// Clears the sample histograms, per-head state, group flags and candidate
// counts, and writes the prefixes
//   seq_off[b]  = sum_{b' < b} H_kv * pages(b')          (scan)
//   samp_off[b] = sum_{b' < b} H_kv * sampled_pages(b')  (sample)
// that map a linear page index to (sequence, KV head, page).
__global__ __launch_bounds__(1024) void prep_kernel(Params p) {
  const size_t heads = size_t(p.B) * p.H_q;
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  const size_t t0 = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const size_t n4 = heads * kHistStride / 4;
  uint4* h4 = reinterpret_cast<uint4*>(p.hist);
  for (size_t i = t0; i < n4; i += stride) h4[i] = make_uint4(0, 0, 0, 0);
  for (size_t i = t0; i < heads * size_t(p.n_tiles); i += stride) p.tcnt[i] = 0;
  for (size_t i = t0; i < heads; i += stride) {
    HeadState& st = p.state[i];
    st.lo_key = 0;
    st.max_w = 0;
    st.max_m = 0;
    st.dense = 0;
    st.thr_shift = 64;  // nothing passes an unset threshold
    st.thr_lo = 0xFFFFFFFFu;
    st.thr_hi = 0xFFFFFFFFu;
  }
  for (size_t i = t0; i < size_t(p.B) * p.H_kv; i += stride) p.gflag[i] = 0;
  if (t0 == 0) *p.any_dense = 0;
  if (blockIdx.x != 0) return;
  __shared__ int64_t tmp[16];
  const int per = (p.B + int(blockDim.x) - 1) / int(blockDim.x);
  int64_t s = 0, ss = 0;
  for (int i = 0; i < per; ++i) {
    const int b = threadIdx.x * per + i;
    if (b < p.B) {
      const int P = (seq_geom(p, b).N + kPage - 1) / kPage;
      s += int64_t(p.H_kv) * P;
      ss += int64_t(p.H_kv) * sampled_pages(P);
    }
  }
  int64_t total, stotal;
  int64_t run = block_excl_scan(s, tmp, &total);
  int64_t srun = block_excl_scan(ss, tmp, &stotal);
  for (int i = 0; i < per; ++i) {
    const int b = threadIdx.x * per + i;
    if (b < p.B) {
      const int P = (seq_geom(p, b).N + kPage - 1) / kPage;
      p.seq_off[b] = run;
      p.samp_off[b] = srun;
      run += int64_t(p.H_kv) * P;
      srun += int64_t(p.H_kv) * sampled_pages(P);
    }
  }
  if (threadIdx.x == 0) {
    p.seq_off[p.B] = total;
    p.samp_off[p.B] = stotal;
  }
}

hipError_t launch_prep(const Params& p, hipStream_t s) {
  hipLaunchKernelGGL(prep_kernel, dim3(unsigned(2 * (p.num_cus > 0 ? p.num_cus : 256))), dim3(1024),
                     0, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------- sample
// Persistent over the linear index of sampled pages (same (b, g, page)
// order as the scan): each block takes one contiguous range, histograms the
// scores of M per head in LDS and adds them to the global sample histogram
// at the end of every (b, g) run.
template <int G>
__global__ __launch_bounds__(kScanThreads) void sample_kernel(Params p) {
  using C = ScanCfg<G>;
  __shared__ uint32_t lhist[G * C::NC * 65];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const Lane<G> L;
  for (int i = tid; i < G * C::NC * 65; i += kScanThreads) lhist[i] = 0;

  const int64_t T = p.samp_off[p.B];
  const int64_t L0 = T * blockIdx.x / gridDim.x;
  const int64_t L1 = T * (blockIdx.x + 1) / gridDim.x;
  for (int64_t Lx = L0; Lx < L1;) {
    // the largest b with samp_off[b] <= Lx (it has at least one sampled page)
    int blo = 0, bhi = p.B - 1;
    while (blo < bhi) {
      const int mid = (blo + bhi + 1) >> 1;
      if (p.samp_off[mid] <= Lx) blo = mid; else bhi = mid - 1;
    }
    const int b = blo;
    const SeqGeom sg = seq_geom(p, b);
    const int P = (sg.N + kPage - 1) / kPage;
    const int S = 1 << sample_log2(P);
    const int half = S >> 1;
    const int ns = sampled_pages(P);
    const int64_t rel = Lx - p.samp_off[b];
    const int g = int(rel / ns);
    const int t0 = int(rel - int64_t(g) * ns);
    const int64_t end = min(L1, p.samp_off[b] + int64_t(g + 1) * ns);
    const int n = int(end - Lx);
    uint4 qreg[G];
    load_q<G>(p, b, g, L, qreg);
    __syncthreads();
    uint32_t* lh = lhist + L.F * C::NC * 65;
    for (int t = t0 + wave; t < t0 + n; t += kScanWaves) {
      const int j = half + t * S;
      float z[G];
      page_scores<G>(p, page_of(p, b, j), g, L, qreg, z);
#pragma unroll
      for (int s = 0; s < G; ++s) {
        const int pos = j * kPage + L.tok(s);
        if (pos >= sg.lo && pos < sg.hi) {
          const uint32_t dg = f2key(z[s]) >> C::SHIFT;
          atomicAdd(&lh[dg + (dg >> 6)], 1u);
        }
      }
    }
    __syncthreads();
    flush_hist<G>(lhist, p.hist, p, b, g);
    __syncthreads();
    Lx = end;
  }
}

hipError_t launch_sample(const Params& p, hipStream_t s) {
  const int64_t pages_max =
      int64_t(p.B) * p.H_kv * ((int64_t(p.max_seq_len) + kPage - 1) / kPage);
  int64_t blocks = (pages_max + 8 * kScanWaves - 1) / (8 * kScanWaves);
  const int64_t cap = p.num_cus > 0 ? p.num_cus : 256;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  const dim3 grid{unsigned(blocks)}, block{unsigned(kScanThreads)};
  switch (p.G) {
    case 1: hipLaunchKernelGGL(sample_kernel<1>, grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL(sample_kernel<2>, grid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL(sample_kernel<4>, grid, block, 0, s, p); break;
    case 8: hipLaunchKernelGGL(sample_kernel<8>, grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- threshold
// Candidate threshold of one head from its sample histogram (run by one
// wave; returns the same key in every lane). With the sample a fraction
// 1/r of M, the threshold is placed where the sample count from the top
// reaches 1.2 k_eff / r + 5 sqrt(k_eff / r) + 8, interpolating linearly
// inside the fine bucket; the expected population above it is then at least
// 1.2 k_eff with a margin of five standard deviations of the sample count.
// A sample that covers all of M gives the exact bucket's lower edge; k_eff
// = 0 gives a threshold no finite score reaches.
__device__ uint32_t candidate_threshold(const Params& p, int bh, const SeqGeom& sg) {
  const int lane = lane_id();
  if (sg.k_eff == 0) return 0xFFFFFFFFu;
  const int HB = hist_bits(p.G);
  const int NC = 1 << (HB - 6);
  const uint32_t* gh = p.hist + size_t(bh) * kHistStride;
  const uint32_t c = lane < NC ? gh[kFineBins + lane] : 0u;
  const uint32_t suf = wave_suffix_sum(c);
  const uint32_t m_s = __shfl(suf, 0);
  const uint32_t m_all = uint32_t(sg.hi - sg.lo);
  if (m_s == 0) return 0u;
  const bool exact = m_s >= m_all;
  float target;
  if (exact) {
    target = float(sg.k_eff);
  } else {
    const float kr = float(sg.k_eff) * float(m_s) / float(m_all);
    target = 1.2f * kr + 5.0f * sqrtf(kr) + 8.0f;
  }
  if (target >= float(m_s)) return 0u;  // keep every member of M
  const uint64_t mc = __ballot(float(suf) >= target);
  const int cs = mc ? 63 - __clzll(mc) : 0;
  const uint32_t above_c = __shfl(suf - c, cs);
  const uint32_t f = gh[cs * 64 + lane];
  const uint32_t fsuf = wave_suffix_sum(f) + above_c;
  const uint64_t mf = __ballot(float(fsuf) >= target);
  const int fl = mf ? 63 - __clzll(mf) : 0;
  const uint32_t d = uint32_t(cs * 64 + fl);
  const uint32_t above = __shfl(fsuf - f, fl);
  const uint32_t cnt = __shfl(f, fl);
  const int shift = 32 - HB;
  const uint32_t lo_edge = d << shift;
  if (exact || cnt == 0) return lo_edge;
  // keys of bucket d span [d << shift, (d + 1) << shift)
  const float frac = fminf(1.0f, (target - float(above)) / float(cnt));
  const uint32_t width = 1u << shift;
  const uint32_t back = uint32_t(frac * float(width));
  const uint64_t top = (uint64_t(d) + 1) << shift;
  const uint64_t key = top - (back >= width ? width : back);
  return uint32_t(key > lo_edge ? key : lo_edge);
}

// ---------------------------------------------------------------- scan
// Persistent over the linear page index: each block takes one contiguous
// range and works through it as segments of one (b, g), flushing its LDS
// candidate staging every kFlushPages pages (such a run spans at most two
// tiles, so one reservation per (head, tile) suffices).
template <int G>
__global__ __launch_bounds__(kScanThreads) void scan_kernel(Params p) {
  __shared__ uint32_t st_key[kStage];
  __shared__ uint32_t st_nh[kStage];  // position | head << 27
  __shared__ uint32_t s_fill;
  __shared__ uint32_t s_lo[G];
  __shared__ uint32_t lmax[G][2];     // max key over W, over M
  __shared__ uint32_t s_cnt[G][2], s_base[G][2];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const Lane<G> L;
  if (tid == 0) s_fill = 0;
  if (tid < 2 * G) lmax[tid >> 1][tid & 1] = 0u;
  __syncthreads();

  const int64_t T = p.seq_off[p.B];
  const int64_t L0 = T * blockIdx.x / gridDim.x;
  const int64_t L1 = T * (blockIdx.x + 1) / gridDim.x;
  for (int64_t Lx = L0; Lx < L1;) {
    const Segment seg = segment_at(p, Lx, L1);
    const int b = seg.b, g = seg.g;
    const SeqGeom sg = seq_geom(p, b);
    const size_t bh0 = size_t(b) * p.H_q + size_t(g) * G;
    if (wave < G) {
      const uint32_t lo = candidate_threshold(p, int(bh0) + wave, sg);
      if (L.lane == 0) {
        s_lo[wave] = lo;
        if (seg.j0 == 0) p.state[bh0 + wave].lo_key = lo;
      }
    }
    uint4 qreg[G];
    load_q<G>(p, b, g, L, qreg);
    __syncthreads();
    const uint32_t lo_f = s_lo[L.F];
    float* srow = p.scores + (bh0 + L.F) * p.n_cap;
    uint64_t* crow = p.cand + (bh0 + L.F) * p.n_cap;
    uint32_t* trow = p.tcnt + (bh0 + L.F) * p.n_tiles;
    uint32_t mw = 0u, mm = 0u;  // running max keys of head F over W and M

    for (int sub0 = 0; sub0 < seg.npages; sub0 += kFlushPages) {
      const int subn = min(kFlushPages, seg.npages - sub0);
      const int tile0 = ((seg.j0 + sub0) * kPage) / kTile;
      for (int jj = wave; jj < subn; jj += kScanWaves) {
        const int j = seg.j0 + sub0 + jj;
        float z[G];
        page_scores<G>(p, page_of(p, b, j), g, L, qreg, z);
#pragma unroll
        for (int s = 0; s < G; ++s) {
          const int n = j * kPage + L.tok(s);
          const uint32_t key = f2key(z[s]);
          const bool in_m = n >= sg.lo && n < sg.hi;
          const bool in_w = !in_m && n < sg.N;
          if (in_w) {
            srow[n] = z[s];
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
              } else {
                // staging full: append straight to the (head, tile) list
                const int t = n / kTile;
                const uint32_t gi = atomicAdd(&trow[t], 1u);
                crow[size_t(t) * kTile + gi] = (uint64_t(key) << 32) | uint32_t(n);
              }
            }
          }
        }
      }
      if (tid < 2 * G) s_cnt[tid >> 1][tid & 1] = 0;
      __syncthreads();
      // burst the staged candidates into the per-(head, tile) lists
      const uint32_t nst = min(s_fill, uint32_t(kStage));
      for (uint32_t i = tid; i < nst; i += kScanThreads) {
        const uint32_t nh = st_nh[i];
        const int n = int(nh & ((1u << 27) - 1u));
        atomicAdd(&s_cnt[nh >> 27][n / kTile - tile0], 1u);
      }
      __syncthreads();
      if (tid < 2 * G) {
        const int hh = tid >> 1, ts = tid & 1;
        const uint32_t c = s_cnt[hh][ts];
        s_base[hh][ts] = c ? atomicAdd(&p.tcnt[(bh0 + hh) * p.n_tiles + tile0 + ts], c) : 0u;
        s_cnt[hh][ts] = 0;
      }
      __syncthreads();
      for (uint32_t i = tid; i < nst; i += kScanThreads) {
        const uint32_t nh = st_nh[i];
        const uint32_t hh = nh >> 27;
        const int n = int(nh & ((1u << 27) - 1u));
        const int t = n / kTile;
        const uint32_t gi = s_base[hh][t - tile0] + atomicAdd(&s_cnt[hh][t - tile0], 1u);
        p.cand[(bh0 + hh) * p.n_cap + size_t(t) * kTile + gi] = (uint64_t(st_key[i]) << 32) | uint32_t(n);
      }
      __syncthreads();
      if (tid == 0) s_fill = 0;
      __syncthreads();
    }
    // maxima: reduce over the lanes that carry the same head, then LDS
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
      if (v) atomicMax((tid & 1) ? &p.state[bh0 + hh].max_m : &p.state[bh0 + hh].max_w, v);
      lmax[hh][tid & 1] = 0u;
    }
    __syncthreads();
    Lx = seg.end;
  }
}

static unsigned scan_blocks(const Params& p) {
  const int64_t pages_max =
      int64_t(p.B) * p.H_kv * ((int64_t(p.max_seq_len) + kPage - 1) / kPage);
  int64_t blocks = (pages_max + kScanWaves - 1) / kScanWaves;
  const int64_t cap = int64_t(2) * (p.num_cus > 0 ? p.num_cus : 256);
  if (blocks > cap) blocks = cap;
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

// ---------------------------------------------------------------- rescan
// For groups with a head whose candidates fell short: every member of M of
// those heads becomes a candidate, written at its place in the tile list
// (the list of tile t holds positions max(t * kTile, lo) .. in order).
// Blocks skip unflagged segments, so without flags nothing is read.
template <int G>
__global__ __launch_bounds__(kScanThreads) void dense_scan_kernel(Params p) {
  if (*p.any_dense == 0u) return;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const Lane<G> L;
  const int64_t T = p.seq_off[p.B];
  const int64_t L0 = T * blockIdx.x / gridDim.x;
  const int64_t L1 = T * (blockIdx.x + 1) / gridDim.x;
  for (int64_t Lx = L0; Lx < L1;) {
    const Segment seg = segment_at(p, Lx, L1);
    Lx = seg.end;
    const int b = seg.b, g = seg.g;
    if (!p.gflag[size_t(b) * p.H_kv + g]) continue;
    const SeqGeom sg = seq_geom(p, b);
    const size_t bh = size_t(b) * p.H_q + size_t(g) * G + L.F;
    const bool mine = p.state[bh].dense != 0u;
    uint4 qreg[G];
    load_q<G>(p, b, g, L, qreg);
    uint64_t* crow = p.cand + bh * p.n_cap;
    for (int jj = wave; jj < seg.npages; jj += kScanWaves) {
      const int j = seg.j0 + jj;
      float z[G];
      page_scores<G>(p, page_of(p, b, j), g, L, qreg, z);
#pragma unroll
      for (int s = 0; s < G; ++s) {
        const int n = j * kPage + L.tok(s);
        if (mine && n >= sg.lo && n < sg.hi) {
          const int t0 = (n / kTile) * kTile;
          crow[size_t(t0) + (n - max(t0, sg.lo))] = (uint64_t(f2key(z[s])) << 32) | uint32_t(n);
        }
      }
    }
  }
}

hipError_t launch_dense_scan(const Params& p, hipStream_t s) {
  const dim3 grid{scan_blocks(p)}, block{unsigned(kScanThreads)};
  switch (p.G) {
    case 1: hipLaunchKernelGGL(dense_scan_kernel<1>, grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL(dense_scan_kernel<2>, grid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL(dense_scan_kernel<4>, grid, block, 0, s, p); break;
    case 8: hipLaunchKernelGGL(dense_scan_kernel<8>, grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ra
