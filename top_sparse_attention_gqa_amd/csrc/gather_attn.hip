// Softmax . V over W u Omega_h as split-K partials, then their log-sum-exp
// merge (RetrievalAttention slides, "Sparse attention renormalizes selected
// tokens", Eq. (2); "Two local softmax outputs need global weights",
// Eqs. (3)-(5); backup frame "the normalization identity": merging disjoint
// partials gives the exact softmax over their union).
//
// The attended set of head h is split into disjoint parts, one partial per
// tile of 8192 positions (two units): the tile's retrieved positions, plus a
// slice of the static set W (W's rows are dealt out evenly over the
// sequence's tiles, so every block has about the same work). Every partial
// of a head uses the same reference m (its largest score over W u Omega,
// which the scan records), so none can overflow: Z = sum e^{z - m},
// N = sum e^{z - m} v.
//
// gather, one block per (sequence, KV head, tile): the block takes each
// head's retrieved members of its tile (the entries of the tile's
// (head, unit) candidate lists at or above the head's exact threshold),
// marks them in an LDS bitmap, stages their scores in LDS, and writes their
// positions, ascending, with their count, over the tile's consumed lists.
// (Scattered 4-byte score stores into the score rows cost several times
// their bytes, so they happen only when the caller keeps the scores, or
// when the tile's lists overflow the staging and the scores are read back.)
// Its rows are the union over the group's G query heads of those positions,
// in ascending order, then its slice of W (attended by every head; the scan
// left those scores). Each V row (256 contiguous bytes) is read once per
// group: the weights e^{z - m} of every (row, head) are put in LDS (the
// retrieved scores from the staging, the W scores loaded up front), then a
// V phase accumulates Z and N for every member head.
//
// merge: per query head, one block combines the partials,
// out = sum_t e^{m_t - m} N_t / sum_t e^{m_t - m} Z_t, lse = m + ln(...),
// and pads out_idx with -1 after k_eff; further blocks each copy the
// retrieved positions of up to kMergeTiles tiles into out_idx at the
// offset the counts of the tiles before them give.
#include "ra_internal.h"

namespace ra {

constexpr int kGathThreads = 256;
constexpr int kGathWaves = kGathThreads / 64;
constexpr int kChunk = 512;    // rows listed in LDS at a time
constexpr int kListBatch = 8;  // list entries per lane in flight
constexpr int kSpec = 64;      // entries per candidate list read up front
constexpr int kSel = 2048;     // retrieved entries of a tile staged in LDS
constexpr uint32_t kPosMask = (1u << 24) - 1u;  // row = position | heads << 24
constexpr int kWPre = 64;      // W-slice rows whose pages the prologue loads

__device__ __forceinline__ float bf16lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }

// Per-head popcounts packed four heads per 64-bit word (16-bit fields: a
// tile holds at most 8192 positions), so one block scan ranks them all.
template <int G>
struct PackedCounts {
  static constexpr int kWords = (G + 3) / 4;
  int64_t v[kWords];
};

// V phase for rows [0, cnt) of a chunk: s_row (position | member heads << 24),
// s_rpg (physical page) and s_w (weight e^{z - m} of (row, head), 0 if the
// head does not attend the row) are in LDS. Adds the rows' contribution to
// acc (this lane's 8 dims, for the 4 rows its 16-lane group covers) and to
// zs (lane r == 0 of each group sums the weights of its rows). Block-wide.
template <int G>
__device__ __forceinline__ void accumulate_rows(const Params& p, int g, int cnt,
                                                const uint32_t* s_row, const int32_t* s_rpg,
                                                const float (*s_w)[G], float (&acc)[G][8],
                                                float (&zs)[G]) {
  constexpr int kVRows = G <= 4 ? 8 : 4;  // V rows per lane in flight
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int row = lane >> 4;
  const int r = lane & 15;
  // 4 rows per wave step, 16 lanes x 8 dims per V row
  const size_t vpage = size_t(p.H_kv) * kPage * kHeadDim;
  const uint16_t* vbase = p.v_pool + size_t(g) * kPage * kHeadDim + r * 8;
  for (int i0 = wave * 4 + row; i0 < cnt; i0 += kGathWaves * 4 * kVRows) {
    uint4 v[kVRows];
#pragma unroll
    for (int u = 0; u < kVRows; ++u) {
      const int i = i0 + u * kGathWaves * 4;
      v[u] = make_uint4(0u, 0u, 0u, 0u);
      if (i < cnt) {
        const uint32_t pos = s_row[i] & kPosMask;
        v[u] = *reinterpret_cast<const uint4*>(vbase + size_t(s_rpg[i]) * vpage +
                                               size_t(pos & 63u) * kHeadDim);
      }
    }
#pragma unroll
    for (int u = 0; u < kVRows; ++u) {
      const int i = i0 + u * kGathWaves * 4;
      if (i >= cnt) break;
      const float vf[8] = {bf16lo(v[u].x), bf16hi(v[u].x), bf16lo(v[u].y), bf16hi(v[u].y),
                           bf16lo(v[u].z), bf16hi(v[u].z), bf16lo(v[u].w), bf16hi(v[u].w)};
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float w = s_w[i][hh];
        if (r == 0) zs[hh] += w;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hh][e] += w * vf[e];
      }
    }
  }
}

template <int G, int UPT>
__global__ __launch_bounds__(kGathThreads) __attribute__((amdgpu_waves_per_eu(4)))
void gather_kernel(Params p) {
  // a tile of UPT units: UPT * 4096 positions, one bitmap word per page
  constexpr int kTileT = UPT * kUnit;
  constexpr int kWordsT = kTileT / 64;
  // the prologue deals its loads to thread ranges: page numbers (one per
  // word), then the list lengths from kWordsT, the head states from
  // kWordsT + 32, the W-slice pages in the last kWPre threads
  static_assert(UPT * G <= 32, "list lengths fit their 32 threads");
  static_assert(kWordsT + 32 + G <= kGathThreads - kWPre, "prologue thread ranges overlap");
  // staged entries pack the tile offset in 13 bits, per-head counts in 16
  static_assert(kTileT <= 8192, "tile offsets fit 13 bits");
  const int tile = blockIdx.y;
  const int bg = blockIdx.x;
  const int b = bg / p.H_kv;
  const int g = bg - b * p.H_kv;
  const SeqGeom sg = seq_geom(p, b);
  const size_t bh0 = size_t(b) * p.H_q + size_t(g) * G;
  const int t0 = tile * kTileT;
  if (t0 >= sg.N) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 15;
  constexpr int kCh = kChunk;
  constexpr int kLists = UPT * G;  // list j: head j / UPT
  constexpr int kSpecPer = (kLists * kSpec + kGathThreads - 1) / kGathThreads;
  constexpr int kWzPer = (kWPre * G + kGathThreads - 1) / kGathThreads;

  __shared__ uint64_t bm[G][kWordsT];
  __shared__ uint64_t s_uw[kWordsT];  // union of the heads' bitmaps
  __shared__ int32_t s_ex[kWordsT];   // union rows before each word
  __shared__ int32_t s_pg[kWordsT];
  __shared__ uint32_t s_row[kCh];
  __shared__ int32_t s_rpg[kCh];
  __shared__ float s_w[kCh][G];             // e^{z - m} of (row, head), 0 if absent
  // the staged retrieved entries (offset in tile | head << 13, and score)
  // share LDS with the final per-wave sums of N
  constexpr int kStageBytes = kSel * 8;
  constexpr int kAccBytes = kGathWaves * G * kHeadDim * 4;
  __shared__ __align__(16) unsigned char s_raw[kStageBytes > kAccBytes ? kStageBytes : kAccBytes];
  uint32_t* s_sel = reinterpret_cast<uint32_t*>(s_raw);
  float* s_selz = reinterpret_cast<float*>(s_raw + kSel * 4);
  float (*s_acc)[G][kHeadDim] = reinterpret_cast<float (*)[G][kHeadDim]>(s_raw);
  __shared__ uint32_t s_nsel;
  __shared__ float s_zs[kGathWaves][G];
  __shared__ int64_t s_tmp[16];
  __shared__ HeadState s_st[G];
  __shared__ float s_mref[G];
  __shared__ uint32_t s_lc[kLists];         // list j: head j / UPT,
  __shared__ uint32_t s_lpre[kLists + 1];   // unit UPT tile + j % UPT
  __shared__ int32_t s_wpg[kWPre];          // pages of the first rows of the W slice

  // this block's slice [w0, w1) of the rows of W = [0, lo) u [hi, N)
  const int nt = (sg.N + kTileT - 1) / kTileT;
  const int wsize = sg.lo + (sg.N - sg.hi);
  const int wper = (wsize + nt - 1) / nt;
  const int w0 = min(wsize, tile * wper);
  const int w1 = min(wsize, w0 + wper);
  auto w_pos = [&](int rr) { return rr < sg.lo ? rr : sg.hi + (rr - sg.lo); };

  // Every load the block can issue up front, in one round: page numbers,
  // list lengths, head states, the pages and scores of the W slice, and the
  // first kSpec entries of each of the 2 G candidate lists (read before
  // their lengths are known; entries past a list's end are dropped).
  const int units_seq = (sg.N + kUnit - 1) / kUnit;
  if (tid < kWordsT) {
    // a 64-bit word covers exactly one 64-token page
    s_pg[tid] = (t0 + tid * 64 < sg.N) ? page_of(p, b, (t0 >> 6) + tid) : 0;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) bm[hh][tid] = 0ull;
  } else if (tid < kWordsT + kLists) {
    const int j = tid - kWordsT;
    const int unit = UPT * tile + j % UPT;
    s_lc[j] = unit < units_seq ? p.ucnt[(bh0 + j / UPT) * p.n_units + unit] : 0u;
  } else if (tid >= kWordsT + 32 && tid < kWordsT + 32 + G) {
    const int hh = tid - kWordsT - 32;
    s_st[hh] = p.state[bh0 + hh];
  } else if (tid >= kGathThreads - kWPre) {
    const int i = tid - (kGathThreads - kWPre);
    if (w0 + i < w1) s_wpg[i] = page_of(p, b, w_pos(w0 + i) >> 6);
  }
  if (tid == 0) s_nsel = 0u;
  uint64_t spec[kSpecPer];
#pragma unroll
  for (int u = 0; u < kSpecPer; ++u) {
    const int e = u * kGathThreads + tid;
    const int j = e / kSpec, i = e - j * kSpec;
    const int unit = UPT * tile + j % UPT;
    spec[u] = (j < kLists && unit < units_seq &&
               RA_IN(size_t(unit) * kUnit + i < size_t(p.n_cap), p, 5))
                  ? p.cand[(bh0 + j / UPT) * p.n_cap + size_t(unit) * kUnit + i]
                  : 0ull;
  }
  float wz[kWzPer];  // score of W-slice row q / G for head q % G, q = u * 256 + tid
#pragma unroll
  for (int u = 0; u < kWzPer; ++u) {
    const int q = u * kGathThreads + tid;
    const int i = q / G;
    wz[u] = (i < kWPre && w0 + i < w1)
                ? p.scores[(bh0 + q % G) * p.n_cap + w_pos(w0 + i)]
                : 0.0f;
  }
  __syncthreads();
  if (tid < G) s_mref[tid] = softmax_ref(s_st[tid], sg.k_eff);
  if (tid < kLists && s_st[tid / UPT].dense != 0u) {
    // a rescanned head's lists hold every member of M at its place: their
    // lengths are the units' overlaps with M
    const int unit = UPT * tile + tid % UPT;
    const int ov = min((unit + 1) * kUnit, sg.hi) - max(unit * kUnit, sg.lo);
    s_lc[tid] = ov > 0 ? uint32_t(ov) : 0u;
  }
  __syncthreads();
  // when the tile's lists fit the LDS staging, the retrieved scores stay in
  // LDS; otherwise they go to the score rows and are read back
  uint32_t listed = 0;
#pragma unroll
  for (int j = 0; j < kLists; ++j) listed += s_lc[j];
  const bool staged = listed <= uint32_t(kSel);
  const bool store = p.keep_scores || !staged;

  // Each head's retrieved members of this tile: the list entries whose
  // composite (key - lo) << 32 | ~n clears the head's threshold. They are
  // marked in the bitmap and their scores staged in LDS (or stored).
  auto take = [&](int hh, uint64_t v) {
    const uint32_t key = uint32_t(v >> 32);
    const uint32_t n = uint32_t(v);
    const uint64_t comp = (uint64_t(key - s_st[hh].lo_key) << 32) | uint32_t(~n);
    const uint64_t thr = (uint64_t(s_st[hh].thr_hi) << 32) | s_st[hh].thr_lo;
    if ((comp >> s_st[hh].thr_shift) < thr) return;
    const int off = int(n) - t0;
    atomicOr(reinterpret_cast<unsigned long long*>(&bm[hh][off >> 6]), 1ull << (off & 63));
    const float z = key2f(key);
    if (store && RA_IN(n < uint32_t(p.n_cap), p, 7)) p.scores[(bh0 + hh) * p.n_cap + n] = z;
    if (staged) {
      const uint32_t at = atomicAdd(&s_nsel, 1u);
      s_sel[at] = uint32_t(off) | (uint32_t(hh) << 13);
      s_selz[at] = z;
    }
  };
#pragma unroll
  for (int u = 0; u < kSpecPer; ++u) {
    const int e = u * kGathThreads + tid;
    const int j = e / kSpec, i = e - j * kSpec;
    if (j < kLists && uint32_t(i) < s_lc[j] && s_st[j / UPT].thr_shift < 64u)
      take(j / UPT, spec[u]);
  }
  // the rest of the lists (past kSpec entries), as one index space
  if (tid == 0) {
    uint32_t run = 0;
    for (int j = 0; j < kLists; ++j) {
      s_lpre[j] = run;
      if (s_st[j / UPT].thr_shift < 64u && s_lc[j] > uint32_t(kSpec)) run += s_lc[j] - kSpec;
    }
    s_lpre[kLists] = run;
  }
  __syncthreads();
  const uint32_t rest = s_lpre[kLists];
  for (uint32_t base = 0; base < rest; base += kGathThreads * kListBatch) {
    uint64_t v[kListBatch];
    int jl[kListBatch];
#pragma unroll
    for (int u = 0; u < kListBatch; ++u) {
      const uint32_t i = base + u * kGathThreads + tid;
      v[u] = 0ull;
      jl[u] = -1;
      if (i < rest) {
        int j = 0;
        while (j + 1 < kLists && s_lpre[j + 1] <= i) ++j;
        jl[u] = j;
        const uint32_t e = kSpec + (i - s_lpre[j]);
        if (RA_IN(e < uint32_t(kUnit), p, 5))
          v[u] = p.cand[(bh0 + j / UPT) * p.n_cap +
                        size_t(UPT * tile + j % UPT) * kUnit + e];
      }
    }
#pragma unroll
    for (int u = 0; u < kListBatch; ++u)
      if (jl[u] >= 0) take(jl[u] / UPT, v[u]);
  }
  __syncthreads();

  // union over the group's heads, and each head's ranks
  uint64_t uw = 0;
  const int nw = t0 + tid * 64;
  PackedCounts<G> pc;
#pragma unroll
  for (int j = 0; j < PackedCounts<G>::kWords; ++j) pc.v[j] = 0;
  if (tid < kWordsT) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      uw |= bm[hh][tid];
      pc.v[hh >> 2] |= int64_t(__popcll(bm[hh][tid])) << (16 * (hh & 3));
    }
  }
  int64_t utotal;
  const int64_t ex = block_excl_scan(__popcll(uw), s_tmp, &utotal);
  PackedCounts<G> px, ptot;
#pragma unroll
  for (int j = 0; j < PackedCounts<G>::kWords; ++j)
    px.v[j] = block_excl_scan(pc.v[j], s_tmp, &ptot.v[j]);
  if (tid < kWordsT) {
    s_uw[tid] = uw;
    s_ex[tid] = int32_t(ex);
    // the tile's retrieved positions, ascending, replace its consumed lists
    // (the merge concatenates the tiles into out_idx)
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      uint64_t y = bm[hh][tid];
      uint32_t rank = uint32_t((px.v[hh >> 2] >> (16 * (hh & 3))) & 0xFFFF);
      int32_t* dst = reinterpret_cast<int32_t*>(p.cand + (bh0 + hh) * p.n_cap + size_t(t0));
      while (y) {
        const int bit = __ffsll((unsigned long long)y) - 1;
        y &= y - 1ull;
        if (RA_IN(rank < uint32_t(2 * kTileT), p, 6)) dst[rank] = nw + bit;
        ++rank;
      }
    }
  }
  if (tid < G)
    p.scnt[(bh0 + tid) * p.n_tiles + tile] =
        uint32_t((ptot.v[tid >> 2] >> (16 * (tid & 3))) & 0xFFFF);

  float acc[G][8], zs[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    zs[hh] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[hh][e] = 0.0f;
  }
  // rows: the union (U rows, ascending), then the W slice
  const int U = int(utotal);
  const int R = U + (w1 - w0);
  for (int cb = 0; cb < R; cb += kCh) {
    const int cnt = min(kCh, R - cb);
    // list this chunk of the rows in LDS, weights cleared
    if (tid < kWordsT && cb < U) {
      int pos = int(ex) - cb;
      uint64_t x = uw;
      while (x && pos < kCh) {
        const int bit = __ffsll((unsigned long long)x) - 1;
        x &= x - 1ull;
        if (pos >= 0) {
          uint32_t mem = 0;
#pragma unroll
          for (int hh = 0; hh < G; ++hh) mem |= uint32_t((bm[hh][tid] >> bit) & 1ull) << hh;
          s_row[pos] = uint32_t(nw + bit) | (mem << 24);
          s_rpg[pos] = s_pg[tid];
        }
        ++pos;
      }
    }
    const int cw0 = max(cb, U), cw1 = cb + cnt;
    for (int i = cw0 + tid; i < cw1; i += kGathThreads) {
      const int wi = i - U;  // row of the slice
      const int pos = w_pos(w0 + wi);
      s_row[i - cb] = uint32_t(pos) | (((1u << G) - 1u) << 24);
      s_rpg[i - cb] = wi < kWPre ? s_wpg[wi] : page_of(p, b, pos >> 6);
    }
    for (int i = tid; i < cnt * G; i += kGathThreads) (&s_w[0][0])[i] = 0.0f;
    __syncthreads();
    // weights of the retrieved rows in this chunk
    if (staged) {
      const uint32_t ns = s_nsel;
      for (uint32_t e = tid; e < ns; e += kGathThreads) {
        const uint32_t sv = s_sel[e];
        const int off = int(sv & 8191u), hh = int(sv >> 13);
        const int word = off >> 6, bit = off & 63;
        const int rr = s_ex[word] + __popcll(s_uw[word] & ((1ull << bit) - 1ull)) - cb;
        if (rr >= 0 && rr < cnt) s_w[rr][hh] = expf(s_selz[e] - s_mref[hh]);
      }
    } else {
      // too many retrieved rows to stage: read their scores back
      for (int q = tid; q < min(cnt, U - cb) * G; q += kGathThreads) {
        const int i = q / G, hh = q % G;
        const uint32_t e = s_row[i];
        if ((e >> (24 + hh)) & 1u)
          s_w[i][hh] = expf(p.scores[(bh0 + hh) * p.n_cap + (e & kPosMask)] - s_mref[hh]);
      }
    }
    // weights of the W rows in this chunk (every head)
#pragma unroll
    for (int u = 0; u < kWzPer; ++u) {
      const int q = u * kGathThreads + tid;
      const int i = U + q / G - cb;  // chunk row of slice row q / G
      if (q / G < kWPre && w0 + q / G < w1 && i >= 0 && i < cnt)
        s_w[i][q % G] = expf(wz[u] - s_mref[q % G]);
    }
    for (int i = max(cw0, U + kWPre) + tid; i < cw1; i += kGathThreads) {
      const int pos = w_pos(w0 + i - U);
      for (int hh = 0; hh < G; ++hh)
        s_w[i - cb][hh] = expf(p.scores[(bh0 + hh) * p.n_cap + pos] - s_mref[hh]);
    }
    __syncthreads();
    accumulate_rows<G>(p, g, cnt, s_row, s_rpg, s_w, acc, zs);
    __syncthreads();
  }

  // Z and N: sum the 4 row groups of each wave, then the waves
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    zs[hh] += __shfl_xor(zs[hh], 16);
    zs[hh] += __shfl_xor(zs[hh], 32);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[hh][e] += __shfl_xor(acc[hh][e], 16);
      acc[hh][e] += __shfl_xor(acc[hh][e], 32);
    }
  }
  if ((lane >> 4) == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) s_acc[wave][hh][r * 8 + e] = acc[hh][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) s_zs[wave][hh] = zs[hh];
  }
  __syncthreads();
  for (int i = tid; i < G * kHeadDim; i += kGathThreads) {
    const int hh = i / kHeadDim;
    const int d = i - hh * kHeadDim;
    float s = 0.0f;
    for (int w = 0; w < kGathWaves; ++w) s += s_acc[w][hh][d];
    p.part_n[((bh0 + hh) * p.n_tiles + tile) * kHeadDim + d] = s;
  }
  if (tid < G) {
    float z = 0.0f;
    for (int w = 0; w < kGathWaves; ++w) z += s_zs[w][tid];
    float* mz = p.part_mz + ((bh0 + tid) * p.n_tiles + tile) * 2;
    mz[0] = s_mref[tid];
    mz[1] = z;
  }
}

// ---------------------------------------------------------------- merge
// One block per (sequence, query head): 8 groups of 32 threads each take
// every 8th partial, 4 dims per thread (float4 loads issued DEPTH deep, so
// up to 8 * DEPTH tiles take one round trip, together with the head state
// that gives the partials' common reference), then the groups are summed
// in LDS in a fixed order.
constexpr int kMergeThreads = 256;
constexpr int kMergeGroups = kMergeThreads / 32;
constexpr int kMergeUnroll = 8;  // positions per thread in flight in the copy
constexpr int kMergeTiles = 8;   // most tiles per out_idx copy block
constexpr int kCopySlots = kMergeThreads * kMergeUnroll;

// out_idx for tiles [c * tpb, (c + 1) * tpb) of head bh. One round of loads
// brings every count the block needs (thread t holds tile t's count; the
// tiles before ta are summed, the block's own go to LDS) together with the
// first spt = 2^spt_log2 positions of each of its tiles (tpb * spt <=
// kCopySlots), read before their counts are known; positions past a count
// are dropped, and only a tile with more than spt takes a second round.
__device__ void copy_positions(const Params& p, int bh, int c, int nt, int tile, int tpb,
                               int spt_log2) {
  const int tid = threadIdx.x;
  const int ta = c * tpb;
  if (ta >= nt) return;
  const int tb = min(nt, ta + tpb);
  const uint32_t spt = 1u << spt_log2;  // positions per tile read up front
  __shared__ uint32_t s_pre[kMergeTiles + 1];
  __shared__ uint32_t s_own[kMergeTiles];
  __shared__ uint32_t s_part[kMergeThreads / 64];
  const uint32_t* sc = p.scnt + size_t(bh) * p.n_tiles;
  const int32_t* src = reinterpret_cast<const int32_t*>(p.cand + size_t(bh) * p.n_cap);
  int32_t spec[kMergeUnroll];
#pragma unroll
  for (int u = 0; u < kMergeUnroll; ++u) {
    const uint32_t e = uint32_t(u * kMergeThreads + tid);
    const int j = int(e >> spt_log2);
    const uint32_t i = e & (spt - 1u);  // < spt <= 2 * tile
    spec[u] = ta + j < tb ? src[size_t(ta + j) * (2 * tile) + i] : 0;
  }
  // offset: retrieved positions of the tiles before ta
  uint32_t before = 0;
  for (int t = tid; t < tb; t += kMergeThreads) {
    const uint32_t v = sc[t];
    if (t < ta) before += v;
    else s_own[t - ta] = v;
  }
  before = wave_sum(before);
  if ((tid & 63) == 0) s_part[tid >> 6] = before;
  __syncthreads();
  if (tid == 0) {
    uint32_t run = 0;
    for (int t = ta; t < tb; ++t) {
      s_pre[t - ta] = run;
      run += s_own[t - ta];
    }
    s_pre[tb - ta] = run;
  }
  __syncthreads();
  uint32_t off = 0;
  for (int w = 0; w < kMergeThreads / 64; ++w) off += s_part[w];
  int32_t* dst = p.out_idx + size_t(bh) * p.k_max + off;
#pragma unroll
  for (int u = 0; u < kMergeUnroll; ++u) {
    const uint32_t e = uint32_t(u * kMergeThreads + tid);
    const int j = int(e >> spt_log2);
    const uint32_t i = e & (spt - 1u);
    if (ta + j < tb && i < s_own[j] && RA_GUARD(off + s_pre[j] + i < uint32_t(p.k_max), p, 9))
      dst[s_pre[j] + i] = spec[u];
  }
  // the rest of the tiles holding more than spt positions
  for (int j = 0; j < tb - ta; ++j) {
    const uint32_t cnt = s_own[j];
    for (uint32_t i = spt + uint32_t(tid); i < cnt; i += kMergeThreads) {
      const int32_t v =
          RA_IN(i < uint32_t(2 * tile), p, 8) ? src[size_t(ta + j) * (2 * tile) + i] : 0;
      if (RA_GUARD(off + s_pre[j] + i < uint32_t(p.k_max), p, 9)) dst[s_pre[j] + i] = v;
    }
  }
}

// Grid (1 + copy blocks, B * H_q): x == 0 merges the partials of head y,
// x > 0 copies positions. tile_units: the gather's tile size, in units;
// tpb: tiles per copy block.
// DEPTH: partials per thread group in flight; 8 groups take 8 * DEPTH tiles
// per round trip, and a smaller DEPTH leaves room for more resident blocks.
template <int DEPTH>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(Params p, int tile_units, int tpb,
                                                              int spt_log2) {
  const int bh = blockIdx.y;
  const int b = bh / p.H_q;
  const SeqGeom sg = seq_geom(p, b);
  const int tile = tile_units * kUnit;
  const int nt = (sg.N + tile - 1) / tile;
  if (blockIdx.x > 0) {
    if (p.k_max > 0 && sg.k_eff > 0)
      copy_positions(p, bh, int(blockIdx.x) - 1, nt, tile, tpb, spt_log2);
    return;
  }
  const int tid = threadIdx.x;
  const int grp = tid >> 5;
  const int d0 = (tid & 31) * 4;
  const float* mz = p.part_mz + size_t(bh) * p.n_tiles * 2;
  const float* pn = p.part_n + size_t(bh) * p.n_tiles * kHeadDim + d0;
  __shared__ float s_red[kMergeGroups][kHeadDim + 4];
  const int np = nt;
  auto slot = [](int j) { return j; };

  // m: every non-empty partial of the head was taken relative to the same
  // reference, the head's largest score over W u Omega, which the head
  // state gives; the state is loaded with the partials, in one round
  const float m = softmax_ref(p.state[bh], sg.k_eff);

  float Z = 0.0f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  {
    for (int j0 = grp; j0 < np; j0 += kMergeGroups * DEPTH) {
      float2 w2[DEPTH];
      float4 v[DEPTH];
#pragma unroll
      for (int u = 0; u < DEPTH; ++u) {
        const int j = j0 + u * kMergeGroups;
        const int t = slot(j);
        w2[u] = j < np ? *reinterpret_cast<const float2*>(mz + 2 * t) : make_float2(0.f, 0.f);
        v[u] = j < np ? *reinterpret_cast<const float4*>(pn + size_t(t) * kHeadDim)
                      : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < DEPTH; ++u) {
        // e^{m_t - m}: 1 for every non-empty partial here, kept general
        const float sc = w2[u].y > 0.0f ? expf(w2[u].x - m) : 0.0f;
        Z += sc * w2[u].y;
        acc.x += sc * v[u].x;
        acc.y += sc * v[u].y;
        acc.z += sc * v[u].z;
        acc.w += sc * v[u].w;
      }
    }
  }
  s_red[grp][d0 + 0] = acc.x;
  s_red[grp][d0 + 1] = acc.y;
  s_red[grp][d0 + 2] = acc.z;
  s_red[grp][d0 + 3] = acc.w;
  if ((tid & 31) == 0) s_red[grp][kHeadDim] = Z;
  __syncthreads();
  if (tid < kHeadDim) {
    float a = 0.0f, zz = 0.0f;
    for (int gI = 0; gI < kMergeGroups; ++gI) {
      a += s_red[gI][tid];
      zz += s_red[gI][kHeadDim];
    }
    p.out[size_t(bh) * kHeadDim + tid] = zz > 0.0f ? a / zz : 0.0f;
    if (tid == 0 && p.lse) p.lse[bh] = zz > 0.0f ? m + logf(zz) : -INFINITY;
  }
  if (p.k_max > 0) {
    int32_t* dst = p.out_idx + size_t(bh) * p.k_max;
    for (int i = sg.k_eff + tid; i < p.k_max; i += kMergeThreads) dst[i] = -1;
  }
}

// The gather's tile size, in units: one when two-unit tiles would give
// fewer than two blocks per CU (short contexts, where the blocks would be
// few and long), else two. Both launches below take it from the same
// host arguments.
static int gather_tile_units(const Params& p) {
  const int64_t cap = std::min<int64_t>(p.max_seq_len, int64_t(p.max_pages) * kPage);
  const int64_t blocks2 = int64_t(p.B) * p.H_kv * ((cap + 2 * kUnit - 1) / (2 * kUnit));
  const int64_t cus = p.num_cus > 0 ? p.num_cus : 256;
  return blocks2 < 2 * cus ? 1 : 2;
}

static int64_t gather_tiles(const Params& p, int upt) {
  const int64_t cap = std::min<int64_t>(p.max_seq_len, int64_t(p.max_pages) * kPage);
  const int64_t tile = int64_t(upt) * kUnit;
  return std::max<int64_t>(1, std::min<int64_t>((cap + tile - 1) / tile, p.n_tiles));
}

// Positions per tile read up front: the power of two at or above 1.5 times
// a tile's mean share of k_max (at most kCopySlots); tiles per copy block:
// as many as those slots allow, up to kMergeTiles.
static void merge_copy_shape(const Params& p, int upt, int* tpb, int* spt_log2) {
  const int64_t nt = gather_tiles(p, upt);
  const int64_t per_tile = (3 * int64_t(p.k_max)) / (2 * nt) + 1;
  int sl = 0;
  while ((int64_t(1) << sl) < per_tile && (1 << sl) < kCopySlots) ++sl;
  *spt_log2 = sl;
  *tpb = std::max(1, std::min(kMergeTiles, kCopySlots >> sl));
}

hipError_t launch_merge(const Params& p, hipStream_t s) {
  const int upt = gather_tile_units(p);
  int tpb, spt_log2;
  merge_copy_shape(p, upt, &tpb, &spt_log2);
  const unsigned copies =
      p.k_max > 0 ? unsigned((gather_tiles(p, upt) + tpb - 1) / tpb) : 0u;
  // 17 x 8 groups: the 129 tiles of a length just past 2^20 in one round
  const dim3 grid{1 + copies, unsigned(p.B * p.H_q)};
  if (gather_tiles(p, upt) <= 8 * 4)
    hipLaunchKernelGGL(merge_kernel<4>, grid, dim3(kMergeThreads), 0, s, p, upt, tpb, spt_log2);
  else
    hipLaunchKernelGGL(merge_kernel<17>, grid, dim3(kMergeThreads), 0, s, p, upt, tpb, spt_log2);
  return hipGetLastError();
}

template <int UPT>
static hipError_t launch_gather_t(const Params& p, hipStream_t s) {
  const dim3 grid{unsigned(p.B * p.H_kv), unsigned(gather_tiles(p, UPT))};
  const dim3 block{unsigned(kGathThreads)};
  switch (p.G) {
    case 1: hipLaunchKernelGGL((gather_kernel<1, UPT>), grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL((gather_kernel<2, UPT>), grid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL((gather_kernel<4, UPT>), grid, block, 0, s, p); break;
    case 8: hipLaunchKernelGGL((gather_kernel<8, UPT>), grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Grid (B * H_kv, tiles): blocks are dispatched group-fastest, so the
// highest tiles come last. When a length runs just past a multiple of the
// tile (2^20 + t: 129 tiles, 1032 blocks against 1024 resident), the blocks
// left for a second wave are then the short tail tiles, which finish under
// the first wave's full ones instead of extending the kernel by a full tile.
hipError_t launch_gather(const Params& p, hipStream_t s) {
  return gather_tile_units(p) == 1 ? launch_gather_t<1>(p, s) : launch_gather_t<2>(p, s);
}

}  // namespace ra
