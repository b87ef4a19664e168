// Exact top-k keys of a block of prefill queries: the input the slides'
// index is built from (RetrievalAttention slides, "Prefill queries teach the
// key graph what matters", step 1: prefill queries find their exact top-k
// keys on the GPU; each query is then linked to those keys). For every query
// row t and query head h: the k_eff largest q . k (Eq. (1) without the
// positive factor 1 / sqrt(d), which orders the keys the same way) over the
// domain M of one sequence, ties to the lower position, ascending.
//
// Per KV head the scores form a dense (T G) x N contraction with K = 128, so
// they run on MFMA. v_mfma_f32_32x32x16_bf16 takes 32 keys as its rows (A)
// and 32 query rows as its columns (B), so a lane's 16 results are 16 keys
// of one query: a page maximum is an in-lane max plus one swap between the
// two lane halves. The score matrix is never stored. Keys compare by the
// pair (score, page), larger score first, then lower page; a set C of keys
// holding every key whose pair reaches some bound t is an upper set of the
// ranking (score, lower position): each key outside C ranks below each key
// in C. So if |C| >= k_eff, the top k_eff of C are the exact answer,
// whatever t is. Two passes use this:
//   sampled (stages 0-3): maxima of one page in 8 (page 8 j + 4); the bound
//      is the need_s-th largest sampled pair, chosen so that about 8 need_s
//      pages reach it; the filter contraction over every page keeps the
//      keys at or above it in fixed-size lists; the select takes the top
//      k_eff, or flags the row if fewer than k_eff were kept or a list
//      overflowed;
//   exact (stages 4-7, flagged rows and the row blocks holding them): maxima
//      of every page; the bound is the k_eff-th largest page pair, which k_eff
//      pages reach, each holding a key (its maximum) at or above it, so
//      |C| >= k_eff and C lies in those pages (|C| <= 64 k_eff); filter and
//      select as before.
// Every pass issues the same MFMA sequence per key on the same inputs, so a
// key's score is bit-identical in all of them.
//
// Contraction block: 8 waves, each holding the B fragments of 64 query rows
// in registers (512 rows of one KV head per block), walking a range of pages.
// A page's 64 K rows (16 KB) are loaded once per block with coalesced 16-byte
// loads, staged through a four-page LDS ring (row chunks XOR-swizzled by row
// so the 16-byte fragment reads are conflict-free), and read by every wave.
// The next two pages are in flight in registers while two are computed.
#include "ra_internal.h"

namespace ra {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kPfWaves = 8;
constexpr int kPfThreads = kPfWaves * 64;
constexpr int kPfQG = kPfBlockRows / (kPfWaves * 32);  // 32-row query groups per wave
constexpr int kPfWaveRows = kPfQG * 32;
static_assert(kPfQG % 2 == 0 && kPfWaves * kPfWaveRows == kPfBlockRows, "block rows");
constexpr int kPfRec = 128;  // score records a wave buffers before it sifts them (filter)
constexpr int kPfPageChunks = kPage * kHeadDim * 2 / 16;    // 16-byte chunks per page: 1024
constexpr int kPfLoads = kPfPageChunks / kPfThreads;         // per thread per page: 2

// The block table is read-only here: read it as constant memory, so the
// (wave-uniform) page lookup is a scalar load that does not sit in the
// vector memory counter behind the K loads in flight.
typedef const __attribute__((address_space(4))) int32_t* pf_const_i32_ptr;

__device__ __forceinline__ int pf_page(const PfParams& p, int j) {
  const int pg = ((pf_const_i32_ptr)p.block_table)[j];
  return ((unsigned)pg < (unsigned)p.num_pages) ? pg : 0;
}

// Key row of the score tile held in register r of this lane (MFMA 32x32
// layout): rows (r / 4) * 8 + (lane / 32) * 4 + r % 4; the query column is
// lane % 32.
__device__ __forceinline__ int tile_row(int r, int lane) {
  return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}

__device__ __forceinline__ float max16(const f32x16_t& c) {
  float a = fmaxf(fmaxf(c[0], c[1]), c[2]);
  float b = fmaxf(fmaxf(c[3], c[4]), c[5]);
  float d = fmaxf(fmaxf(c[6], c[7]), c[8]);
  float e = fmaxf(fmaxf(c[9], c[10]), c[11]);
  float f = fmaxf(fmaxf(c[12], c[13]), c[14]);
  return fmaxf(fmaxf(fmaxf(a, b), fmaxf(d, e)), fmaxf(f, c[15]));
}

// This thread's share of one page of K, in flight. Named members passed by
// value, not an array, so it stays in registers.
struct PfStage {
  uint4 a, b, c, d;
};
static_assert(kPfLoads == 2 || kPfLoads == 4, "two or four 16-byte loads per thread per page");

struct PfFrags {
  bf16x8_t a[8];  // one tile's A fragments (32 keys x 128 dims)
};

struct PfLds {
  uint4 ring[4][kPfPageChunks];  // four pages of K, 16-byte chunks, swizzled
  union {
    uint32_t pm[kPfWaves][kPfWaveRows * (kPfChunk + 1)];  // page-maxima keys, [row][page]
    struct {
      // a record: one lane's 16 scores of a tile whose maximum reached the
      // row's threshold, with (wave row << 24 | position of its first key)
      uint4 rec[kPfWaves][kPfRec][4];
      uint32_t meta[kPfWaves][kPfRec];
      uint32_t cnt[kPfWaves][kPfWaveRows];   // candidates per wave row in this page range
      uint64_t tau[kPfWaves][kPfWaveRows];   // per wave row: threshold pair
      uint64_t base[kPfWaves][kPfWaveRows];  // per wave row: first slot of the range's list
    } f;
  } u;
};

// Block -> (KV head g, page range z, row block rb). With xcd_groups, blocks
// b, b + 8, b + 16, ... (dispatched to the same XCD) take the row blocks of
// one (g, z) in turn, so they read the same K pages through one L2.
__device__ __forceinline__ void pf_block_coords(const PfParams& p, int& g, int& z, int& rb) {
  const int b = blockIdx.x;
  int c;
  if (p.xcd_groups) {
    const int x = b & 7, i = b >> 3;
    rb = i % p.row_blocks;
    c = (i / p.row_blocks) * 8 + x;
  } else {
    rb = b % p.row_blocks;
    c = b / p.row_blocks;
  }
  g = c / p.splits;
  z = c - g * p.splits;
}

template <int G, bool FILTER>
__global__ __launch_bounds__(kPfThreads) void pf_contract_kernel(PfParams p) {
  __shared__ PfLds sm;
  int g, z, rb;
  pf_block_coords(p, g, z, rb);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hl = lane >> 5;
  const int TG = p.T * G;
  const int rw = rb * kPfBlockRows + wave * kPfWaveRows;  // wave's first local row

  // B fragments: query row rw + 32 q + lane % 32, dims 16 s + 8 hl .. + 8
  bf16x8_t qf[kPfQG][8];
  int R[kPfQG];        // this lane's query column, as a global row t H_q + h
  bool rv[kPfQG];
#pragma unroll
  for (int q = 0; q < kPfQG; ++q) {
    const int r = rw + 32 * q + (lane & 31);
    rv[q] = r < TG;
    const int t = r / G, hh = r - (r / G) * G;
    R[q] = rv[q] ? t * p.H_q + g * G + hh : 0;
  }
  if (p.subset) {
    // the exact pass: only row blocks holding a flagged row run (the others
    // leave before reading anything else), and the filter keeps candidates
    // of flagged rows only
    bool any = false;
#pragma unroll
    for (int q = 0; q < kPfQG; ++q) {
      const bool f = rv[q] && p.fail[R[q]] != 0u;
      any = any || f;
      if (FILTER) rv[q] = f;
    }
    if (!__syncthreads_or(any)) return;  // block-uniform
  }
#pragma unroll
  for (int q = 0; q < kPfQG; ++q) {
    const uint16_t* qr = p.q + size_t(R[q]) * kHeadDim + 8 * hl;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      qf[q][s] = rv[q] ? *reinterpret_cast<const bf16x8_t*>(qr + 16 * s) : bf16x8_t{};
  }
  float thr[kPfQG];  // a score below it is no candidate
  if constexpr (FILTER) {
#pragma unroll
    for (int q = 0; q < kPfQG; ++q) {
      const uint64_t t = rv[q] ? p.tau[R[q]] : ~0ull;
      thr[q] = key2f(uint32_t(t >> 32));  // key 0: -inf, every score passes
      if (t == ~0ull) thr[q] = __uint_as_float(0x7FC00000u);  // nothing passes
      // lane l keeps the wave rows 64 i + l (group 2 i + l / 32, column l % 32)
      if ((q & 1) == hl) {
        const int wr = 32 * q + (lane & 31);
        sm.u.f.cnt[wave][wr] = 0u;
        sm.u.f.tau[wave][wr] = t;
        sm.u.f.base[wave][wr] =
            rv[q] ? size_t(R[q]) * p.cap + p.seg_off[size_t(R[q]) * p.splits + z] : 0ull;
      }
    }
  }

  // The maxima of the sampled pass walk the sampled pages: index j stands
  // for page 8 j + 4 (the last page, in a short last group).
  const bool samp = !FILTER && p.sampled;
  auto page_at = [&](int j) { return samp ? min(kPfStride * j + kPfStride / 2, p.P - 1) : j; };
  const int chunks = (samp ? p.Ps_pad : p.Ppad) / kPfChunk;
  const int j0 = int(int64_t(chunks) * z / p.splits) * kPfChunk;
  const int j1 = min(samp ? p.Ps : p.P, int(int64_t(chunks) * (z + 1) / p.splits) * kPfChunk);
  if (j0 >= j1) return;  // block-uniform

  const size_t head_off = size_t(g) * (kPage * kHeadDim);
  // Issued unconditionally (past the range it re-reads the last page), so
  // every iteration has the same loads in flight and the waits before the
  // LDS writes cover only the page being written.
  auto gload = [&](int j) {
    const uint4* kb = reinterpret_cast<const uint4*>(
        p.k_pool + size_t(pf_page(p, page_at(min(j, j1 - 1)))) * p.H_kv * (kPage * kHeadDim) + head_off);
    PfStage st;
    st.a = kb[tid];
    st.b = kb[tid + kPfThreads];
    if constexpr (kPfLoads == 4) {
      st.c = kb[tid + 2 * kPfThreads];
      st.d = kb[tid + 3 * kPfThreads];
    }
    return st;
  };
  // chunk c % 16 of key row c / 16 goes to position (c % 16) ^ (row % 16)
  auto pos = [&](int i) {
    const int c = tid + kPfThreads * i;
    return (c >> 4) * 16 + ((c & 15) ^ ((c >> 4) & 15));
  };
  auto lwrite = [&](const PfStage st, int slot) {
    sm.ring[slot][pos(0)] = st.a;
    sm.ring[slot][pos(1)] = st.b;
    if constexpr (kPfLoads == 4) {
      sm.ring[slot][pos(2)] = st.c;
      sm.ring[slot][pos(3)] = st.d;
    }
  };



  // Sift the buffered records, one per lane: every score whose pair
  // (score, page) reaches the row's threshold is appended to the row's list.
  // The buffer is a ring: records r_head .. r_tail - 1 (mod kPfRec) wait;
  // they are sifted 64 at a time (the rest at the end of the range). Under
  // the sampled bound a list holds seg_cap slots: the count goes on past it,
  // the keys are not written.
  uint32_t r_head = 0, r_tail = 0;  // wave-uniform
  const uint32_t lim = p.sampled ? uint32_t(p.seg_cap) : 0xFFFFFFFFu;
  auto sift = [&](bool all) {
    while (r_tail - r_head >= 64u || (all && r_tail != r_head)) {
      const uint32_t n = min(64u, r_tail - r_head);
      if (uint32_t(lane) < n) {
        const uint32_t i = (r_head + lane) % uint32_t(kPfRec);
        const uint32_t meta = sm.u.f.meta[wave][i];
        const uint32_t qi = meta >> 24, n0 = meta & 0xFFFFFFu;
        const uint64_t t = sm.u.f.tau[wave][qi];
        // a score above the bound's passes, one below fails, NaN fails; an
        // equal one (ties, or -0 against +0) is decided by the full pair
        const float th = key2f(uint32_t(t >> 32));
        const float* rs = reinterpret_cast<const float*>(&sm.u.f.rec[wave][i][0]);
        float v[16];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint4 x = sm.u.f.rec[wave][i][c];
          v[4 * c] = __uint_as_float(x.x);
          v[4 * c + 1] = __uint_as_float(x.y);
          v[4 * c + 2] = __uint_as_float(x.z);
          v[4 * c + 3] = __uint_as_float(x.w);
        }
        uint32_t okm = 0, eqm = 0;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          okm |= v[r] > th ? (1u << r) : 0u;
          eqm |= v[r] == th ? (1u << r) : 0u;
        }
        if (eqm) {
          const uint32_t npg = ~(n0 >> 6);  // ~page
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (((eqm >> r) & 1u) && ((uint64_t(f2key(v[r])) << 32) | npg) >= t) okm |= 1u << r;
        }
        // one reservation per record, then its keys in order
        uint32_t at = atomicAdd(&sm.u.f.cnt[wave][qi], uint32_t(__popc(okm)));
        uint64_t* list = p.cand + sm.u.f.base[wave][qi];
        while (okm) {
          const int r = __ffs(okm) - 1;
          okm &= okm - 1u;
          if (at < lim) {
            const uint32_t pos = n0 + uint32_t((r >> 2) * 8 + (r & 3));
            list[at] = (uint64_t(f2key(rs[r])) << 32) | uint32_t(~pos);
          }
          ++at;
        }
      }
      r_head += n;
    }
  };
  uint32_t* const pm_dst = samp ? p.smax : p.pmax;
  const int pm_stride = samp ? p.Ps_pad : p.Ppad;
  auto pm_flush = [&](int cs) {
    // rows of this wave x pages cs .. cs + 15: four lanes per row, 16 bytes each
#pragma unroll
    for (int i = 0; i < kPfWaveRows / 16; ++i) {
      const int qi = 16 * i + (lane >> 2);
      const int r = rw + qi;
      if (r < TG) {
        const int t = r / G, hh = r - (r / G) * G;
        const size_t Rg = size_t(t) * p.H_q + g * G + hh;
        const int e0 = 4 * (lane & 3);
        uint32_t v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = cs + e0 + e < j1 ? sm.u.pm[wave][qi * (kPfChunk + 1) + e0 + e] : 0u;
        *reinterpret_cast<uint4*>(pm_dst + Rg * pm_stride + cs + e0) = uint4{v[0], v[1], v[2], v[3]};
      }
    }
  };

  // The 8 A fragments of one tile: keys half * 32 + lane % 32 of the page in
  // ring slot `slot`, dims 16 s + 8 hl .. + 8.
  auto frags = [&](int slot, int half) {
    PfFrags f;
    const int kr = half * 32 + (lane & 31);
#pragma unroll
    for (int s = 0; s < 8; ++s)
      f.a[s] = *reinterpret_cast<const bf16x8_t*>(&sm.ring[slot][kr * 16 + ((2 * s + hl) ^ (kr & 15))]);
    return f;
  };
  auto mma = [&](const PfFrags& f, f32x16_t (&acc)[kPfQG]) {
#pragma unroll
    for (int q = 0; q < kPfQG; ++q) {
      acc[q] = f32x16_t{};
#pragma unroll
      for (int s = 0; s < 8; ++s)
        acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[s], qf[q][s], acc[q], 0, 0, 0);
    }
  };
  // Keys outside M (or past N) become NaN: ignored by the maxima, never at
  // or above a threshold. nt: position of the tile's first key.
  auto mask = [&](f32x16_t (&acc)[kPfQG], int nt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int n = nt + tile_row(r, lane);
      if (n < p.lo || n >= p.hi) {
#pragma unroll
        for (int q = 0; q < kPfQG; ++q) acc[q][r] = __uint_as_float(0x7FC00000u);
      }
    }
  };
  // The tile's scores: into the page maxima pm, or (filter) a lane whose 16
  // scores of a group reach its row's threshold buffers them as a record.
  auto tile_out = [&](const f32x16_t (&acc)[kPfQG], int nt, float (&pm)[kPfQG]) {
    if constexpr (!FILTER) {
#pragma unroll
      for (int q = 0; q < kPfQG; ++q) pm[q] = fmaxf(pm[q], max16(acc[q]));
    } else {
#pragma unroll
      for (int q = 0; q < kPfQG; ++q) {
        const bool hit = max16(acc[q]) >= thr[q];
        const uint64_t m = __ballot(hit);
        if (m) {
          if (r_tail - r_head > uint32_t(kPfRec - 64)) sift(false);
          if (hit) {
            const uint32_t at =
                (r_tail + uint32_t(__popcll(m & ((1ull << lane) - 1ull)))) % uint32_t(kPfRec);
#pragma unroll
            for (int c = 0; c < 4; ++c)
              sm.u.f.rec[wave][at][c] = uint4{__float_as_uint(acc[q][4 * c]), __float_as_uint(acc[q][4 * c + 1]),
                                              __float_as_uint(acc[q][4 * c + 2]), __float_as_uint(acc[q][4 * c + 3])};
            sm.u.f.meta[wave][at] = (uint32_t(32 * q + (lane & 31)) << 24) | uint32_t(nt + hl * 4);
          }
          r_tail += uint32_t(__popcll(m));
        }
      }
    }
  };
  // Page j's maxima: both lane halves hold 32 of the page's keys; lane l
  // then records the wave rows 64 i + l (group 2 i + l / 32).
  auto page_out = [&](float (&pm)[kPfQG], int j) {
#pragma unroll
    for (int q = 0; q < kPfQG; ++q) pm[q] = fmaxf(pm[q], __shfl_xor(pm[q], 32));
#pragma unroll
    for (int i = 0; i < kPfQG / 2; ++i) {
      const float mv = hl ? pm[2 * i + 1] : pm[2 * i];
      sm.u.pm[wave][(64 * i + lane) * (kPfChunk + 1) + (j & (kPfChunk - 1))] =
          mv == -INFINITY ? 0u : f2key(mv);
    }
  };
  auto chunk_end = [&](int j) { return (j & (kPfChunk - 1)) == kPfChunk - 1 || j == j1 - 1; };

  // One page; keys outside M are masked on pages at the edges of M.
  auto compute = [&](int j, int slot) {
    const int n0 = page_at(j) * kPage;
    const bool full = n0 >= p.lo && n0 + kPage <= p.hi;
    float pm[kPfQG];
#pragma unroll
    for (int q = 0; q < kPfQG; ++q) pm[q] = -INFINITY;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      f32x16_t acc[kPfQG];
      mma(frags(slot, half), acc);
      if (!full) mask(acc, n0 + half * 32);
      tile_out(acc, n0 + half * 32, pm);
    }
    if constexpr (!FILTER) {
      page_out(pm, j);
      if (chunk_end(j)) pm_flush(j & ~(kPfChunk - 1));
    }
  };
  // Pages j and j + 1 of the pass, both wholly inside M (maxima only): four
  // tiles in straight-line code, each tile's fragments read while the
  // previous tile's MFMAs run. Odd waves take the two pages in the other
  // order, so the waves do not all read the same fragments at once.
  auto compute_pair = [&](int j, int s0) {
    const int odd = wave & 1;
    const int pa = j + odd, pb = j + 1 - odd;
    const int sa_ = s0 + odd, sb_ = s0 + 1 - odd;
    float pmA[kPfQG], pmB[kPfQG];
#pragma unroll
    for (int q = 0; q < kPfQG; ++q) pmA[q] = pmB[q] = -INFINITY;
    f32x16_t acc[kPfQG];
    PfFrags f = frags(sa_, 0);
    PfFrags g = frags(sa_, 1);
    mma(f, acc);
    tile_out(acc, pa * kPage, pmA);
    f = frags(sb_, 0);
    mma(g, acc);
    tile_out(acc, pa * kPage + 32, pmA);
    g = frags(sb_, 1);
    mma(f, acc);
    tile_out(acc, pb * kPage, pmB);
    mma(g, acc);
    tile_out(acc, pb * kPage + 32, pmB);
    if constexpr (!FILTER) {
      page_out(pmA, pa);
      page_out(pmB, pb);
      if (chunk_end(j + 1)) pm_flush(j & ~(kPfChunk - 1));
    }
  };


  // Ring of four pages: pages j, j + 1 are computed between two barriers
  // while pages j + 2, j + 3 wait in registers to be written.
  PfStage sa = gload(j0);
  PfStage sb = gload(j0 + 1);
  lwrite(sa, 0);
  lwrite(sb, 1);
  sa = gload(j0 + 2);
  sb = gload(j0 + 3);
  __syncthreads();
  for (int j = j0; j < j1; j += 2) {
    const int s0 = j & 3;  // j0 is a multiple of 16
    if (j + 2 < j1) lwrite(sa, (j + 2) & 3);
    if (j + 3 < j1) lwrite(sb, (j + 3) & 3);
    sa = gload(j + 4);
    sb = gload(j + 5);
    // (the filter's record path leaves no registers for the pair's
    // prefetched fragments: it takes the pages one by one)
    if (!FILTER && j + 1 < j1 && page_at(j) * kPage >= p.lo && (page_at(j + 1) + 1) * kPage <= p.hi) {
      compute_pair(j, s0);
    } else {
      compute(j, s0);
      if (j + 1 < j1) compute(j + 1, s0 + 1);
    }
    __syncthreads();
  }
  if constexpr (FILTER) {
    sift(true);
    // lane l: the wave rows 64 i + l (group 2 i + l / 32, column l % 32)
#pragma unroll
    for (int i = 0; i < kPfQG / 2; ++i) {
      const bool valid = hl ? rv[2 * i + 1] : rv[2 * i];
      const int Rl = hl ? R[2 * i + 1] : R[2 * i];
      if (valid) p.seg_cnt[size_t(Rl) * p.splits + z] = sm.u.f.cnt[wave][64 * i + lane];
    }
  }
}

// ---------------------------------------------------------------- wave select
// Split z of S covers page chunks [chunks z / S, chunks (z + 1) / S).
__device__ __forceinline__ int pf_split_first_chunk(int z, int chunks, int S) {
  return int(int64_t(chunks) * z / S);
}

// The bits shared by every non-zero value (and_all over them, or_all over
// them): their count and the shared prefix, as the starting point of a radix
// select that skips the digits every value has in common.
__device__ __forceinline__ int common_prefix_len(uint64_t and_all, uint64_t or_all, int width) {
  const uint64_t diff = and_all ^ or_all;
  return diff == 0 ? width : __clzll((long long)diff) - (64 - width);
}

// The need-th largest of the non-zero values a wave visits (visit(fn) calls
// fn(v) for each value of this lane; the values are distinct), by an 8-bit
// radix below their common prefix; hist is this wave's 256 LDS bins. Returns
// a bound t such that exactly `need` of the values are >= t. Every lane of
// the wave calls it with the same arguments; at least `need` values exist.
template <typename Visit>
__device__ __forceinline__ uint64_t wave_kth(Visit&& visit, uint32_t need, uint32_t* hist) {
  const int lane = lane_id();
  uint64_t and_all = ~0ull, or_all = 0ull;
  visit([&](uint64_t v) {
    if (v != 0ull) {
      and_all &= v;
      or_all |= v;
    }
  });
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    and_all &= __shfl_xor(and_all, off);
    or_all |= __shfl_xor(or_all, off);
  }
  int plen = common_prefix_len(and_all, or_all, 64);
  if (plen == 64) return and_all;  // a single value
  uint64_t prefix = plen == 0 ? 0ull : and_all >> (64 - plen);
  for (;;) {
#pragma unroll
    for (int i = 0; i < 4; ++i) hist[lane * 4 + i] = 0u;
    const int d = min(8, 64 - plen);
    const int sh = 64 - plen - d;
    visit([&](uint64_t v) {
      if (v != 0ull && (plen == 0 || (v >> (64 - plen)) == prefix))
        atomicAdd(&hist[uint32_t(v >> sh) & ((1u << d) - 1u)], 1u);
    });
    // lane l holds bins 255 - 4 l .. 252 - 4 l (largest digits first)
    uint32_t c[4], s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[i] = hist[255 - 4 * lane - i];
      s += c[i];
    }
    uint32_t incl = s;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t t = __shfl_up(incl, off);
      if (lane >= off) incl += t;
    }
    const uint64_t reach = __ballot(incl >= need);
    const int L = reach ? __ffsll((unsigned long long)reach) - 1 : 63;
    uint32_t run = incl - s, digit = 0, above = 0, cd = 0;
    bool found = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (!found && run + c[i] >= need) {
        found = true;
        digit = 255u - 4u * uint32_t(lane) - uint32_t(i);
        above = run;
        cd = c[i];
      }
      run += c[i];
    }
    digit = __shfl(digit, L);
    above = __shfl(above, L);
    cd = __shfl(cd, L);
    prefix = (prefix << d) | digit;
    plen += d;
    need -= above;
    if (cd == need || plen == 64) return prefix << (64 - plen);
  }
}

// ---------------------------------------------------------------- threshold
// The need-th largest of the non-zero keys v (NV per lane, repeats allowed),
// by 8-bit radix passes over registers below the keys' common prefix; hist
// is this wave's 256 LDS bins. Requires at least `need` non-zero keys.
// Returns the key and, in *above, how many keys are strictly larger.
template <int NV>
__device__ __forceinline__ uint32_t reg_kth(const uint32_t (&v)[NV], uint32_t need,
                                            uint32_t* hist, uint32_t* above_out) {
  const int lane = lane_id();
  uint32_t and_all = ~0u, or_all = 0u;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    if (v[i] != 0u) {
      and_all &= v[i];
      or_all |= v[i];
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    and_all &= __shfl_xor(and_all, off);
    or_all |= __shfl_xor(or_all, off);
  }
  int rem = 32 - common_prefix_len(and_all, or_all, 32);  // bits still open
  uint32_t prefix = rem == 32 ? 0u : and_all & ~((1u << rem) - 1u);
  uint32_t above_all = 0;
#pragma unroll 1
  while (rem > 0) {
    const int d = min(8, rem);
    const int sh = rem - d;
#pragma unroll
    for (int i = 0; i < 4; ++i) hist[lane * 4 + i] = 0u;
    // the bits above the digit must equal the prefix's
    const uint32_t hi_mask = sh + d == 32 ? 0u : ~((1u << (sh + d)) - 1u);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const uint32_t x = v[i];
      if (x != 0u && (x & hi_mask) == prefix) atomicAdd(&hist[(x >> sh) & ((1u << d) - 1u)], 1u);
    }
    uint32_t c[4], s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[i] = hist[255 - 4 * lane - i];
      s += c[i];
    }
    uint32_t incl = s;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t t = __shfl_up(incl, off);
      if (lane >= off) incl += t;
    }
    const uint64_t reach = __ballot(incl >= need);
    const int L = reach ? __ffsll((unsigned long long)reach) - 1 : 63;
    uint32_t run = incl - s, digit = 0, above = 0;
    bool found = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (!found && run + c[i] >= need) {
        found = true;
        digit = 255u - 4u * uint32_t(lane) - uint32_t(i);
        above = run;
      }
      run += c[i];
    }
    digit = __shfl(digit, L);
    above = __shfl(above, L);
    prefix |= digit << sh;
    need -= above;
    above_all += above;
    rem = sh;
  }
  *above_out = above_all;
  return prefix;
}

// One wave per row: the threshold pair over the row's page maxima and the
// first candidate slot of each page range (64 per page at or above the
// threshold: no other page holds a candidate). Under the sampled bound the
// pair is the need_s-th largest over the sampled pages' maxima, and every
// page range gets seg_cap slots.
constexpr int kPfSelWaves = 4;

// Page of entry j of a row's maxima: page j, or sampled page 8 j + 4.
__device__ __forceinline__ int pf_entry_page(const PfParams& p, int j) {
  return p.sampled ? min(kPfStride * j + kPfStride / 2, p.P - 1) : j;
}

// The bound's rank among the row's maxima.
__device__ __forceinline__ uint32_t pf_need(const PfParams& p) {
  return p.sampled ? uint32_t(p.need_s) : uint32_t(p.k_eff);
}

__device__ __forceinline__ bool pf_pair_at_least(uint32_t key, int page, uint64_t t) {
  return key != 0u && ((uint64_t(key) << 32) | uint32_t(~uint32_t(page))) >= t;
}

// Lane l holds pages 256 i + 4 l + e in registers.
template <int NV>
__global__ __launch_bounds__(kPfSelWaves * 64) void pf_threshold_kernel(PfParams p) {
  __shared__ uint32_t s_hist[kPfSelWaves][256];
  __shared__ uint32_t s_pre[kPfSelWaves][NV * 16 / 4 + 1];  // per chunk, then prefix
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  const int R = blockIdx.x * kPfSelWaves + wave;
  if (R >= p.T * p.H_q) return;
  if (p.subset && p.fail[R] == 0u) return;
  const int width = p.sampled ? p.Ps_pad : p.Ppad;
  const uint32_t* pm = p.sampled ? p.smax + size_t(R) * p.Ps_pad : p.pmax + size_t(R) * p.Ppad;
  uint32_t v[NV];
  uint32_t present = 0;
#pragma unroll
  for (int i = 0; i < NV / 4; ++i) {
    const int j = 256 * i + 4 * lane;
    const uint4 x = j < width ? *reinterpret_cast<const uint4*>(pm + j) : uint4{0u, 0u, 0u, 0u};
    v[4 * i] = x.x;
    v[4 * i + 1] = x.y;
    v[4 * i + 2] = x.z;
    v[4 * i + 3] = x.w;
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) present += v[i] ? 1u : 0u;
  present = wave_sum(present);
  const uint32_t need0 = pf_need(p);
  uint64_t t;
  if (p.k_eff == 0) {
    t = ~0ull;  // nothing is retrieved
  } else if (present <= need0) {
    t = 1ull;   // every member of M is a candidate
  } else {
    uint32_t above;
    const uint32_t key = reg_kth<NV>(v, need0, s_hist[wave], &above);
    // the pair's page: the (need0 - above)-th lowest page whose maximum is key
    uint32_t need = need0 - above;
    int page = 0;
#pragma unroll
    for (int i = 0; i < NV / 4; ++i) {
      uint32_t c = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) c += v[4 * i + e] == key ? 1u : 0u;
      uint32_t incl = c;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t u = __shfl_up(incl, off);
        if (lane >= off) incl += u;
      }
      const uint32_t tot = __shfl(incl, 63);
      if (need <= tot) {
        const uint64_t reach = __ballot(incl >= need);
        const int L = __ffsll((unsigned long long)reach) - 1;
        uint32_t run = incl - c;
        int pg = 0;
        bool found = false;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (v[4 * i + e] == key) {
            ++run;
            if (!found && run == need) {
              found = true;
              pg = 256 * i + 4 * lane + e;
            }
          }
        }
        page = __shfl(pg, L);
        break;
      }
      need -= tot;
    }
    t = (uint64_t(key) << 32) | uint32_t(~uint32_t(pf_entry_page(p, page)));
  }
  if (p.sampled) {
    if (lane < p.splits) p.seg_off[size_t(R) * p.splits + lane] = uint32_t(lane) * uint32_t(p.seg_cap);
    if (lane == 0) p.tau[R] = t;
    return;
  }
  // pages at or above t per chunk of 16 (lanes 4 m .. 4 m + 3 share chunk
  // 16 i + m), then the exclusive prefix over chunks
  const int chunks = p.Ppad / kPfChunk;
#pragma unroll
  for (int i = 0; i < NV / 4; ++i) {
    uint32_t c = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) c += pf_pair_at_least(v[4 * i + e], 256 * i + 4 * lane + e, t) ? 1u : 0u;
    c += __shfl_xor(c, 1);
    c += __shfl_xor(c, 2);
    if ((lane & 3) == 0) s_pre[wave][16 * i + (lane >> 2)] = c;
  }
  {
    constexpr int kCh = NV * 4;               // chunks of 16 pages held
    constexpr int kPer = (kCh + 63) / 64;     // chunks per lane
    uint32_t c[kPer], sum = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      c[i] = kPer * lane + i < kCh ? s_pre[wave][kPer * lane + i] : 0u;
      sum += c[i];
    }
    uint32_t incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t u = __shfl_up(incl, off);
      if (lane >= off) incl += u;
    }
    uint32_t run = incl - sum;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (kPer * lane + i < kCh) s_pre[wave][kPer * lane + i] = run;
      run += c[i];
    }
  }
  if (lane < p.splits)
    p.seg_off[size_t(R) * p.splits + lane] =
        uint32_t(kPage) * s_pre[wave][pf_split_first_chunk(lane, chunks, p.splits)];
  if (lane == 0) p.tau[R] = t;
}

// Rows with more pages than registers hold: the same pair, by the radix
// over the 64-bit pairs read from global memory, and the same offsets.
__global__ __launch_bounds__(kPfSelWaves * 64) void pf_threshold_wide_kernel(PfParams p) {
  __shared__ uint32_t s_hist[kPfSelWaves][256];
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  const int R = blockIdx.x * kPfSelWaves + wave;
  if (R >= p.T * p.H_q) return;
  if (p.subset && p.fail[R] == 0u) return;
  const int count = p.sampled ? p.Ps : p.P;
  const uint32_t* pm = p.sampled ? p.smax + size_t(R) * p.Ps_pad : p.pmax + size_t(R) * p.Ppad;
  uint32_t present = 0;
  for (int j = lane; j < count; j += 64) present += pm[j] ? 1u : 0u;
  present = wave_sum(present);
  const uint32_t need0 = pf_need(p);
  uint64_t t;
  if (p.k_eff == 0) {
    t = ~0ull;
  } else if (present <= need0) {
    t = 1ull;
  } else {
    auto visit = [&](auto&& fn) {
      for (int j = lane; j < count; j += 64) {
        const uint32_t key = pm[j];
        fn(key ? (uint64_t(key) << 32) | uint32_t(~uint32_t(pf_entry_page(p, j))) : 0ull);
      }
    };
    t = wave_kth(visit, need0, s_hist[wave]);
  }
  if (p.sampled) {
    if (lane < p.splits) p.seg_off[size_t(R) * p.splits + lane] = uint32_t(lane) * uint32_t(p.seg_cap);
    if (lane == 0) p.tau[R] = t;
    return;
  }
  const int chunks = p.Ppad / kPfChunk;
  uint32_t before = 0;  // pages at or above t in the ranges so far
  for (int z = 0; z < p.splits; ++z) {
    const int a = pf_split_first_chunk(z, chunks, p.splits) * kPfChunk;
    const int b = min(p.P, pf_split_first_chunk(z + 1, chunks, p.splits) * kPfChunk);
    uint32_t c = 0;
    for (int j = a + lane; j < b; j += 64) c += pf_pair_at_least(pm[j], j, t) ? 1u : 0u;
    c = wave_sum(c);
    if (lane == 0) p.seg_off[size_t(R) * p.splits + z] = uint32_t(kPage) * before;
    before += c;
  }
  if (lane == 0) p.tau[R] = t;
}

// One wave per row: the exact top k_eff of the row's candidates (the page
// ranges' lists, in range order), ascending. Under the sampled bound a row
// whose candidates are fewer than k_eff, or did not all fit their lists, is
// flagged instead and left to the exact pass.
constexpr uint32_t kPfSelLds = 512;  // candidates a row copies to LDS before its radix

__global__ __launch_bounds__(kPfSelWaves * 64) void pf_select_kernel(PfParams p) {
  __shared__ uint32_t s_hist[kPfSelWaves][256];
  __shared__ __align__(16) int32_t s_pos[kPfSelWaves][RA_PREFILL_MAX_K];
  __shared__ uint64_t s_cand[kPfSelWaves][kPfSelLds];
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  const int R = blockIdx.x * kPfSelWaves + wave;
  if (R >= p.T * p.H_q) return;
  if (p.subset && p.fail[R] == 0u) return;
  int32_t* out = p.out_idx + size_t(R) * p.k;
  const uint32_t ke = uint32_t(p.k_eff);
  if (p.sampled && ke == 0 && lane == 0) p.fail[R] = 0u;
  if (ke > 0) {
    const uint64_t* cl = p.cand + size_t(R) * p.cap;
    // lane z holds page range z's list: its count, first slot, and where
    // it starts in the concatenation of the lists
    const int S = p.splits;
    const uint32_t cnt_z = lane < S ? p.seg_cnt[size_t(R) * S + lane] : 0u;
    const uint32_t off_z = lane < S ? p.seg_off[size_t(R) * S + lane] : 0u;
    uint32_t pre_z = cnt_z;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t t = __shfl_up(pre_z, o);
      if (lane >= o) pre_z += t;
    }
    const uint32_t n = __shfl(pre_z, 63);
    pre_z -= cnt_z;
    if (p.sampled) {
      const bool short_ = __ballot(cnt_z > uint32_t(p.seg_cap)) != 0ull || n < ke;
      if (lane == 0) p.fail[R] = short_ ? 1u : 0u;
      if (short_) return;
    }
    // the winners' positions, in list order
    uint32_t filled = 0;
    auto winners = [&](const uint64_t* b, uint32_t cnt, uint64_t th) {
      for (uint32_t base = 0; base < cnt; base += 64) {
        const uint32_t i = base + lane;
        const uint64_t v = i < cnt ? b[i] : 0ull;
        const bool win = i < cnt && v >= th;
        const uint64_t m = __ballot(win);
        const uint32_t at = filled + uint32_t(__popcll(m & ((1ull << lane) - 1ull)));
        if (win && at < ke) s_pos[wave][at] = int32_t(~uint32_t(v));
        filled += uint32_t(__popcll(m));
      }
    };
    if (n <= kPfSelLds) {
      // the lists, concatenated in LDS (four loads in flight per lane); the
      // radix passes then read LDS. Entry c is in the last range whose
      // start is <= c.
      uint64_t* sv = s_cand[wave];
      for (uint32_t c0 = 0; c0 < n; c0 += 256) {
        uint64_t x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t c = c0 + 64u * u + uint32_t(lane);
          int zs = 0;
          for (int z = 1; z < S; ++z) zs = __shfl(pre_z, z) <= c ? z : zs;
          const uint32_t src = __shfl(off_z, zs) + (c - __shfl(pre_z, zs));
          x[u] = c < n ? cl[src] : 0ull;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t c = c0 + 64u * u + uint32_t(lane);
          if (c < n) sv[c] = x[u];
        }
      }
      auto visit = [&](auto&& fn) {
        for (uint32_t i = lane; i < n; i += 64) fn(sv[i]);
      };
      const uint64_t th = n > ke ? wave_kth(visit, ke, s_hist[wave]) : 1ull;
      winners(sv, n, th);
    } else {
      auto visit = [&](auto&& fn) {
        for (int z = 0; z < S; ++z) {
          const uint32_t cnt = __shfl(cnt_z, z);
          const uint64_t* b = cl + __shfl(off_z, z);
          for (uint32_t i = lane; i < cnt; i += 64) fn(b[i]);
        }
      };
      const uint64_t th = n > ke ? wave_kth(visit, ke, s_hist[wave]) : 1ull;
      for (int z = 0; z < S; ++z) winners(cl + __shfl(off_z, z), __shfl(cnt_z, z), th);
    }
    // ascending: each winner's rank is the number of smaller positions
    // (four at a time; the slots past ke rank above every position)
    const uint32_t ke4 = (ke + 3u) & ~3u;
    if (uint32_t(lane) < ke4 - ke) s_pos[wave][ke + lane] = INT32_MAX;
    const int4* s4 = reinterpret_cast<const int4*>(s_pos[wave]);
    for (uint32_t i = lane; i < ke; i += 64) {
      const int32_t x = s_pos[wave][i];
      uint32_t rank = 0;
      for (uint32_t j = 0; j < ke4 / 4; ++j) {
        const int4 y = s4[j];
        rank += (y.x < x ? 1u : 0u) + (y.y < x ? 1u : 0u) + (y.z < x ? 1u : 0u) + (y.w < x ? 1u : 0u);
      }
      out[rank] = x;
    }
  }
  for (int i = int(ke) + lane; i < p.k; i += 64) out[i] = -1;
}

// ---------------------------------------------------------------- launch
template <int G>
static void launch_pf_contract(const PfParams& p, bool filter, hipStream_t s) {
  const dim3 grid{unsigned(p.H_kv) * unsigned(p.splits) * unsigned(p.row_blocks)};
  if (filter)
    hipLaunchKernelGGL((pf_contract_kernel<G, true>), grid, dim3(kPfThreads), 0, s, p);
  else
    hipLaunchKernelGGL((pf_contract_kernel<G, false>), grid, dim3(kPfThreads), 0, s, p);
}

// Stages 0-3 run under the sampled bound, 4-7 the exact pass on the rows
// stage 3 flagged; within each half: maxima, threshold, filter, select.
hipError_t launch_prefill(const PfParams& p0, int first, int last, hipStream_t s) {
  const int G = p0.H_q / p0.H_kv;
  const unsigned row_waves = unsigned((int64_t(p0.T) * p0.H_q + kPfSelWaves - 1) / kPfSelWaves);
  for (int st = first; st <= last; ++st) {
    PfParams p = p0;
    p.sampled = st < 4 ? 1 : 0;
    p.subset = st < 4 ? 0 : 1;
    const int kind = st & 3;
    if (kind == 0 && p.sampled) {
      // the sampled maxima have 1/8 of the pages: fewer page ranges
      p.splits = min(p.splits, p.Ps_pad / kPfChunk);
      p.xcd_groups = (p.H_kv * p.splits) % 8 == 0 ? 1 : 0;
    }
    if (kind == 0 || kind == 2) {
      switch (G) {
        case 1: launch_pf_contract<1>(p, kind == 2, s); break;
        case 2: launch_pf_contract<2>(p, kind == 2, s); break;
        case 4: launch_pf_contract<4>(p, kind == 2, s); break;
        case 8: launch_pf_contract<8>(p, kind == 2, s); break;
        default: return hipErrorInvalidValue;
      }
    } else if (kind == 1) {
      const dim3 grid(row_waves), block(kPfSelWaves * 64);
      const int width = p.sampled ? p.Ps_pad : p.Ppad;
      if (width <= 256)
        hipLaunchKernelGGL(pf_threshold_kernel<4>, grid, block, 0, s, p);
      else if (width <= 512)
        hipLaunchKernelGGL(pf_threshold_kernel<8>, grid, block, 0, s, p);
      else if (width <= 1024)
        hipLaunchKernelGGL(pf_threshold_kernel<16>, grid, block, 0, s, p);
      else if (width <= 2048)
        hipLaunchKernelGGL(pf_threshold_kernel<32>, grid, block, 0, s, p);
      else if (width <= 4096)
        hipLaunchKernelGGL(pf_threshold_kernel<64>, grid, block, 0, s, p);
      else
        hipLaunchKernelGGL(pf_threshold_wide_kernel, grid, block, 0, s, p);
    } else {
      hipLaunchKernelGGL(pf_select_kernel, dim3(row_waves), dim3(kPfSelWaves * 64), 0, s, p);
    }
  }
  return hipGetLastError();
}

}  // namespace ra
