// Internal definitions shared by the host API (ra_api.cpp) and the gfx950
// kernels: workspace layout, kernel parameters, launchers.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "ra.h"

namespace ra {

constexpr int kHeadDim = 128;
constexpr int kPage = 64;
// Candidate lists are kept per (query head, unit of 64 pages): the scan
// block that owns a unit writes its lists and counts without atomics.
constexpr int kUnitPages = 64;
constexpr int kUnit = kUnitPages * kPage;  // 4096 positions
// A gather tile (one split-K partial) is one or two units, as the launch
// picks; kTile is the larger. Workspace rows hold whole pairs of them.
constexpr int kTile = 2 * kUnit;
// Largest number of units of one sequence (RA_MAX_SEQ_LEN / kUnit).
constexpr int kMaxUnits = RA_MAX_SEQ_LEN / kUnit;
// Sampling: one page in S is scored before the main scan, S a power of two
// chosen so that at least kSampleMinPages pages of a (sequence, KV head)
// are sampled, and S <= 2^kSampleMaxLog2. Page j is sampled iff
// j % S == S / 2.
constexpr int kSampleMinPages = 16;
constexpr int kSampleMaxLog2 = 6;

__host__ __device__ inline int sample_log2(int P) {
  int s = 0;
  while (s < kSampleMaxLog2 && (P >> (s + 1)) >= kSampleMinPages) ++s;
  return s;
}

__host__ __device__ inline int sampled_pages(int P) {
  const int S = 1 << sample_log2(P);
  const int half = S >> 1;
  return P > half ? (P - half + S - 1) / S : 0;
}

// Candidate entries: key << 32 | position (order-preserving score key).
// The list of (head, unit u) starts at entry u * kUnit of the head's row and
// has capacity kUnit, so it can hold every position of the unit.

struct alignas(8) HeadState {
  // lo_key and lo_set form one 64-bit word, written once per call with a
  // single atomic store once the bound is known (sample_bound.h)
  uint32_t lo_key;      // candidates are the members of M with key >= lo_key
  uint32_t lo_set;      // 1: lo_key is this call's bound
  uint32_t max_w;       // order-preserving key of the largest score over W
  uint32_t max_m;       // ... over M (0 = no position seen)
  uint32_t dense;       // 1: too few candidates; rescanned with lo_key = 0
  // decision: a candidate with composite c = (key - lo_key) << 32 | ~n is
  // retrieved iff thr_shift < 64 and (c >> thr_shift) >= thr
  uint32_t thr_shift;
  uint32_t thr_lo, thr_hi;
};
static_assert(sizeof(HeadState) == 32 && offsetof(HeadState, lo_set) == 4,
              "the bound and its flag share the first 64-bit word");

struct WsLayout {
  int64_t n_cap;    // row stride (positions), a multiple of kTile
  int32_t n_tiles;  // n_cap / kUnit: per-tile arrays hold the smallest tiles
  int32_t n_units;  // n_cap / kUnit
  int32_t samp_cap; // sampled key slots per head
  size_t off_scores, off_samp, off_state, off_gdone, off_misc, off_unitoff,
      off_ucnt, off_scnt, off_cand, off_part_mz, off_part_n, total;
};

// Pure host function; returns false for invalid capacities.
bool ws_layout(int32_t B, int32_t H_q, int32_t H_kv, int32_t max_seq_len,
               int32_t k_max, WsLayout* out);

struct Params {
  // a token's K and V rows to append before the scan (null: none)
  const uint16_t* app_k;     // [B][H_kv][128]
  const uint16_t* app_v;
  const int32_t* app_pos;    // [B]
  const uint16_t* q;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* kk;
  float* out;
  float* lse;
  int32_t* out_idx;
  int32_t B, H_q, H_kv, G, max_pages, num_pages, max_seq_len, k_max, n_sink,
      window;
  // workspace
  float* scores;       // [B*H_q][n_cap]: W scores (scan); the retrieved
                       // positions' scores of a tile (its gather block)
                       // when kept, or when the tile's lists overflow
                       // the gather's LDS staging
  uint32_t* samp;      // [B*H_q][samp_cap] keys of the sampled positions
                       // (0: past the sequence's end)
  HeadState* state;    // [B*H_q]
  uint32_t* gdone;     // [B*H_kv] units of the group rescanned so far
  uint32_t* any_dense; // heads rescanned in this call
  uint32_t* dbg;       // debug builds: bounds checks that failed in this
                       // call, one bit per check site (reset per call)
  int64_t* unit_off;   // [B + 1] prefix of H_kv * units(b)
  uint32_t* ucnt;      // [B*H_q][n_units] candidates per (head, unit)
  uint32_t* scnt;      // [B*H_q][n_tiles] retrieved per (head, tile)
  uint64_t* cand;      // [B*H_q][n_cap] per-unit candidate lists; after the
                       // gather, tile t's region holds its retrieved
                       // positions (int32, ascending)
  float* part_mz;      // [B*H_q][n_tiles][2]  (m, Z)
  float* part_n;       // [B*H_q][n_tiles][128]
  int64_t n_cap;
  int32_t n_tiles;
  int32_t n_units;
  int32_t samp_cap;
  int32_t num_cus;
  int32_t keep_scores;  // also store the retrieved set's scores in the rows
  int32_t scan_bounds;  // 1: the scan's blocks compute the heads' candidate
                        // bounds up front (no threshold launch in this call)
};

// Prefill top-k (prefill_topk.hip).
constexpr int kPfChunk = 16;       // pages per page-maxima row segment
constexpr int kPfBlockRows = 512;  // query rows (of one KV head) per contraction block
constexpr int kPfMaxSplits = 64;   // page ranges per (KV head, row block), at most
constexpr int kPfMinCapPages = 32; // candidate slots per row: 64 x max(k, this)
constexpr int kPfStride = 8;       // the sampled pass takes page 8 j + 4 of every 8

// Sampled pages of a row of P pages: ceil(P / 8), each inside its group.
__host__ __device__ inline int pf_sampled_pages(int P) { return (P + kPfStride - 1) / kPfStride; }

struct PfParams {
  const uint16_t* q;          // [T][H_q][128]
  const uint16_t* k_pool;
  const int32_t* block_table; // the sequence's row
  int32_t T, H_q, H_kv, N, P, num_pages;
  int32_t Ppad;               // P rounded up to kPfChunk: row stride of pmax
  int32_t lo, hi;             // M = [lo, hi)
  int32_t k, k_eff, cap;
  int32_t row_blocks;         // contraction row blocks per KV head
  int32_t splits;             // page ranges per (KV head, row block), <= kPfMaxSplits
  int32_t xcd_groups;         // 1: the row blocks of a page range share an XCD
  // set per launch: sampled = the pass over the sampled pages (page
  // 8 j + 4 of each group j of 8 pages) and the bound they give; subset = the
  // exact pass, restricted to flagged rows (and the row blocks holding one)
  int32_t sampled, subset;
  int32_t Ps, Ps_pad;         // sampled pages; row stride of smax
  int32_t need_s;             // rank of the sampled bound among a row's sampled maxima
  int32_t seg_cap;            // slots of a (row, page range) list (sampled bound)
  uint32_t* smax;   // [T*H_q][Ps_pad] maxima of the sampled pages
  uint32_t* fail;   // [T*H_q] 1: the row's sampled filter fell short
  uint32_t* pmax;   // [T*H_q][Ppad] largest score key per page over M (0: none)
  uint64_t* tau;    // [T*H_q] threshold pair (key << 32 | ~page)
  uint32_t* seg_off;  // [T*H_q][splits] first candidate slot of each page range
  uint32_t* seg_cnt;  // [T*H_q][splits] candidates found in each page range
  uint64_t* cand;   // [T*H_q][cap] candidates (key << 32 | ~n), by page range
  int32_t* out_idx; // [T][H_q][k]
};

struct PfLayout {
  size_t off_pmax, off_tau, off_seg_off, off_seg_cnt, off_cand, off_smax, off_fail, total;
  int64_t cap;  // candidate slots per row
};

// Attention over listed positions, and the merge of two partials
// (sparse_attend.hip).
struct SaParams {
  const uint16_t* q;          // [H_q][128]
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* block_table; // the sequence's row
  int32_t H_q, H_kv, N, num_pages, k;
  const int32_t* idx;         // [H_q][k]
  float* out;                 // [H_q][128]
  float* out_lse;             // [H_q]
};
hipError_t launch_sparse_attend(const SaParams& p, hipStream_t s);
hipError_t launch_merge_partials(const float* oa, const float* la, const float* ob,
                                 const float* lb, int32_t H, float* out, float* lse,
                                 hipStream_t s);

// Key-graph search (graph_search.hip).
constexpr int kGsBatch = RA_GRAPH_BATCH;  // keys expanded per round of the search
struct GsParams {
  const uint16_t* q;          // [H_q][128]
  const uint16_t* k_pool;
  const int32_t* block_table; // the sequence's row
  int32_t H_q, H_kv, N, num_pages;
  const int32_t* nbr;         // [H_q][N][D], -1 padded
  const int32_t* entry;       // [H_q]
  int32_t D, ef, k;
  int32_t vis_words;          // visited-bitmap words (in LDS)
  int32_t* out_idx;           // [H_q][k]
  int32_t* out_visited;       // [H_q]
};
hipError_t launch_graph_search(const GsParams& p, hipStream_t s);

bool pf_layout(int32_t T, int32_t H_q, int32_t N, int32_t k, PfLayout* out);
hipError_t launch_prefill(const PfParams& p, int first, int last, hipStream_t s);

// Launchers (each enqueues its kernels on `s`; they never synchronise).
hipError_t launch_sample(const Params& p, hipStream_t s);
hipError_t launch_threshold(const Params& p, hipStream_t s);
hipError_t launch_scan(const Params& p, hipStream_t s);
hipError_t launch_select(const Params& p, hipStream_t s);  // + rescan of short heads
// Grid of the persistent unit loops (scan, rescan): one block per CU, at
// most one per unit.
unsigned scan_blocks(const Params& p);
// True when the scan, run right after the sample, should compute the
// heads' candidate bounds itself instead of a threshold launch.
bool scan_computes_bounds(const Params& p);
hipError_t launch_gather(const Params& p, hipStream_t s);
hipError_t launch_merge(const Params& p, hipStream_t s);
hipError_t launch_kv_append(const ra_kv_layer& kv, const uint16_t* k_new,
                            const uint16_t* v_new, const int32_t* pos,
                            int32_t B, hipStream_t s);

#if defined(__HIPCC__)
// ---------------------------------------------------------------- device

// Debug builds (-DRA_DEBUG): bounds checks at the decode kernels' computed
// global accesses. RA_IN(cond, p, bit) is cond; when it fails, bit `bit`
// is set in *p.dbg (a workspace word that a debug build's first kernel of
// the step clears, read back as a diagnostic) and the guarded access is skipped, so a debug run reports an
// index out of its buffer instead of touching memory outside it; no check
// ever traps. Release builds compile every check to `true`.
//   bit 0: a candidate list slot (scan flush)       bit 1: the same, staging full
//   bit 2: a score row entry (scan, W)              bit 3: a sampled key's row
//   bit 4: a rescanned list slot                    bit 5: a list entry the gather reads
//   bit 6: a tile position the gather writes        bit 7: a retrieved score the gather stores
//   bit 8: a position the merge copies              bit 9: an out_idx slot the merge writes
// RA_GUARD is the same record for a condition that release builds test too.
#if defined(RA_DEBUG)
#define RA_IN(cond, p, bit) ((cond) || (atomicOr((p).dbg, 1u << (bit)), false))
#define RA_GUARD(cond, p, bit) RA_IN(cond, p, bit)
#else
#define RA_IN(cond, p, bit) true
#define RA_GUARD(cond, p, bit) (cond)
#endif

// Order-preserving map fp32 -> uint32 (larger float, larger key); -0 maps
// like +0 so that equal scores compare equal.
__device__ __forceinline__ uint32_t f2key(float x) {
  x = x + 0.0f;
  uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of f2key; key 0 (nothing recorded) maps to -inf.
__device__ __forceinline__ float key2f(uint32_t k) {
  if (k == 0u) return -INFINITY;
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Reference point of the softmax over W u Omega: the largest score in that
// set. The top-ranked member of M is in Omega whenever k_eff > 0, so it is
// max(max over W, max over M) then, and the max over W otherwise.
__device__ __forceinline__ float softmax_ref(const HeadState& st, int k_eff) {
  const uint32_t k = k_eff > 0 ? max(st.max_w, st.max_m) : st.max_w;
  return key2f(k);
}

struct SeqGeom {
  int N;      // clamped length
  int lo, hi; // M = [lo, hi)
  int k_eff;
};

__device__ __forceinline__ SeqGeom seq_geom(const Params& p, int b) {
  SeqGeom g;
  int cap = min(p.max_seq_len, p.max_pages * kPage);
  int n = p.seq_lens[b];
  g.N = n < 0 ? 0 : (n > cap ? cap : n);
  g.lo = min(p.n_sink, g.N);
  int hi = g.N - p.window;
  g.hi = hi > g.lo ? hi : g.lo;
  int kb = p.kk[b];
  kb = kb < 0 ? 0 : (kb > p.k_max ? p.k_max : kb);
  g.k_eff = min(kb, g.hi - g.lo);
  return g;
}

__device__ __forceinline__ int page_of(const Params& p, int b, int j) {
  int pg = p.block_table[(size_t)b * p.max_pages + j];
  return ((unsigned)pg < (unsigned)p.num_pages) ? pg : 0;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Unit x of the linear unit index over (sequence, KV head, unit), unit
// fastest: unit_off[b] = sum_{b' < b} H_kv * units(b').
struct UnitRef {
  int b, g, u, npages;
};

__device__ __forceinline__ UnitRef unit_at(const Params& p, int64_t x) {
  int blo = 0, bhi = p.B - 1;
  while (blo < bhi) {
    const int mid = (blo + bhi + 1) >> 1;
    if (p.unit_off[mid] <= x) blo = mid; else bhi = mid - 1;
  }
  UnitRef r;
  r.b = blo;
  const int P = (seq_geom(p, blo).N + kPage - 1) / kPage;
  const int nu = (P + kUnitPages - 1) / kUnitPages;
  const int64_t rel = x - p.unit_off[blo];
  r.g = int(rel / nu);
  r.u = int(rel - int64_t(r.g) * nu);
  r.npages = min(kUnitPages, P - r.u * kUnitPages);
  return r;
}

// Sum over this lane and every higher lane of the wave.
__device__ __forceinline__ uint32_t wave_suffix_sum(uint32_t v) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t t = __shfl_down(v, off);
    if (lane + off < 64) v += t;
  }
  return v;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// Exclusive prefix sum over the threads of a block (blockDim.x a multiple
// of 64, at most 1024). `tmp` holds 16 entries of LDS. Every thread must
// call it. Returns the exclusive prefix; *total gets the block sum.
__device__ __forceinline__ int64_t block_excl_scan(int64_t v, int64_t* tmp,
                                                   int64_t* total) {
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  int64_t inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int64_t t = __shfl_up(inc, off);
    if (lane >= off) inc += t;
  }
  __syncthreads();
  if (lane == 63) tmp[wave] = inc;
  __syncthreads();
  int64_t before = 0, all = 0;
  for (int w = 0; w < nw; ++w) {
    int64_t x = tmp[w];
    if (w < wave) before += x;
    all += x;
  }
  *total = all;
  return before + inc - v;
}
#endif

}  // namespace ra
