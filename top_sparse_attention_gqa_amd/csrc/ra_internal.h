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
// Positions per filter / gather tile: one tile is one split-K partial.
constexpr int kTile = 8192;
constexpr int kWordsPerTile = kTile / 64;
// Global histogram stride per head: 4096 fine bins then 64 coarse bins.
constexpr int kFineBins = 4096;
constexpr int kHistStride = kFineBins + 64;
// Candidate list capacity per head (threshold-bucket members).
constexpr int kCandCapMax = 32768;

// Selection modes chosen from the histogram.
constexpr uint32_t kModeCand = 1;     // bucket fits the candidate list
constexpr uint32_t kModeRescan = 2;   // bucket too large: rescan the row

struct HeadState {
  uint32_t b1;        // threshold bucket (fine digit) of the k_eff-th largest
  uint32_t above1;    // members of M with a larger digit
  uint32_t need1;     // how many to take from the bucket
  uint32_t mode;      // kModeCand / kModeRescan / 0 (nothing to select)
  uint32_t cand_count;
  uint32_t pad[3];
};

struct WsLayout {
  int64_t n_cap;    // score row stride (positions), a multiple of kTile
  int32_t n_tiles;  // n_cap / kTile
  int32_t cap;      // candidate capacity per head
  size_t off_scores, off_hist, off_state, off_seqoff, off_tilecnt, off_bitmap,
      off_cand, off_part_mz, off_part_n, total;
};

// Pure host function; returns false for invalid capacities.
bool ws_layout(int32_t B, int32_t H_q, int32_t H_kv, int32_t max_seq_len,
               int32_t k_max, WsLayout* out);

struct Params {
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
  float* scores;
  uint32_t* hist;
  HeadState* state;
  int64_t* seq_off;   // [B + 1] prefix of H_kv * pages(b)
  uint32_t* tile_cnt; // [B*H_q][n_tiles]
  uint64_t* bitmap;   // [B*H_q][n_cap / 64]
  uint64_t* cand;     // [B*H_q][cap]
  float* part_mz;     // [B*H_q][n_tiles][2]  (m, Z)
  float* part_n;      // [B*H_q][n_tiles][128]
  int64_t n_cap;
  int32_t n_tiles;
  int32_t cap;
  int32_t num_cus;
};

// Launchers (each enqueues its kernels on `s`; they never synchronise).
hipError_t launch_prep(const Params& p, hipStream_t s);
hipError_t launch_scan(const Params& p, hipStream_t s);
hipError_t launch_filter(const Params& p, hipStream_t s);
hipError_t launch_resolve(const Params& p, hipStream_t s);
hipError_t launch_gather(const Params& p, hipStream_t s);
hipError_t launch_merge(const Params& p, hipStream_t s);
hipError_t launch_kv_append(const ra_kv_layer& kv, const uint16_t* k_new,
                            const uint16_t* v_new, const int32_t* pos,
                            int32_t B, hipStream_t s);

#if defined(__HIPCC__)
// ---------------------------------------------------------------- device

// Order-preserving map fp32 -> uint32 (larger float, larger key); -0 maps
// like +0 so that equal scores compare equal.
__device__ __forceinline__ uint32_t f2key(float x) {
  x = x + 0.0f;
  uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
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

// Histogram digit width for a GQA group size: 12 bits (4096 fine bins in 64
// coarse bins of 64) up to G = 4, 11 bits for G = 8 so the per-block LDS
// histogram stays at 64 KiB.
__device__ __forceinline__ int hist_bits(int G) { return G <= 4 ? 12 : 11; }

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
