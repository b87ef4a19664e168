// Exact scores of one (page, KV head) block of 64 cached keys for every
// query head of the GQA group, z = q . k / sqrt(128) (RetrievalAttention
// slides, "Sparse attention renormalizes selected tokens", Eq. (1)), by one
// wave. Used by the sampling pass, the scan and the rescan.
//
// Mapping on gfx950 (wave64): the wave reads the block as 16 fully
// coalesced 1 KiB loads; in each load lane l holds 16 bytes (8 dims) of key
// (l / 16). Each lane keeps the same 8 dims of all G query heads of the
// group in registers and forms 8-term partial dot products with
// v_dot2_f32_bf16 (bf16 products are exact in fp32, fp32 accumulation). The
// 16 partials of a key are then summed across the 16-lane row with a
// reduce-scatter over DPP row permutations (mirror, half-mirror, two quad
// swaps): every step halves the number of heads a lane carries, so G heads
// cost G - 1 + 4 - log2(G) DPP adds instead of 4 G. The query slots are
// loaded in a lane-dependent order so that no selects are needed.
#pragma once

#include "ra_internal.h"

namespace ra {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kScanThreads = 512;
constexpr int kScanWaves = kScanThreads / 64;
constexpr float kInvSqrtD = 0.08838834764831845f;  // 1 / sqrt(128)

template <int G>
struct ScanCfg {
  static constexpr int D = 16 / G;  // lanes of a row sharing a head
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

}  // namespace ra
