// Exact scores of every cached key for every query head of its GQA group,
// z = q . k / sqrt(128) (RetrievalAttention slides, "Sparse attention
// renormalizes selected tokens", Eq. (1)), streamed once from HBM, plus a
// per-head radix histogram of the scores over the selection domain M that the
// top-k selection starts from.
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
#include "ra_internal.h"

namespace ra {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kScanThreads = 512;
constexpr int kScanWaves = kScanThreads / 64;
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

// ---------------------------------------------------------------- prep
// Clears the global histograms and candidate counters, and writes the
// prefix seq_off[b] = sum_{b' < b} H_kv * pages(b') that maps the scan's
// linear page index to (sequence, KV head, page).
__global__ __launch_bounds__(1024) void prep_kernel(Params p) {
  const size_t heads = size_t(p.B) * p.H_q;
  const size_t n4 = heads * kHistStride / 4;
  uint4* h4 = reinterpret_cast<uint4*>(p.hist);
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n4;
       i += stride)
    h4[i] = make_uint4(0, 0, 0, 0);
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < heads;
       i += stride)
    p.state[i].cand_count = 0;
  if (blockIdx.x != 0) return;
  __shared__ int64_t tmp[16];
  const int per = (p.B + int(blockDim.x) - 1) / int(blockDim.x);
  int64_t s = 0;
  for (int i = 0; i < per; ++i) {
    const int b = threadIdx.x * per + i;
    if (b < p.B) s += int64_t(p.H_kv) * ((seq_geom(p, b).N + kPage - 1) / kPage);
  }
  int64_t total;
  int64_t run = block_excl_scan(s, tmp, &total);
  for (int i = 0; i < per; ++i) {
    const int b = threadIdx.x * per + i;
    if (b < p.B) {
      p.seq_off[b] = run;
      run += int64_t(p.H_kv) * ((seq_geom(p, b).N + kPage - 1) / kPage);
    }
  }
  if (threadIdx.x == 0) p.seq_off[p.B] = total;
}

hipError_t launch_prep(const Params& p, hipStream_t s) {
  const size_t n4 = size_t(p.B) * p.H_q * kHistStride / 4;
  unsigned blocks = unsigned((n4 + 1023) / 1024);
  if (blocks < 1) blocks = 1;
  if (blocks > 256) blocks = 256;
  hipLaunchKernelGGL(prep_kernel, dim3(blocks), dim3(1024), 0, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------- scan
// The linear page index L in [0, seq_off[B]) enumerates (b, g, page) with
// the page fastest. Each block takes one contiguous range of L, processes it
// as runs of one (b, g), and after each run adds its LDS histogram into the
// global per-head histogram (one atomic per non-empty bin).
template <int G>
__global__ __launch_bounds__(kScanThreads) void scan_kernel(Params p) {
  using C = ScanCfg<G>;
  __shared__ uint32_t lhist[G * C::NC * 65];  // 64 fine bins + 1 pad per coarse bin

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int row = lane >> 4;
  const int r = lane & 15;
  const int F = head_of_lane<G>(r);
  const int qsel = r & (C::D - 1);

  for (int i = tid; i < G * C::NC * 65; i += kScanThreads) lhist[i] = 0;
  __syncthreads();

  const int64_t T = p.seq_off[p.B];
  const int64_t L0 = T * blockIdx.x / gridDim.x;
  const int64_t L1 = T * (blockIdx.x + 1) / gridDim.x;
  int64_t L = L0;
  while (L < L1) {
    // sequence: the largest b with seq_off[b] <= L (it has at least one page)
    int blo = 0, bhi = p.B - 1;
    while (blo < bhi) {
      const int mid = (blo + bhi + 1) >> 1;
      if (p.seq_off[mid] <= L) blo = mid; else bhi = mid - 1;
    }
    const int b = blo;
    const SeqGeom sg = seq_geom(p, b);
    const int P = (sg.N + kPage - 1) / kPage;
    const int64_t rel = L - p.seq_off[b];
    const int g = int(rel / P);
    const int j0 = int(rel - int64_t(g) * P);
    const int64_t seg_end = min(L1, p.seq_off[b] + int64_t(g + 1) * P);
    const int npages = int(seg_end - L);

    // this lane's 8 dims of the group's G query heads, slot s = head s ^ F
    uint4 qreg[G];
    const uint16_t* qb = p.q + (size_t(b) * p.H_q + size_t(g) * G) * kHeadDim;
#pragma unroll
    for (int s = 0; s < G; ++s)
      qreg[s] = *reinterpret_cast<const uint4*>(qb + size_t(s ^ F) * kHeadDim + r * 8);

    float* srow = p.scores + (size_t(b) * p.H_q + size_t(g) * G + F) * p.n_cap;
    uint32_t* lh = lhist + F * C::NC * 65;

    for (int jj = wave; jj < npages; jj += kScanWaves) {
      const int j = j0 + jj;
      const int pg = page_of(p, b, j);
      const uint4* kb = reinterpret_cast<const uint4*>(
          p.k_pool + (size_t(pg) * p.H_kv + g) * (kPage * kHeadDim));
      uint4 kd[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) kd[i] = kb[(i * 4 + row) * 16 + r];
      float kept[G];
#pragma unroll
      for (int s = 0; s < G; ++s) kept[s] = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float v[G];
#pragma unroll
        for (int s = 0; s < G; ++s) v[s] = dot8(kd[i], qreg[s]);
        const float x = reduce16<G>(v);
        // after load i, lane (row, r) holds key 4 i + row for head F; the
        // D lanes sharing F take turns keeping it
        if ((i % C::D) == qsel) kept[i / C::D] = x;
      }
      const int nbase = j * kPage;
#pragma unroll
      for (int s = 0; s < G; ++s) {
        const int n = nbase + 4 * (s * C::D + qsel) + row;
        const float z = kept[s] * kInvSqrtD;
        srow[n] = z;
        if (n >= sg.lo && n < sg.hi) {
          const uint32_t dg = f2key(z) >> C::SHIFT;
          atomicAdd(&lh[dg + (dg >> 6)], 1u);
        }
      }
    }
    __syncthreads();
    if (tid < G * C::NC) {
      const int hh = tid / C::NC;
      const int c = tid - hh * C::NC;
      uint32_t* rowp = lhist + (hh * C::NC + c) * 65;
      uint32_t* gh = p.hist + (size_t(b) * p.H_q + size_t(g) * G + hh) * kHistStride;
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
    __syncthreads();
    L = seg_end;
  }
}

hipError_t launch_scan(const Params& p, hipStream_t s) {
  const int64_t pages_max =
      int64_t(p.B) * p.H_kv * ((int64_t(p.max_seq_len) + kPage - 1) / kPage);
  int64_t blocks = (pages_max + kScanWaves - 1) / kScanWaves;
  const int64_t cap = int64_t(2) * (p.num_cus > 0 ? p.num_cus : 256);
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  const dim3 grid{unsigned(blocks)}, block{unsigned(kScanThreads)};
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
