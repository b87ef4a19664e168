// Exact top-k keys of a block of prefill queries: the input the slides'
// index is built from (RetrievalAttention slides, "Prefill queries teach the
// key graph what matters", step 1: prefill queries find their exact top-k
// keys on the GPU; each query is then linked to those keys). For every query
// row t and query head h: the k_eff largest z = q . k / sqrt(128) (Eq. (1))
// over the domain M of one sequence, ties to the lower position, ascending.
//
// Per KV head the scores form a dense (T G) x N contraction, so they run on
// MFMA: v_mfma_f32_32x32x16_bf16 takes, per lane, 16 contiguous bytes of a
// q row (A) and of a K row (B) and leaves a 32 x 32 tile of fp32 scores. The
// score matrix is never stored; the contraction runs twice:
//   1. page maxima: for every row and page of 64 keys, the largest score
//      over the page's members of M;
//   2. threshold (one wave per row): the k_eff-th largest pair
//      (page maximum, page), ordered by maximum, then lower page first;
//   3. filter: the contraction again; a key is a candidate iff its pair
//      (score, page) is at or above the threshold;
//   4. select (one wave per row): the exact top k_eff of the candidates by
//      (score, lower position), written ascending.
// Every member of the top-k is a candidate: the k_eff pages whose pairs
// clear the threshold each hold a key (their maximum) that beats any key
// whose pair falls below it (a larger score, or an equal one on an earlier
// page). Candidates lie in those k_eff pages only, so a row has at most
// 64 k_eff of them. Both passes issue the same MFMA sequence on the same
// inputs, so a key's score is bit-identical in both.
#include "ra_internal.h"

namespace ra {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kPfWaves = 4;
constexpr int kPfThreads = kPfWaves * 64;
constexpr int kPfRows = kPfWaves * 32;     // query rows per block (32 per wave)
constexpr float kPfScale = 0.08838834764831845f;  // 1 / sqrt(128)

__device__ __forceinline__ int pf_page(const PfParams& p, int j) {
  const int pg = p.block_table[j];
  return ((unsigned)pg < (unsigned)p.num_pages) ? pg : 0;
}

// Row of the score tile held in register r of this lane (MFMA 32x32 layout):
// rows (r / 4) * 8 + (lane / 32) * 4 + r % 4, column lane % 32.
__device__ __forceinline__ int tile_row(int r, int lane) {
  return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}

// Grid (row blocks, H_kv, page splits). Each block: kPfRows query rows of KV
// head blockIdx.y (local row r is query t = r / G, head g G + r % G) against
// the pages of its split. FILTER false: page maxima; true: candidates.
template <int G, bool FILTER>
__global__ __launch_bounds__(kPfThreads) void pf_scores_kernel(PfParams p) {
  const int g = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int TG = p.T * G;
  const int r0 = blockIdx.x * kPfRows + wave * 32;
  if (r0 >= TG) return;  // wave-uniform

  // A fragments: row r0 + lane % 32, dims 16 s + 8 (lane / 32) .. + 8
  bf16x8_t a[8];
  {
    const int ra = r0 + (lane & 31);
    if (ra < TG) {
      const int t = ra / G, hh = ra - (ra / G) * G;
      const uint16_t* qr = p.q + (size_t(t) * p.H_q + size_t(g) * G + hh) * kHeadDim + 8 * (lane >> 5);
#pragma unroll
      for (int s = 0; s < 8; ++s) a[s] = *reinterpret_cast<const bf16x8_t*>(qr + 16 * s);
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) a[s] = bf16x8_t{};
    }
  }
  // the rows this lane's registers hold, as global row indices t H_q + h
  int R[16];
  bool rv[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int lr = r0 + tile_row(r, lane);
    rv[r] = lr < TG;
    const int t = lr / G, hh = lr - (lr / G) * G;
    R[r] = rv[r] ? t * p.H_q + g * G + hh : 0;
  }
  uint64_t tau[16];
  if constexpr (FILTER) {
#pragma unroll
    for (int r = 0; r < 16; ++r) tau[r] = rv[r] ? p.tau[R[r]] : ~0ull;
  }

  const int j0 = int(int64_t(p.P) * blockIdx.z / gridDim.z);
  const int j1 = int(int64_t(p.P) * (blockIdx.z + 1) / gridDim.z);
  for (int j = j0; j < j1; ++j) {
    const uint16_t* kb = p.k_pool + (size_t(pf_page(p, j)) * p.H_kv + g) * (kPage * kHeadDim) +
                         8 * (lane >> 5);
    float m[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) m[r] = -INFINITY;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int col = half * 32 + (lane & 31);  // key within the page
      const int n = j * kPage + col;
      bf16x8_t b[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) b[s] = *reinterpret_cast<const bf16x8_t*>(kb + col * kHeadDim + 16 * s);
      f32x16_t c = {};
#pragma unroll
      for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], b[s], c, 0, 0, 0);
      const bool in_m = n >= p.lo && n < p.hi;
      if constexpr (!FILTER) {
#pragma unroll
        for (int r = 0; r < 16; ++r) m[r] = in_m ? fmaxf(m[r], c[r]) : m[r];
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t key = f2key(c[r] * kPfScale);
          const uint64_t pair = (uint64_t(key) << 32) | uint32_t(~uint32_t(j));
          if (in_m && rv[r] && pair >= tau[r]) {
            const uint32_t slot = atomicAdd(&p.cnt[R[r]], 1u);
            if (slot < uint32_t(p.cap))
              p.cand[size_t(R[r]) * p.cap + slot] = (uint64_t(key) << 32) | uint32_t(~uint32_t(n));
          }
        }
      }
    }
    if constexpr (!FILTER) {
      // maximum over the 32 columns of each half-wave
#pragma unroll
      for (int r = 0; r < 16; ++r) {
#pragma unroll
        for (int off = 1; off < 32; off <<= 1) m[r] = fmaxf(m[r], __shfl_xor(m[r], off));
      }
      if ((lane & 31) == 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (rv[r]) p.pmax[size_t(R[r]) * p.P + j] = m[r] == -INFINITY ? 0u : f2key(m[r] * kPfScale);
      }
    }
  }
}

// ---------------------------------------------------------------- wave select
// The need-th largest of the non-zero values get(0 .. n - 1) (distinct), by
// an 8-bit radix over the 64-bit values held in global memory; hist is this
// wave's 256 LDS bins. Returns a bound t such that exactly `need` of the
// values are >= t. Every lane of the wave calls it with the same arguments.
template <typename Get>
__device__ __forceinline__ uint64_t wave_kth(Get&& get, uint32_t n, uint32_t need, uint32_t* hist) {
  const int lane = lane_id();
  uint64_t prefix = 0;
  int plen = 0;
  for (;;) {
#pragma unroll
    for (int i = 0; i < 4; ++i) hist[lane * 4 + i] = 0u;
    const int sh = 56 - plen;
    for (uint32_t i = lane; i < n; i += 64) {
      const uint64_t v = get(i);
      if (v != 0ull && (plen == 0 || (v >> (64 - plen)) == prefix))
        atomicAdd(&hist[uint32_t(v >> sh) & 255u], 1u);
    }
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
    prefix = (prefix << 8) | digit;
    plen += 8;
    need -= above;
    if (cd == need || plen == 64) return prefix << (64 - plen);
  }
}

// One wave per row: the threshold pair over the row's page maxima, and the
// row's candidate count reset.
constexpr int kPfSelWaves = 4;

__global__ __launch_bounds__(kPfSelWaves * 64) void pf_threshold_kernel(PfParams p) {
  __shared__ uint32_t s_hist[kPfSelWaves][256];
  const int wave = threadIdx.x >> 6;
  const int R = blockIdx.x * kPfSelWaves + wave;
  if (R >= p.T * p.H_q) return;
  const uint32_t* pm = p.pmax + size_t(R) * p.P;
  auto pair = [&](uint32_t j) -> uint64_t {
    const uint32_t key = pm[j];
    return key ? (uint64_t(key) << 32) | uint32_t(~j) : 0ull;
  };
  uint32_t present = 0;
  for (uint32_t j = lane_id(); j < uint32_t(p.P); j += 64) present += pm[j] ? 1u : 0u;
  present = wave_sum(present);
  uint64_t t;
  if (p.k_eff == 0)
    t = ~0ull;                      // nothing is retrieved
  else if (present <= uint32_t(p.k_eff))
    t = 1ull;                       // every member of M is a candidate
  else
    t = wave_kth(pair, uint32_t(p.P), uint32_t(p.k_eff), s_hist[wave]);
  if (lane_id() == 0) {
    p.tau[R] = t;
    p.cnt[R] = 0u;
  }
}

// One wave per row: the exact top k_eff of the row's candidates, ascending.
__global__ __launch_bounds__(kPfSelWaves * 64) void pf_select_kernel(PfParams p) {
  __shared__ uint32_t s_hist[kPfSelWaves][256];
  __shared__ int32_t s_pos[kPfSelWaves][RA_PREFILL_MAX_K];
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  const int R = blockIdx.x * kPfSelWaves + wave;
  if (R >= p.T * p.H_q) return;
  int32_t* out = p.out_idx + size_t(R) * p.k;
  const uint32_t ke = uint32_t(p.k_eff);
  if (ke > 0) {
    const uint32_t n = min(p.cnt[R], uint32_t(p.cap));
    const uint64_t* cl = p.cand + size_t(R) * p.cap;
    auto get = [&](uint32_t i) -> uint64_t { return cl[i]; };
    const uint64_t th = n > ke ? wave_kth(get, n, ke, s_hist[wave]) : 1ull;
    // the winners' positions, in list order
    uint32_t filled = 0;
    for (uint32_t base = 0; base < n; base += 64) {
      const uint32_t i = base + lane;
      const uint64_t v = i < n ? cl[i] : 0ull;
      const bool win = i < n && v >= th;
      const uint64_t m = __ballot(win);
      const uint32_t at = filled + uint32_t(__popcll(m & ((1ull << lane) - 1ull)));
      if (win && at < ke) s_pos[wave][at] = int32_t(~uint32_t(v));
      filled += uint32_t(__popcll(m));
    }
    // ascending: each winner's rank is the number of smaller positions
    for (uint32_t i = lane; i < ke; i += 64) {
      const int32_t x = s_pos[wave][i];
      uint32_t rank = 0;
      for (uint32_t j = 0; j < ke; ++j) rank += s_pos[wave][j] < x ? 1u : 0u;
      out[rank] = x;
    }
  }
  for (int i = int(ke) + lane; i < p.k; i += 64) out[i] = -1;
}

// ---------------------------------------------------------------- launch
template <int G>
static void launch_pf_scores(const PfParams& p, bool filter, hipStream_t s) {
  const unsigned row_blocks = unsigned((int64_t(p.T) * G + kPfRows - 1) / kPfRows);
  const dim3 grid{row_blocks, unsigned(p.H_kv), unsigned(p.splits)};
  if (filter)
    hipLaunchKernelGGL((pf_scores_kernel<G, true>), grid, dim3(kPfThreads), 0, s, p);
  else
    hipLaunchKernelGGL((pf_scores_kernel<G, false>), grid, dim3(kPfThreads), 0, s, p);
}

hipError_t launch_prefill(const PfParams& p, int first, int last, hipStream_t s) {
  const int G = p.H_q / p.H_kv;
  const unsigned row_waves = unsigned((int64_t(p.T) * p.H_q + kPfSelWaves - 1) / kPfSelWaves);
  for (int st = first; st <= last; ++st) {
    if (st == 0 || st == 2) {
      switch (G) {
        case 1: launch_pf_scores<1>(p, st == 2, s); break;
        case 2: launch_pf_scores<2>(p, st == 2, s); break;
        case 4: launch_pf_scores<4>(p, st == 2, s); break;
        case 8: launch_pf_scores<8>(p, st == 2, s); break;
        default: return hipErrorInvalidValue;
      }
    } else if (st == 1) {
      hipLaunchKernelGGL(pf_threshold_kernel, dim3(row_waves), dim3(kPfSelWaves * 64), 0, s, p);
    } else {
      hipLaunchKernelGGL(pf_select_kernel, dim3(row_waves), dim3(kPfSelWaves * 64), 0, s, p);
    }
  }
  return hipGetLastError();
}

}  // namespace ra
