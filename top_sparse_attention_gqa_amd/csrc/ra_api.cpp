// Host side of the C ABI: argument validation (pure host code, no HIP call
// before it passes), workspace carving and the launch sequence of one decode
// step. Every kernel is enqueued on the caller's stream; nothing here
// allocates, synchronises or reads device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <numeric>
#include <vector>

#include "ra.h"
#include "ra_internal.h"

namespace ra {

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool ws_layout(int32_t B, int32_t H_q, int32_t H_kv, int32_t max_seq_len,
               int32_t k_max, WsLayout* L) {
  if (B <= 0 || B > RA_MAX_BATCH || H_q <= 0 || H_kv <= 0 || H_q % H_kv != 0)
    return false;
  if (max_seq_len <= 0 || max_seq_len > RA_MAX_SEQ_LEN || k_max < 0)
    return false;
  const int64_t heads = int64_t(B) * H_q;
  if (heads > 65535) return false;  // grid y limit of the per-head kernels
  // Row stride of the per-head score and candidate rows: a whole number of
  // tile pairs. With an odd number of tiles per row (for lengths just past
  // 2^20: 2^20 + 8192 entries, a 64 KB offset between heads' candidate rows
  // mod 128 KB) the scan, which writes those rows while it streams K,
  // measured 5 % slower; an even number showed no such loss.
  L->n_cap = (int64_t(max_seq_len) + 2 * kTile - 1) / (2 * kTile) * (2 * kTile);
  L->n_tiles = int32_t(L->n_cap / kUnit);  // tiles of the smallest size (one unit)
  L->n_units = int32_t(L->n_cap / kUnit);
  // sampled_pages(P) is not monotone below 2048 pages (the stride doubles
  // as P grows) but stays <= 64 there, and is monotone above.
  L->samp_cap = std::max(64, sampled_pages((max_seq_len + kPage - 1) / kPage)) * kPage;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  L->off_scores = take(size_t(heads) * L->n_cap * sizeof(float));
  L->off_samp = take(size_t(heads) * L->samp_cap * sizeof(uint32_t));
  L->off_state = take(size_t(heads) * sizeof(HeadState));
  L->off_gdone = take(size_t(B) * H_kv * sizeof(uint32_t));
  L->off_misc = take(64);
  L->off_unitoff = take(size_t(B + 1) * sizeof(int64_t));
  L->off_ucnt = take(size_t(heads) * L->n_units * sizeof(uint32_t));
  L->off_scnt = take(size_t(heads) * L->n_tiles * sizeof(uint32_t));
  L->off_cand = take(size_t(heads) * L->n_cap * sizeof(uint64_t));
  L->off_part_mz = take(size_t(heads) * L->n_tiles * 2 * sizeof(float));
  L->off_part_n = take(size_t(heads) * L->n_tiles * kHeadDim * sizeof(float));
  L->total = off;
  return true;
}

bool pf_layout(int32_t T, int32_t H_q, int32_t N, int32_t k, PfLayout* L) {
  if (T <= 0 || H_q <= 0 || N <= 0 || N > RA_MAX_SEQ_LEN || k < 0 || k > RA_PREFILL_MAX_K)
    return false;
  const int64_t rows = int64_t(T) * H_q;
  if (rows > (int64_t(1) << 30)) return false;
  const int64_t P = (int64_t(N) + kPage - 1) / kPage;
  const int64_t Ppad = (P + kPfChunk - 1) / kPfChunk * kPfChunk;
  // 64 per page of the exact threshold's k pages, and room for the sampled
  // bound's larger candidate sets at small k
  const int64_t cap = int64_t(kPage) * std::max<int64_t>(k, kPfMinCapPages);
  L->cap = cap;
  const int64_t Ps_pad = (pf_sampled_pages(int(P)) + kPfChunk - 1) / kPfChunk * kPfChunk;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  L->off_pmax = take(size_t(rows) * Ppad * sizeof(uint32_t));
  L->off_tau = take(size_t(rows) * sizeof(uint64_t));
  L->off_seg_off = take(size_t(rows) * kPfMaxSplits * sizeof(uint32_t));
  L->off_seg_cnt = take(size_t(rows) * kPfMaxSplits * sizeof(uint32_t));
  L->off_cand = take(size_t(rows) * cap * sizeof(uint64_t));
  L->off_smax = take(size_t(rows) * Ps_pad * sizeof(uint32_t));
  L->off_fail = take(size_t(rows) * sizeof(uint32_t));
  L->total = off;
  return true;
}

static int cu_count() {
  // CU count per device, read once.
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> g(mu);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
            hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// Vector loads need 16-byte aligned rows; scalar arrays need their element
// alignment.
static bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

static ra_status check_kv(const ra_kv_layer* kv) {
  if (!kv || !kv->k_pool || !kv->v_pool || !kv->block_table)
    return RA_ERR_INVALID_ARGUMENT;
  if (!aligned(kv->k_pool, 16) || !aligned(kv->v_pool, 16) ||
      !aligned(kv->block_table, 4))
    return RA_ERR_INVALID_ARGUMENT;
  if (kv->num_pages <= 0 || kv->max_pages <= 0 || kv->H_kv <= 0)
    return RA_ERR_INVALID_ARGUMENT;
  if (kv->head_dim != RA_HEAD_DIM || kv->page_size != RA_PAGE_SIZE)
    return RA_ERR_UNSUPPORTED;
  return RA_OK;
}

static ra_status validate_decode(const uint16_t* q, int32_t H_q,
                                 const ra_kv_layer* kv, const int32_t* seq_lens,
                                 int32_t B, int32_t max_seq_len,
                                 const int32_t* k, int32_t k_max,
                                 int32_t n_sink, int32_t window, float* out,
                                 int32_t* out_idx, void* ws, size_t ws_bytes,
                                 WsLayout* L) {
  ra_status st = check_kv(kv);
  if (st != RA_OK) return st;
  if (!q || !seq_lens || !k || !out || !ws) return RA_ERR_INVALID_ARGUMENT;
  if (k_max > 0 && !out_idx) return RA_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(seq_lens, 4) || !aligned(k, 4) ||
      !aligned(out, 4) || (out_idx && !aligned(out_idx, 4)))
    return RA_ERR_INVALID_ARGUMENT;
  if (B <= 0 || B > RA_MAX_BATCH || H_q <= 0 || max_seq_len <= 0 ||
      max_seq_len > RA_MAX_SEQ_LEN || k_max < 0 || n_sink < 0 || window < 0)
    return RA_ERR_INVALID_ARGUMENT;
  if (H_q % kv->H_kv != 0) return RA_ERR_INVALID_ARGUMENT;
  const int G = H_q / kv->H_kv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return RA_ERR_UNSUPPORTED;
  if (reinterpret_cast<uintptr_t>(ws) & 255) return RA_ERR_INVALID_ARGUMENT;
  if (!ws_layout(B, H_q, kv->H_kv, max_seq_len, k_max, L))
    return RA_ERR_INVALID_ARGUMENT;
  if (ws_bytes < L->total) return RA_ERR_WORKSPACE;
  return RA_OK;
}

static Params make_params(const uint16_t* q, int32_t H_q, const ra_kv_layer* kv,
                          const int32_t* seq_lens, int32_t B,
                          int32_t max_seq_len, const int32_t* k, int32_t k_max,
                          int32_t n_sink, int32_t window, float* out,
                          float* out_lse, int32_t* out_idx, void* ws,
                          const WsLayout& L) {
  Params p{};
  char* base = static_cast<char*>(ws);
  p.q = q;
  p.k_pool = kv->k_pool;
  p.v_pool = kv->v_pool;
  p.block_table = kv->block_table;
  p.seq_lens = seq_lens;
  p.kk = k;
  p.out = out;
  p.lse = out_lse;
  p.out_idx = out_idx;
  p.B = B;
  p.H_q = H_q;
  p.H_kv = kv->H_kv;
  p.G = H_q / kv->H_kv;
  p.max_pages = kv->max_pages;
  p.num_pages = kv->num_pages;
  p.max_seq_len = max_seq_len;
  p.k_max = k_max;
  p.n_sink = n_sink;
  p.window = window;
  p.scores = reinterpret_cast<float*>(base + L.off_scores);
  p.samp = reinterpret_cast<uint32_t*>(base + L.off_samp);
  p.state = reinterpret_cast<HeadState*>(base + L.off_state);
  p.gdone = reinterpret_cast<uint32_t*>(base + L.off_gdone);
  p.any_dense = reinterpret_cast<uint32_t*>(base + L.off_misc);
  p.dbg = reinterpret_cast<uint32_t*>(base + L.off_misc + 4);
  p.unit_off = reinterpret_cast<int64_t*>(base + L.off_unitoff);
  p.ucnt = reinterpret_cast<uint32_t*>(base + L.off_ucnt);
  p.scnt = reinterpret_cast<uint32_t*>(base + L.off_scnt);
  p.cand = reinterpret_cast<uint64_t*>(base + L.off_cand);
  p.part_mz = reinterpret_cast<float*>(base + L.off_part_mz);
  p.part_n = reinterpret_cast<float*>(base + L.off_part_n);
  p.n_cap = L.n_cap;
  p.n_tiles = L.n_tiles;
  p.n_units = L.n_units;
  p.samp_cap = L.samp_cap;
  return p;
}

// ------------------------------------------------------------------
// Workspace of ra_decode_step_noalloc: a file-scope device array, one copy
// per GPU the library runs on, held until the process ends. In host code
// `scratch` names a host-side stand-in, never a device address: its device
// address comes from hipGetSymbolAddress, taken once per device (with that
// device current) on the entry point's first call there, and only that
// address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[RA_NOALLOC_WS_BYTES];

constexpr int kMaxDevices = 64;

// The device address of `scratch` on the current device, or null.
static void* scratch_on_current_device() {
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> g(mu);
  if (ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();  // clear the sticky error
      return nullptr;
    }
    ptr[dev] = p;
  }
  return ptr[dev];
}

}  // namespace ra

using namespace ra;

extern "C" {

int ra_abi_version(void) { return RA_ABI_VERSION; }

const char* ra_status_str(ra_status s) {
  switch (s) {
    case RA_OK: return "RA_OK";
    case RA_ERR_INVALID_ARGUMENT: return "RA_ERR_INVALID_ARGUMENT";
    case RA_ERR_WORKSPACE: return "RA_ERR_WORKSPACE";
    case RA_ERR_UNSUPPORTED: return "RA_ERR_UNSUPPORTED";
    case RA_ERR_HIP: return "RA_ERR_HIP";
  }
  return "RA_ERR_UNKNOWN";
}

size_t ra_decode_workspace_bytes(int32_t B, int32_t H_q, int32_t H_kv,
                                 int32_t max_seq_len, int32_t k_max) {
  WsLayout L;
  if (!ws_layout(B, H_q, H_kv, max_seq_len, k_max, &L)) return 0;
  return L.total;
}

size_t ra_workspace_scores_offset(int32_t B, int32_t H_q, int32_t H_kv,
                                  int32_t max_seq_len, int32_t k_max,
                                  int64_t* row_stride) {
  WsLayout L;
  if (!ws_layout(B, H_q, H_kv, max_seq_len, k_max, &L)) return size_t(-1);
  if (row_stride) *row_stride = L.n_cap;
  return L.off_scores;
}

size_t ra_workspace_rescan_count_offset(int32_t B, int32_t H_q, int32_t H_kv,
                                        int32_t max_seq_len, int32_t k_max) {
  WsLayout L;
  if (!ws_layout(B, H_q, H_kv, max_seq_len, k_max, &L)) return size_t(-1);
  return L.off_misc;  // any_dense; the next word holds a debug build's failed checks
}

ra_status ra_kv_append(const ra_kv_layer* kv, const uint16_t* k_new,
                       const uint16_t* v_new, const int32_t* pos, int32_t B,
                       hipStream_t stream) {
  ra_status st = check_kv(kv);
  if (st != RA_OK) return st;
  if (!k_new || !v_new || !pos || B <= 0 || B > RA_MAX_BATCH)
    return RA_ERR_INVALID_ARGUMENT;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(pos, 4))
    return RA_ERR_INVALID_ARGUMENT;
  if (launch_kv_append(*kv, k_new, v_new, pos, B, stream) != hipSuccess)
    return RA_ERR_HIP;
  return RA_OK;
}

ra_status ra_decode_stages(const uint16_t* q, int32_t H_q,
                           const ra_kv_layer* kv, const int32_t* seq_lens,
                           int32_t B, int32_t max_seq_len, const int32_t* k,
                           int32_t k_max, int32_t n_sink, int32_t window,
                           float* out, float* out_lse, int32_t* out_idx,
                           void* ws, size_t ws_bytes, uint32_t flags,
                           int32_t first_stage, int32_t last_stage,
                           hipStream_t stream) {
  WsLayout L;
  ra_status st = validate_decode(q, H_q, kv, seq_lens, B, max_seq_len, k,
                                 k_max, n_sink, window, out, out_idx, ws,
                                 ws_bytes, &L);
  if (st != RA_OK) return st;
  if (flags & ~RA_DECODE_KEEP_SCORES) return RA_ERR_INVALID_ARGUMENT;
  if (first_stage < 0 || last_stage >= RA_STAGE_COUNT ||
      first_stage > last_stage)
    return RA_ERR_INVALID_ARGUMENT;
  Params p = make_params(q, H_q, kv, seq_lens, B, max_seq_len, k, k_max,
                         n_sink, window, out, out_lse, out_idx, ws, L);
  p.num_cus = cu_count();
  p.keep_scores = (flags & RA_DECODE_KEEP_SCORES) ? 1 : 0;
  using Launcher = hipError_t (*)(const Params&, hipStream_t);
  static const Launcher stages[RA_STAGE_COUNT] = {
      launch_sample, launch_threshold, launch_scan,
      launch_select, launch_gather,    launch_merge};
  // with the scan in the same call, the scan may compute the bounds; a scan
  // that follows the threshold launch in the same call finds them published
  const bool thr_here = first_stage <= RA_STAGE_THRESHOLD && last_stage >= RA_STAGE_THRESHOLD;
  const bool fuse = thr_here && last_stage >= RA_STAGE_SCAN && scan_computes_bounds(p);
  p.scan_bounds = (thr_here && !fuse) ? 0 : 1;
  for (int s = first_stage; s <= last_stage; ++s) {
    if (s == RA_STAGE_THRESHOLD && fuse) continue;
    if (stages[s](p, stream) != hipSuccess) return RA_ERR_HIP;
  }
  return RA_OK;
}

ra_status ra_append_decode_step(const uint16_t* k_new, const uint16_t* v_new,
                                const int32_t* pos, const uint16_t* q, int32_t H_q,
                                const ra_kv_layer* kv, const int32_t* seq_lens, int32_t B,
                                int32_t max_seq_len, const int32_t* k, int32_t k_max,
                                int32_t n_sink, int32_t window, float* out, float* out_lse,
                                int32_t* out_idx, void* ws, size_t ws_bytes, uint32_t flags,
                                hipStream_t stream) {
  if (!k_new || !v_new || !pos) return RA_ERR_INVALID_ARGUMENT;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(pos, 4))
    return RA_ERR_INVALID_ARGUMENT;
  WsLayout L;
  ra_status st = validate_decode(q, H_q, kv, seq_lens, B, max_seq_len, k,
                                 k_max, n_sink, window, out, out_idx, ws,
                                 ws_bytes, &L);
  if (st != RA_OK) return st;
  if (flags & ~RA_DECODE_KEEP_SCORES) return RA_ERR_INVALID_ARGUMENT;
  Params p = make_params(q, H_q, kv, seq_lens, B, max_seq_len, k, k_max,
                         n_sink, window, out, out_lse, out_idx, ws, L);
  p.num_cus = cu_count();
  p.keep_scores = (flags & RA_DECODE_KEEP_SCORES) ? 1 : 0;
  p.app_k = k_new;
  p.app_v = v_new;
  p.app_pos = pos;
  p.scan_bounds = scan_computes_bounds(p) ? 1 : 0;
  if (launch_sample(p, stream) != hipSuccess ||
      (!p.scan_bounds && launch_threshold(p, stream) != hipSuccess) ||
      launch_scan(p, stream) != hipSuccess || launch_select(p, stream) != hipSuccess ||
      launch_gather(p, stream) != hipSuccess || launch_merge(p, stream) != hipSuccess)
    return RA_ERR_HIP;
  return RA_OK;
}

ra_status ra_decode_step_ex(const uint16_t* q, int32_t H_q, const ra_kv_layer* kv,
                            const int32_t* seq_lens, int32_t B,
                            int32_t max_seq_len, const int32_t* k, int32_t k_max,
                            int32_t n_sink, int32_t window, float* out,
                            float* out_lse, int32_t* out_idx, void* ws,
                            size_t ws_bytes, uint32_t flags, hipStream_t stream) {
  return ra_decode_stages(q, H_q, kv, seq_lens, B, max_seq_len, k, k_max,
                          n_sink, window, out, out_lse, out_idx, ws, ws_bytes,
                          flags, RA_STAGE_SAMPLE, RA_STAGE_MERGE, stream);
}

ra_status ra_decode_step_noalloc(const uint16_t* q, int32_t H_q, const ra_kv_layer* kv,
                                 const int32_t* seq_lens, int32_t B, int32_t max_seq_len,
                                 const int32_t* k, int32_t k_max, int32_t n_sink,
                                 int32_t window, float* out, float* out_lse, int32_t* out_idx,
                                 uint32_t flags, hipStream_t stream) {
  // sizes beyond the array are rejected before anything else is looked at
  WsLayout L;
  if (kv != nullptr && ws_layout(B, H_q, kv->H_kv, max_seq_len, k_max, &L) &&
      L.total > size_t(RA_NOALLOC_WS_BYTES))
    return RA_ERR_WORKSPACE;
  void* ws = scratch_on_current_device();
  if (ws == nullptr) return RA_ERR_HIP;
  return ra_decode_step_ex(q, H_q, kv, seq_lens, B, max_seq_len, k, k_max, n_sink, window,
                           out, out_lse, out_idx, ws, size_t(RA_NOALLOC_WS_BYTES), flags,
                           stream);
}

ra_status ra_decode_step(const uint16_t* q, int32_t H_q, const ra_kv_layer* kv,
                         const int32_t* seq_lens, int32_t B,
                         int32_t max_seq_len, const int32_t* k, int32_t k_max,
                         int32_t n_sink, int32_t window, float* out,
                         int32_t* out_idx, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  return ra_decode_step_ex(q, H_q, kv, seq_lens, B, max_seq_len, k, k_max, n_sink,
                           window, out, nullptr, out_idx, ws, ws_bytes, 0u, stream);
}

size_t ra_prefill_workspace_fail_offset(int32_t T, int32_t H_q, int32_t N, int32_t k) {
  PfLayout L;
  if (!pf_layout(T, H_q, N, k, &L)) return 0;
  return L.off_fail;
}

size_t ra_prefill_workspace_bytes(int32_t T, int32_t H_q, int32_t N, int32_t k) {
  PfLayout L;
  if (!pf_layout(T, H_q, N, k, &L)) return 0;
  return L.total;
}

ra_status ra_prefill_topk(const uint16_t* q, int32_t T, int32_t H_q,
                          const ra_kv_layer* kv, int32_t seq, int32_t N,
                          int32_t k, int32_t n_sink, int32_t window,
                          int32_t* out_idx, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  return ra_prefill_stages(q, T, H_q, kv, seq, N, k, n_sink, window, out_idx, ws,
                           ws_bytes, RA_PF_STAGE_SAMPLE, RA_PF_STAGE_EXACT_SELECT, stream);
}

ra_status ra_prefill_stages(const uint16_t* q, int32_t T, int32_t H_q,
                            const ra_kv_layer* kv, int32_t seq, int32_t N,
                            int32_t k, int32_t n_sink, int32_t window,
                            int32_t* out_idx, void* ws, size_t ws_bytes,
                            int32_t first_stage, int32_t last_stage,
                            hipStream_t stream) {
  ra_status st = check_kv(kv);
  if (st != RA_OK) return st;
  if (!q || !ws || (k > 0 && !out_idx)) return RA_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || (out_idx && !aligned(out_idx, 4)) || !aligned(ws, 256))
    return RA_ERR_INVALID_ARGUMENT;
  if (T <= 0 || H_q <= 0 || seq < 0 || n_sink < 0 || window < 0 || k < 0 ||
      k > RA_PREFILL_MAX_K)
    return RA_ERR_INVALID_ARGUMENT;
  if (H_q % kv->H_kv != 0) return RA_ERR_INVALID_ARGUMENT;
  const int G = H_q / kv->H_kv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return RA_ERR_UNSUPPORTED;
  if (N <= 0 || int64_t(N) > int64_t(kv->max_pages) * kPage) return RA_ERR_INVALID_ARGUMENT;
  PfLayout L;
  if (!pf_layout(T, H_q, N, k, &L)) return RA_ERR_INVALID_ARGUMENT;
  if (ws_bytes < L.total) return RA_ERR_WORKSPACE;
  if (first_stage < 0 || last_stage >= RA_PF_STAGE_COUNT || first_stage > last_stage)
    return RA_ERR_INVALID_ARGUMENT;
  if (k == 0) return RA_OK;  // nothing to retrieve, nothing to write
  PfParams p{};
  char* base = static_cast<char*>(ws);
  p.q = q;
  p.k_pool = kv->k_pool;
  p.block_table = kv->block_table + size_t(seq) * kv->max_pages;
  p.T = T;
  p.H_q = H_q;
  p.H_kv = kv->H_kv;
  p.N = N;
  p.P = (N + kPage - 1) / kPage;
  p.num_pages = kv->num_pages;
  p.lo = std::min(n_sink, N);
  p.hi = std::max(N - window, p.lo);
  p.k = k;
  p.k_eff = std::min(k, p.hi - p.lo);
  p.cap = int32_t(L.cap);
  p.pmax = reinterpret_cast<uint32_t*>(base + L.off_pmax);
  p.smax = reinterpret_cast<uint32_t*>(base + L.off_smax);
  p.fail = reinterpret_cast<uint32_t*>(base + L.off_fail);
  p.tau = reinterpret_cast<uint64_t*>(base + L.off_tau);
  p.seg_off = reinterpret_cast<uint32_t*>(base + L.off_seg_off);
  p.seg_cnt = reinterpret_cast<uint32_t*>(base + L.off_seg_cnt);
  p.cand = reinterpret_cast<uint64_t*>(base + L.off_cand);
  p.out_idx = out_idx;
  p.Ppad = (p.P + kPfChunk - 1) / kPfChunk * kPfChunk;
  // one contraction block per CU: split the page chunks over enough blocks
  // to fill the GPU; the row blocks of one page range share an XCD (its L2)
  // when the (KV head, range) pairs divide evenly over the eight XCDs
  const int64_t chunks = p.Ppad / kPfChunk;
  p.row_blocks = int32_t((int64_t(T) * G + kPfBlockRows - 1) / kPfBlockRows);
  const int64_t have = int64_t(p.row_blocks) * kv->H_kv;
  const int64_t S_max = std::min<int64_t>(chunks, kPfMaxSplits);
  int64_t S = std::max<int64_t>(1, std::min<int64_t>(S_max, (cu_count() + have - 1) / have));
  const int64_t step = 8 / std::gcd<int64_t>(kv->H_kv, 8);
  const int64_t S8 = (S + step - 1) / step * step;
  if (S8 <= S_max) S = S8;
  p.splits = int32_t(S);
  p.xcd_groups = (int64_t(kv->H_kv) * S) % 8 == 0 ? 1 : 0;
  // The sampled bound is the R-th largest maximum over the sampled pages
  // (one page in 8). About 8 R pages of the row then have a maximum at or
  // above it, with a spread of about 8 sqrt(R) for keys in no particular
  // order; R is the least with R - z sqrt(R) >= k_eff / 8, z = 4.5, so that
  // fewer than k_eff candidates (the row then falls to the exact pass) is a
  // 4.5-sigma event.
  p.Ps = int32_t(pf_sampled_pages(p.P));
  p.Ps_pad = int32_t((p.Ps + kPfChunk - 1) / kPfChunk * kPfChunk);
  {
    const double z = 4.5, kf = double(p.k_eff) * double(p.Ps) / double(p.P);
    const double r = 0.5 * z + std::sqrt(0.25 * z * z + kf);
    p.need_s = int32_t(std::ceil(r * r));
  }
  p.seg_cap = int32_t(p.cap / S);
  if (launch_prefill(p, first_stage, last_stage, stream) != hipSuccess) return RA_ERR_HIP;
  return RA_OK;
}

ra_status ra_layer_budgets(int32_t n_layers, int32_t k_mean, int32_t slope_permille,
                           int32_t* k_out) {
  if (!k_out || n_layers <= 0 || n_layers > 4096 || k_mean < 0 || slope_permille < 0 ||
      slope_permille > 1000)
    return RA_ERR_INVALID_ARGUMENT;
  const int64_t L = n_layers;
  if (L == 1) {
    k_out[0] = k_mean;
    return RA_OK;
  }
  // k_l = num_l / den exactly; num_l >= 0 since the slope is at most 1
  const int64_t den = 1000 * (L - 1);
  std::vector<int64_t> rem(static_cast<size_t>(L), 0);
  int64_t left = L * k_mean;
  for (int64_t l = 0; l < L; ++l) {
    const int64_t num = int64_t(k_mean) * (den + int64_t(slope_permille) * (L - 1 - 2 * l));
    k_out[l] = int32_t(num / den);
    rem[size_t(l)] = num % den;
    left -= num / den;
  }
  // the fractional parts sum to `left` (< L): one more for the largest ones
  std::vector<int32_t> order(static_cast<size_t>(L));
  for (int32_t l = 0; l < n_layers; ++l) order[size_t(l)] = l;
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t a, int32_t b) { return rem[size_t(a)] > rem[size_t(b)]; });
  for (int64_t i = 0; i < left; ++i) ++k_out[order[size_t(i)]];
  return RA_OK;
}

ra_status ra_graph_build(const int32_t* hubs, const int32_t* lists, int32_t T, int32_t K,
                         int32_t N, int32_t D, int32_t* nbr, int32_t* entry) {
  if (!nbr || !entry || (T > 0 && (!hubs || !lists)) || T < 0 || K < 1 || N < 1 || D < 1 ||
      D > RA_GRAPH_MAX_DEGREE)
    return RA_ERR_INVALID_ARGUMENT;
  for (int64_t i = 0; i < int64_t(T); ++i)
    if (hubs[i] < -1 || hubs[i] >= N) return RA_ERR_INVALID_ARGUMENT;
  for (int64_t i = 0; i < int64_t(T) * K; ++i)
    if (lists[i] < -1 || lists[i] >= N) return RA_ERR_INVALID_ARGUMENT;
  std::fill(nbr, nbr + size_t(N) * D, -1);
  std::vector<int32_t> deg(static_cast<size_t>(N), 0), hub_count(static_cast<size_t>(N), 0);
  auto link = [&](int32_t a, int32_t b) {
    int32_t* row = nbr + size_t(a) * D;
    int32_t& n = deg[size_t(a)];
    if (a == b || n >= D) return;
    for (int32_t i = 0; i < n; ++i)
      if (row[i] == b) return;
    row[n++] = b;
  };
  std::vector<int32_t> keys(static_cast<size_t>(K));
  for (int32_t t = 0; t < T; ++t) {
    const int32_t a = hubs[t];
    if (a < 0) continue;
    ++hub_count[size_t(a)];
    const int32_t* L = lists + size_t(t) * K;
    keys.assign(L, L + K);
    std::sort(keys.begin(), keys.end());
    for (int32_t b : keys) {
      if (b < 0 || b == a) continue;
      link(a, b);
      link(b, a);
    }
  }
  int32_t best = -1;
  for (int32_t a = 0; a < N; ++a)
    if (hub_count[size_t(a)] > 0 && (best < 0 || hub_count[size_t(a)] > hub_count[size_t(best)]))
      best = a;
  *entry = best;
  return RA_OK;
}

ra_status ra_graph_search(const uint16_t* q, int32_t H_q, const ra_kv_layer* kv, int32_t seq,
                          int32_t N, const int32_t* nbr, int32_t D, const int32_t* entry,
                          int32_t ef, int32_t k, int32_t* out_idx, int32_t* out_visited,
                          hipStream_t stream) {
  ra_status st = check_kv(kv);
  if (st != RA_OK) return st;
  if (!q || !nbr || !entry || !out_idx || !out_visited) return RA_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(nbr, 4) || !aligned(out_idx, 4) || !aligned(entry, 4) ||
      !aligned(out_visited, 4))
    return RA_ERR_INVALID_ARGUMENT;
  if (H_q <= 0 || seq < 0 || D < 1 || D > RA_GRAPH_MAX_DEGREE || k < 1 || ef < k ||
      ef > RA_GRAPH_MAX_EF)
    return RA_ERR_INVALID_ARGUMENT;
  if (H_q % kv->H_kv != 0) return RA_ERR_INVALID_ARGUMENT;
  if (N <= 0 || N > RA_GRAPH_MAX_N || int64_t(N) > int64_t(kv->max_pages) * kPage)
    return RA_ERR_INVALID_ARGUMENT;
  GsParams p{};
  p.q = q;
  p.k_pool = kv->k_pool;
  p.block_table = kv->block_table + size_t(seq) * kv->max_pages;
  p.H_q = H_q;
  p.H_kv = kv->H_kv;
  p.N = N;
  p.num_pages = kv->num_pages;
  p.nbr = nbr;
  p.entry = entry;
  p.D = D;
  p.ef = ef;
  p.k = k;
  p.vis_words = (N + 31) / 32;
  p.out_idx = out_idx;
  p.out_visited = out_visited;
  if (launch_graph_search(p, stream) != hipSuccess) return RA_ERR_HIP;
  return RA_OK;
}

ra_status ra_sparse_attend(const uint16_t* q, int32_t H_q, const ra_kv_layer* kv, int32_t seq,
                           int32_t N, const int32_t* idx, int32_t k, float* out, float* out_lse,
                           hipStream_t stream) {
  ra_status st = check_kv(kv);
  if (st != RA_OK) return st;
  if (!q || !idx || !out || !out_lse) return RA_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(idx, 4) || !aligned(out, 4) || !aligned(out_lse, 4))
    return RA_ERR_INVALID_ARGUMENT;
  if (H_q <= 0 || seq < 0 || k < 1 || k > RA_SPARSE_MAX_K) return RA_ERR_INVALID_ARGUMENT;
  if (H_q % kv->H_kv != 0) return RA_ERR_INVALID_ARGUMENT;
  if (N <= 0 || int64_t(N) > int64_t(kv->max_pages) * kPage) return RA_ERR_INVALID_ARGUMENT;
  SaParams p{};
  p.q = q;
  p.k_pool = kv->k_pool;
  p.v_pool = kv->v_pool;
  p.block_table = kv->block_table + size_t(seq) * kv->max_pages;
  p.H_q = H_q;
  p.H_kv = kv->H_kv;
  p.N = N;
  p.num_pages = kv->num_pages;
  p.k = k;
  p.idx = idx;
  p.out = out;
  p.out_lse = out_lse;
  if (launch_sparse_attend(p, stream) != hipSuccess) return RA_ERR_HIP;
  return RA_OK;
}

ra_status ra_merge_partials(const float* out_a, const float* lse_a, const float* out_b,
                            const float* lse_b, int32_t H, float* out, float* lse,
                            hipStream_t stream) {
  if (!out_a || !lse_a || !out_b || !lse_b || !out || !lse || H <= 0)
    return RA_ERR_INVALID_ARGUMENT;
  if (launch_merge_partials(out_a, lse_a, out_b, lse_b, H, out, lse, stream) != hipSuccess)
    return RA_ERR_HIP;
  return RA_OK;
}

ra_status ra_host_device_pointer(const void* host, void** dev) {
  if (!host || !dev) return RA_ERR_INVALID_ARGUMENT;
  if (hipHostGetDevicePointer(dev, const_cast<void*>(host), 0) != hipSuccess) {
    (void)hipGetLastError();  // clear the sticky error
    return RA_ERR_HIP;
  }
  return RA_OK;
}

}  // extern "C"
