// Host-side checks of the C ABI's host code (ra_api.cpp), built with g++
// under AddressSanitizer and UndefinedBehaviorSanitizer (tests/
// test_host_sanitizers.py). No GPU: the kernel launchers and the five HIP
// runtime calls ra_api.cpp makes are stubbed here; the stubs record the
// parameters each launcher receives, and the checks below verify them:
//  - workspace layouts: regions 256-byte aligned, disjoint, inside the total;
//  - validation: every entry point's status codes for bad host arguments;
//  - valid calls: the launch sequence and every workspace pointer the
//    kernels would get lies inside the caller's workspace;
//  - the graph build and the layer budgets on many inputs (memory safety
//    under the sanitizers, plus their stated invariants).
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <string>
#include <vector>

#include "ra.h"
#include "ra_internal.h"

#define CHECK(c)                                                          \
  do {                                                                    \
    if (!(c)) {                                                           \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
      std::abort();                                                       \
    }                                                                     \
  } while (0)

// ------------------------------------------------------------------ stubs
static std::vector<std::string> g_calls;
static ra::Params g_p;
static ra::PfParams g_pf;
static bool g_fused = true;  // what the scan_computes_bounds stub answers

namespace ra {
hipError_t launch_sample(const Params& p, hipStream_t) { g_calls.push_back("sample"); g_p = p; return hipSuccess; }
hipError_t launch_threshold(const Params& p, hipStream_t) { g_calls.push_back("threshold"); g_p = p; return hipSuccess; }
bool scan_computes_bounds(const Params&) { return g_fused; }
hipError_t launch_scan(const Params& p, hipStream_t) { g_calls.push_back("scan"); g_p = p; return hipSuccess; }
hipError_t launch_select(const Params& p, hipStream_t) { g_calls.push_back("select"); g_p = p; return hipSuccess; }
hipError_t launch_gather(const Params& p, hipStream_t) { g_calls.push_back("gather"); g_p = p; return hipSuccess; }
hipError_t launch_merge(const Params& p, hipStream_t) { g_calls.push_back("merge"); g_p = p; return hipSuccess; }
hipError_t launch_kv_append(const ra_kv_layer&, const uint16_t*, const uint16_t*, const int32_t*,
                            int32_t, hipStream_t) { g_calls.push_back("append"); return hipSuccess; }
hipError_t launch_prefill(const PfParams& p, int, int, hipStream_t) { g_calls.push_back("prefill"); g_pf = p; return hipSuccess; }
hipError_t launch_graph_search(const GsParams&, hipStream_t) { g_calls.push_back("graph"); return hipSuccess; }
hipError_t launch_sparse_attend(const SaParams&, hipStream_t) { g_calls.push_back("attend"); return hipSuccess; }
hipError_t launch_merge_partials(const float*, const float*, const float*, const float*, int32_t,
                                 float*, float*, hipStream_t) { g_calls.push_back("mergep"); return hipSuccess; }
}  // namespace ra

extern "C" {
hipError_t hipGetDevice(int* d) { *d = 0; return hipSuccess; }
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) { *v = 256; return hipSuccess; }
hipError_t hipGetLastError(void) { return hipSuccess; }
hipError_t hipHostGetDevicePointer(void** dev, void* host, unsigned int) { *dev = host; return hipSuccess; }
hipError_t hipGetSymbolAddress(void** p, const void* sym) { *p = const_cast<void*>(sym); return hipSuccess; }
}

// ------------------------------------------------------------------ helpers
struct Region { size_t off, bytes; };

static void check_regions(std::vector<Region> r, size_t total) {
  std::sort(r.begin(), r.end(), [](const Region& a, const Region& b) { return a.off < b.off; });
  for (size_t i = 0; i < r.size(); ++i) {
    CHECK(r[i].off % 256 == 0);
    CHECK(r[i].off + r[i].bytes <= (i + 1 < r.size() ? r[i + 1].off : total));
  }
}

static std::vector<Region> decode_regions(const ra::WsLayout& L, int64_t B, int64_t H_q, int64_t H_kv) {
  const size_t h = size_t(B * H_q);
  return {{L.off_scores, h * L.n_cap * 4},      {L.off_samp, h * L.samp_cap * 4},
          {L.off_state, h * sizeof(ra::HeadState)}, {L.off_gdone, size_t(B * H_kv) * 4},
          {L.off_misc, 64},                      {L.off_unitoff, size_t(B + 1) * 8},
          {L.off_ucnt, h * L.n_units * 4},       {L.off_scnt, h * L.n_tiles * 4},
          {L.off_cand, h * L.n_cap * 8},         {L.off_part_mz, h * L.n_tiles * 8},
          {L.off_part_n, h * L.n_tiles * 512}};
}

// a host buffer standing in for device memory; only its addresses are used
static std::vector<unsigned char> g_mem(1 << 20);
static void* at(size_t off) { return g_mem.data() + 4096 + off; }

static ra_kv_layer kv_of(int32_t H_kv, int32_t num_pages, int32_t max_pages) {
  ra_kv_layer kv{};
  kv.k_pool = static_cast<uint16_t*>(at(0));
  kv.v_pool = static_cast<uint16_t*>(at(256));
  kv.block_table = static_cast<const int32_t*>(at(512));
  kv.num_pages = num_pages;
  kv.max_pages = max_pages;
  kv.H_kv = H_kv;
  kv.head_dim = 128;
  kv.page_size = 64;
  return kv;
}

static void check_params_in(const ra::Params& p, const char* ws, size_t total) {
  auto inside = [&](const void* q, size_t bytes) {
    const char* c = static_cast<const char*>(q);
    CHECK(c >= ws && c + bytes <= ws + total);
  };
  const size_t h = size_t(p.B) * p.H_q;
  inside(p.scores, h * p.n_cap * 4);
  inside(p.samp, h * p.samp_cap * 4);
  inside(p.state, h * sizeof(ra::HeadState));
  inside(p.gdone, size_t(p.B) * p.H_kv * 4);
  inside(p.any_dense, 4);
  inside(p.unit_off, size_t(p.B + 1) * 8);
  inside(p.ucnt, h * p.n_units * 4);
  inside(p.scnt, h * p.n_tiles * 4);
  inside(p.cand, h * p.n_cap * 8);
  inside(p.part_mz, h * p.n_tiles * 8);
  inside(p.part_n, h * p.n_tiles * 512);
  CHECK(p.n_cap >= p.max_seq_len && p.n_cap % ra::kTile == 0);
  CHECK(int64_t(p.n_units) * ra::kUnit == p.n_cap && int64_t(p.n_tiles) * ra::kUnit == p.n_cap);
}

// ------------------------------------------------------------------ checks
static void layouts() {
  const int32_t Bs[] = {1, 2, 3, 16, 100, 2047};
  const int32_t HH[][2] = {{4, 1}, {32, 8}, {8, 8}, {16, 2}, {64, 8}};
  const int32_t Ns[] = {1, 63, 64, 65, 4095, 4096, 8193, 131072, 1 << 20, (1 << 20) + 1000, 1 << 24};
  const int32_t Ks[] = {0, 1, 64, 2048, 31457};
  int n = 0;
  for (int32_t B : Bs)
    for (auto& hh : HH)
      for (int32_t N : Ns)
        for (int32_t k : Ks) {
          ra::WsLayout L;
          const bool ok = ra::ws_layout(B, hh[0], hh[1], N, k, &L);
          CHECK(ok == (int64_t(B) * hh[0] <= 65535));
          if (!ok) continue;
          check_regions(decode_regions(L, B, hh[0], hh[1]), L.total);
          CHECK(L.n_cap >= N && L.samp_cap % 64 == 0);
          CHECK(ra_decode_workspace_bytes(B, hh[0], hh[1], N, k) == L.total);
          ++n;
        }
  CHECK(n > 500);
  ra::WsLayout L;
  CHECK(!ra::ws_layout(0, 4, 1, 10, 1, &L) && !ra::ws_layout(1, 4, 3, 10, 1, &L));
  CHECK(!ra::ws_layout(1, 4, 1, 0, 1, &L) && !ra::ws_layout(1, 4, 1, (1 << 24) + 1, 1, &L));
  CHECK(!ra::ws_layout(1, 4, 1, 10, -1, &L));
  // prefill layouts
  for (int32_t T : {1, 7, 512, 4096})
    for (int32_t N : {1, 64, 5000, 131072, 1 << 20})
      for (int32_t k : {0, 1, 100, 256}) {
        ra::PfLayout P;
        CHECK(ra::pf_layout(T, 32, N, k, &P));
        const size_t rows = size_t(T) * 32, pages = (size_t(N) + 63) / 64;
        const size_t ppad = (pages + ra::kPfChunk - 1) / ra::kPfChunk * ra::kPfChunk;
        const size_t ps = (size_t(ra::pf_sampled_pages(int(pages))) + ra::kPfChunk - 1) /
                          ra::kPfChunk * ra::kPfChunk;
        check_regions({{P.off_pmax, rows * ppad * 4}, {P.off_tau, rows * 8},
                       {P.off_seg_off, rows * ra::kPfMaxSplits * 4},
                       {P.off_seg_cnt, rows * ra::kPfMaxSplits * 4},
                       {P.off_cand, rows * P.cap * 8}, {P.off_smax, rows * ps * 4},
                       {P.off_fail, rows * 4}},
                      P.total);
        CHECK(ra_prefill_workspace_bytes(T, 32, N, k) == P.total);
      }
  ra::PfLayout P;
  CHECK(!ra::pf_layout(1, 32, 100, 257, &P) && !ra::pf_layout(0, 32, 100, 1, &P));
}

static void decode_calls() {
  // a valid call: the six kernels in order, every workspace pointer inside
  const int32_t B = 3, H_q = 8, H_kv = 2, N = 70000, K = 500;
  ra_kv_layer kv = kv_of(H_kv, 4000, 2000);
  const size_t need = ra_decode_workspace_bytes(B, H_q, H_kv, N, K);
  std::vector<unsigned char> wsbuf(need + 512);
  char* ws = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(wsbuf.data()) + 255) & ~uintptr_t(255));
  const uint16_t* q = static_cast<const uint16_t*>(at(1024));
  const int32_t* i32 = static_cast<const int32_t*>(at(2048));
  float* f32 = static_cast<float*>(at(4096));
  int32_t* oi = static_cast<int32_t*>(at(8192));
  // the threshold launch is left out when the scan computes the bounds
  g_fused = false;
  g_calls.clear();
  CHECK(ra_decode_step(q, H_q, &kv, i32, B, N, i32, K, 128, 512, f32, oi, ws, need, nullptr) == RA_OK);
  CHECK((g_calls == std::vector<std::string>{"sample", "threshold", "scan", "select", "gather", "merge"}));
  CHECK(g_p.scan_bounds == 0);  // the scan finds the bounds published
  g_calls.clear();
  CHECK(ra_append_decode_step(q, q, i32, q, H_q, &kv, i32, B, N, i32, K, 128, 512, f32, nullptr,
                              oi, ws, need, 0, nullptr) == RA_OK);
  CHECK((g_calls == std::vector<std::string>{"sample", "threshold", "scan", "select", "gather", "merge"}));
  g_fused = true;
  g_calls.clear();
  CHECK(ra_decode_step(q, H_q, &kv, i32, B, N, i32, K, 128, 512, f32, oi, ws, need, nullptr) == RA_OK);
  CHECK((g_calls == std::vector<std::string>{"sample", "scan", "select", "gather", "merge"}));
  CHECK(g_p.scan_bounds == 1);
  // a scan in a call of its own computes whatever bounds are missing
  g_calls.clear();
  CHECK(ra_decode_stages(q, H_q, &kv, i32, B, N, i32, K, 128, 512, f32, nullptr, oi, ws, need, 0,
                         RA_STAGE_SCAN, RA_STAGE_MERGE, nullptr) == RA_OK);
  CHECK(g_calls.size() == 4 && g_p.scan_bounds == 1);
  check_params_in(g_p, ws, need);
  CHECK(g_p.lse == nullptr && g_p.keep_scores == 0 && g_p.app_pos == nullptr);
  CHECK(g_p.num_cus == 256 && g_p.G == 4);
  g_calls.clear();
  CHECK(ra_decode_step_ex(q, H_q, &kv, i32, B, N, i32, K, 0, 0, f32, f32, oi, ws, need,
                          RA_DECODE_KEEP_SCORES, nullptr) == RA_OK);
  CHECK(g_calls.size() == 5 && g_p.keep_scores == 1 && g_p.lse == f32);
  g_calls.clear();
  CHECK(ra_append_decode_step(q, q, i32, q, H_q, &kv, i32, B, N, i32, K, 128, 512, f32, nullptr,
                              oi, ws, need, 0, nullptr) == RA_OK);
  CHECK((g_calls == std::vector<std::string>{"sample", "scan", "select", "gather", "merge"}));
  CHECK(g_p.app_pos == i32);
  for (int fused = 0; fused < 2; ++fused)
    for (int a = 0; a < 6; ++a)
      for (int b = a; b < 6; ++b) {
        g_fused = fused != 0;
        g_calls.clear();
        CHECK(ra_decode_stages(q, H_q, &kv, i32, B, N, i32, K, 128, 512, f32, nullptr, oi, ws, need,
                               0, a, b, nullptr) == RA_OK);
        // the threshold stage launches nothing when the scan follows in the call
        const bool skipped = fused && a <= RA_STAGE_THRESHOLD && b >= RA_STAGE_SCAN;
        CHECK(int(g_calls.size()) == b - a + 1 - (skipped ? 1 : 0));
      }
  g_fused = true;
  // invalid host arguments: nothing is launched
  g_calls.clear();
  CHECK(ra_decode_step(nullptr, H_q, &kv, i32, B, N, i32, K, 1, 1, f32, oi, ws, need, nullptr) == RA_ERR_INVALID_ARGUMENT);
  CHECK(ra_decode_step(q, H_q, nullptr, i32, B, N, i32, K, 1, 1, f32, oi, ws, need, nullptr) == RA_ERR_INVALID_ARGUMENT);
  CHECK(ra_decode_step(q, H_q, &kv, i32, B, N, i32, K, 1, 1, f32, oi, ws, need - 1, nullptr) == RA_ERR_WORKSPACE);
  CHECK(ra_decode_step(q, H_q, &kv, i32, B, N, i32, K, 1, 1, f32, oi, ws + 16, need, nullptr) == RA_ERR_INVALID_ARGUMENT);
  CHECK(ra_decode_step(q, 12, &kv, i32, B, N, i32, K, 1, 1, f32, oi, ws, need, nullptr) == RA_ERR_UNSUPPORTED);  // G = 6
  CHECK(ra_decode_step(q, 7, &kv, i32, B, N, i32, K, 1, 1, f32, oi, ws, need, nullptr) == RA_ERR_INVALID_ARGUMENT);
  CHECK(ra_decode_step(q, H_q, &kv, i32, 0, N, i32, K, 1, 1, f32, oi, ws, need, nullptr) == RA_ERR_INVALID_ARGUMENT);
  CHECK(ra_decode_step(q, H_q, &kv, i32, B, N, i32, K, -1, 1, f32, oi, ws, need, nullptr) == RA_ERR_INVALID_ARGUMENT);
  CHECK(ra_decode_step(q, H_q, &kv, i32, B, N, i32, K, 1, 1, f32, nullptr, ws, need, nullptr) == RA_ERR_INVALID_ARGUMENT);
  CHECK(ra_decode_step_ex(q, H_q, &kv, i32, B, N, i32, K, 1, 1, f32, nullptr, oi, ws, need, 2u, nullptr) == RA_ERR_INVALID_ARGUMENT);
  CHECK(ra_decode_stages(q, H_q, &kv, i32, B, N, i32, K, 1, 1, f32, nullptr, oi, ws, need, 0, 3, 2, nullptr) == RA_ERR_INVALID_ARGUMENT);
  ra_kv_layer bad = kv;
  bad.head_dim = 64;
  CHECK(ra_decode_step(q, H_q, &bad, i32, B, N, i32, K, 1, 1, f32, oi, ws, need, nullptr) == RA_ERR_UNSUPPORTED);
  bad = kv;
  bad.k_pool = reinterpret_cast<uint16_t*>(at(8));
  CHECK(ra_decode_step(q, H_q, &bad, i32, B, N, i32, K, 1, 1, f32, oi, ws, need, nullptr) == RA_ERR_INVALID_ARGUMENT);
  CHECK(g_calls.empty());
  // the call without a workspace: its array, or RA_ERR_WORKSPACE past it
  g_calls.clear();
  CHECK(ra_decode_step_noalloc(q, H_q, &kv, i32, 1, 4096, i32, 64, 16, 64, f32, nullptr, oi, 0, nullptr) == RA_OK);
  CHECK(g_calls.size() == 5);
  check_params_in(g_p, reinterpret_cast<const char*>(g_p.scores), RA_NOALLOC_WS_BYTES);
  const size_t big = ra_decode_workspace_bytes(1, 32, 8, 1 << 20, 10485);
  CHECK(big > RA_NOALLOC_WS_BYTES);
  ra_kv_layer kv8 = kv_of(8, 20000, 20000);
  g_calls.clear();
  CHECK(ra_decode_step_noalloc(q, 32, &kv8, i32, 1, 1 << 20, i32, 10485, 128, 512, f32, nullptr, oi, 0, nullptr) == RA_ERR_WORKSPACE);
  CHECK(g_calls.empty());
  // the append alone
  g_calls.clear();
  CHECK(ra_kv_append(&kv, q, q, i32, 4, nullptr) == RA_OK && g_calls.size() == 1);
  CHECK(ra_kv_append(&kv, q, q, i32, 0, nullptr) == RA_ERR_INVALID_ARGUMENT);
  CHECK(ra_kv_append(&kv, q + 4, q, i32, 1, nullptr) == RA_ERR_INVALID_ARGUMENT);
}

static void prefill_graph_attend_calls() {
  ra_kv_layer kv = kv_of(8, 3000, 3000);
  const uint16_t* q = static_cast<const uint16_t*>(at(1024));
  int32_t* oi = static_cast<int32_t*>(at(8192));
  const size_t need = ra_prefill_workspace_bytes(64, 32, 100000, 100);
  std::vector<unsigned char> wsbuf(need + 512);
  char* ws = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(wsbuf.data()) + 255) & ~uintptr_t(255));
  g_calls.clear();
  CHECK(ra_prefill_topk(q, 64, 32, &kv, 0, 100000, 100, 128, 512, oi, ws, need, nullptr) == RA_OK);
  CHECK(g_calls.size() == 1 && g_pf.k_eff == 100 && g_pf.lo == 128 && g_pf.hi == 100000 - 512);
  CHECK(g_pf.splits >= 1 && g_pf.splits <= ra::kPfMaxSplits && g_pf.seg_cap * g_pf.splits <= g_pf.cap);
  CHECK(reinterpret_cast<char*>(g_pf.fail) + 64 * 32 * 4 <= ws + need);
  CHECK(ra_prefill_topk(q, 64, 32, &kv, 0, 100000, 257, 128, 512, oi, ws, need, nullptr) == RA_ERR_INVALID_ARGUMENT);
  CHECK(ra_prefill_topk(q, 64, 32, &kv, 0, 3000 * 64 + 1, 100, 128, 512, oi, ws, need, nullptr) == RA_ERR_INVALID_ARGUMENT);
  CHECK(ra_prefill_topk(q, 64, 32, &kv, 0, 100000, 100, 128, 512, oi, ws, need - 1, nullptr) == RA_ERR_WORKSPACE);
  const int32_t* nb = static_cast<const int32_t*>(at(2048));
  g_calls.clear();
  CHECK(ra_graph_search(q, 32, &kv, 0, 5000, nb, 16, nb, 64, 32, oi, oi, nullptr) == RA_OK);
  CHECK(ra_graph_search(q, 32, &kv, 0, 5000, nb, 65, nb, 64, 32, oi, oi, nullptr) == RA_ERR_INVALID_ARGUMENT);
  CHECK(ra_graph_search(q, 32, &kv, 0, 5000, nb, 16, nb, 16, 32, oi, oi, nullptr) == RA_ERR_INVALID_ARGUMENT);
  CHECK(ra_graph_search(q, 32, &kv, 0, (1 << 20) + 1, nb, 16, nb, 64, 32, oi, oi, nullptr) == RA_ERR_INVALID_ARGUMENT);
  float* f = static_cast<float*>(at(4096));
  CHECK(ra_sparse_attend(q, 32, &kv, 0, 5000, nb, 100, f, f, nullptr) == RA_OK);
  CHECK(ra_sparse_attend(q, 32, &kv, 0, 5000, nb, RA_SPARSE_MAX_K + 1, f, f, nullptr) == RA_ERR_INVALID_ARGUMENT);
  CHECK(ra_merge_partials(f, f, f, f, 32, f, f, nullptr) == RA_OK);
  CHECK(ra_merge_partials(f, f, f, f, 0, f, f, nullptr) == RA_ERR_INVALID_ARGUMENT);
  CHECK(g_calls.size() == 3);
  void* dev = nullptr;
  CHECK(ra_host_device_pointer(at(0), &dev) == RA_OK && dev == at(0));
  CHECK(ra_host_device_pointer(nullptr, &dev) == RA_ERR_INVALID_ARGUMENT);
}

static void graph_build_and_budgets() {
  std::mt19937 rng(7);
  for (int rep = 0; rep < 200; ++rep) {
    const int32_t N = 1 + int32_t(rng() % 600), T = int32_t(rng() % 300);
    const int32_t K = 1 + int32_t(rng() % 20), D = 1 + int32_t(rng() % 64);
    std::vector<int32_t> hubs(size_t(T) + 1), lists(size_t(T) * K + 1), nbr(size_t(N) * D);
    for (int32_t t = 0; t < T; ++t) {
      hubs[t] = int32_t(rng() % (N + 1)) - 1;
      for (int32_t j = 0; j < K; ++j) lists[size_t(t) * K + j] = int32_t(rng() % (N + 1)) - 1;
    }
    int32_t entry = -5;
    CHECK(ra_graph_build(hubs.data(), lists.data(), T, K, N, D, nbr.data(), &entry) == RA_OK);
    CHECK(entry >= -1 && entry < N);
    for (int32_t a = 0; a < N; ++a) {
      const int32_t* row = nbr.data() + size_t(a) * D;
      bool pad = false;
      for (int32_t j = 0; j < D; ++j) {
        CHECK(row[j] >= -1 && row[j] < N && row[j] != a);
        if (row[j] < 0) pad = true;
        else CHECK(!pad);  // -1 only after the neighbours
        for (int32_t i = 0; i < j; ++i) CHECK(row[j] < 0 || row[i] != row[j]);
      }
    }
    if (T > 0) {
      hubs[0] = N;  // out of range
      CHECK(ra_graph_build(hubs.data(), lists.data(), T, K, N, D, nbr.data(), &entry) == RA_ERR_INVALID_ARGUMENT);
    }
  }
  {
    std::vector<int32_t> nbr(40);
    int32_t entry = 0;
    CHECK(ra_graph_build(nullptr, nullptr, 0, 1, 10, 4, nbr.data(), &entry) == RA_OK && entry == -1);
  }
  for (int32_t L = 1; L <= 64; ++L)
    for (int32_t k : {0, 1, 7, 100, 10485})
      for (int32_t s : {0, 1, 333, 500, 999, 1000}) {
        std::vector<int32_t> out(static_cast<size_t>(L));
        CHECK(ra_layer_budgets(L, k, s, out.data()) == RA_OK);
        int64_t sum = 0;
        for (int32_t v : out) {
          CHECK(v >= 0);
          sum += v;
        }
        CHECK(sum == int64_t(L) * k);
      }
  std::vector<int32_t> out(5000);
  CHECK(ra_layer_budgets(4097, 1, 0, out.data()) == RA_ERR_INVALID_ARGUMENT);
  CHECK(ra_layer_budgets(4, 1, 1001, out.data()) == RA_ERR_INVALID_ARGUMENT);
  CHECK(ra_layer_budgets(4, 1, 0, nullptr) == RA_ERR_INVALID_ARGUMENT);
}

int main() {
  CHECK(ra_abi_version() == RA_ABI_VERSION);
  CHECK(std::string(ra_status_str(RA_ERR_HIP)) == "RA_ERR_HIP");
  layouts();
  decode_calls();
  prefill_graph_attend_calls();
  graph_build_and_budgets();
  std::puts("host checks ok");
  return 0;
}
