/*
 * ra.h - C ABI of the exact top-k sparse GQA decode step (MI355X / gfx950).
 *
 * One call computes, for every sequence b and query head h, the decode step
 * of RetrievalAttention with an exact retrieval:
 *
 *   z[n]   = q_h . k_n / sqrt(128) for every cached position n
 *            (RetrievalAttention slides, "Sparse attention renormalizes
 *            selected tokens", Eq. (1));
 *   W      = the first n_sink and the last `window` positions (frame "The GPU
 *            keeps 640 fixed positions": first 128 + last 512 tokens);
 *   Omega  = the k_eff = min(k[b], |M|) positions of M = [0, N) \ W with the
 *            largest z, ties to the lower position (the fixed retrieval
 *            budget of the Eq. (2) frame; W and Omega disjoint);
 *   out    = softmax(z) . V over W u Omega, renormalised on that set (Eq. (2)),
 *            computed as partials merged by log-sum-exp (frame "Two local
 *            softmax outputs need global weights", Eqs. (3)-(5)).
 *
 * GQA: query head h reads KV head h / G, G = H_q / H_kv (contiguous groups);
 * each query head gets its own retrieved indices over the shared KV storage
 * (frame "The GPU keeps 640 fixed positions").
 *
 * Conventions for every entry point:
 *  - Pointers marked "device" are HIP device memory owned by the caller; the
 *    library never allocates, frees, synchronises or reads device memory on
 *    the host. Work is enqueued on `stream` in order; buffers must stay live
 *    until the stream has executed it.
 *  - bf16 tensors are passed as uint16_t bit patterns.
 *  - Host arguments are validated before anything is enqueued; on an error
 *    nothing is enqueued and the status says why. Device contents (lengths,
 *    budgets, block-table entries) are trusted, but clamped so that no access
 *    leaves its buffer: a length is clamped to [0, min(max_seq_len,
 *    64 * max_pages)], a budget to [0, k_max], and a page id outside
 *    [0, num_pages) reads page 0.
 *  - The library is stateless and reentrant; no C++ exception crosses it.
 */
#ifndef RA_H
#define RA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RA_ABI_VERSION 5
#define RA_HEAD_DIM 128
#define RA_PAGE_SIZE 64
#define RA_MAX_SEQ_LEN (1 << 24) /* 16,777,216 positions per sequence */
#define RA_MAX_BATCH 65535

typedef enum ra_status {
  RA_OK = 0,
  RA_ERR_INVALID_ARGUMENT = 1, /* null pointer, non-positive size, H_q % H_kv != 0, ... */
  RA_ERR_WORKSPACE = 2,        /* ws_bytes below ra_decode_workspace_bytes(...) */
  RA_ERR_UNSUPPORTED = 3,      /* head_dim != 128, page_size != 64, G not in {1,2,4,8} */
  RA_ERR_HIP = 4               /* a kernel launch reported an error */
} ra_status;

/*
 * One layer's paged KV cache.
 *  k_pool, v_pool: device bf16 [num_pages][H_kv][64][128], 16-byte aligned;
 *                  the 64 x 128 block of one (page, KV head) is contiguous
 *                  (16 KiB).
 *  block_table:    device int32 [B][max_pages]; entry [b][j] is the physical
 *                  page holding positions 64 j .. 64 j + 63 of sequence b.
 * Page allocation is the caller's job. Misaligned pointers are rejected with
 * RA_ERR_INVALID_ARGUMENT (int32 and fp32 arrays need 4-byte alignment).
 */
typedef struct ra_kv_layer {
  uint16_t* k_pool;
  uint16_t* v_pool;
  const int32_t* block_table;
  int32_t num_pages;
  int32_t max_pages;
  int32_t H_kv;
  int32_t head_dim;  /* must be 128 */
  int32_t page_size; /* must be 64 */
} ra_kv_layer;

/* RA_ABI_VERSION of the built library. */
int ra_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char* ra_status_str(ra_status s);

/*
 * Bytes of scratch workspace ra_decode_step needs for these capacities
 * (score rows, sample histograms, per-tile candidate lists and split-K
 * partials). Returns 0 if the arguments are invalid.
 */
size_t ra_decode_workspace_bytes(int32_t B, int32_t H_q, int32_t H_kv,
                                 int32_t max_seq_len, int32_t k_max);

/*
 * Append one token's key and value per (sequence, KV head): write k_new[b][g]
 * and v_new[b][g] to slot pos[b] % 64 of page block_table[b][pos[b] / 64].
 * This is the "decode one new token at a time" step of the slides' setting
 * frame ("One question: how can decoding read less KV?").
 *  k_new, v_new: device bf16 [B][H_kv][128], 16-byte aligned.
 *  pos:          device int32 [B], the new token's position (its sequence's
 *                length before the append). Positions outside
 *                [0, 64 * max_pages) are skipped.
 */
ra_status ra_kv_append(const ra_kv_layer* kv, const uint16_t* k_new,
                       const uint16_t* v_new, const int32_t* pos, int32_t B,
                       hipStream_t stream);

/* Flags of ra_decode_step_ex, ra_append_decode_step and ra_decode_stages
   (other bits are rejected). */
#define RA_DECODE_KEEP_SCORES 1u /* also leave the scores of the retrieved set
                                    in the workspace score rows (a check of
                                    the scores; it costs scattered writes) */

/*
 * One decode step (see the top of this file for what it computes), in the
 * shape of the problem the slides pose: decode one new token at a time over
 * a prefilled cache (frame "One question: how can decoding read less KV?"),
 * with a fixed retrieval budget per query head and the static first/last
 * positions (frames "Sparse attention renormalizes selected tokens" and "The
 * GPU keeps 640 fixed positions").
 *  q:           device bf16 [B][H_q][128], the new token's queries,
 *               16-byte aligned.
 *  seq_lens:    device int32 [B], lengths N_b after the append, so the recent
 *               window includes the new token.
 *  max_seq_len: host capacity >= every N_b; sizes the grids and workspace.
 *  k:           device int32 [B], per-sequence budget k_b (0 <= k_b <= k_max).
 *  n_sink, window: sizes of the static set (>= 0).
 *  out:         device fp32 [B][H_q][128].
 *  out_idx:     device int32 [B][H_q][k_max]: Omega in ascending position
 *               order, then -1 up to k_max (may be NULL only if k_max == 0).
 *  ws, ws_bytes: device workspace of at least ra_decode_workspace_bytes(B,
 *               H_q, kv->H_kv, max_seq_len, k_max) bytes, 256-byte aligned;
 *               no initial contents are required. Calls that share a
 *               workspace must be ordered on one stream.
 * An empty W u Omega gives out = 0. Launch count and grid sizes depend only on
 * the host arguments, so the call can be captured into a HIP graph.
 * Equivalent to ra_decode_step_ex with out_lse = NULL and flags = 0.
 */
ra_status ra_decode_step(const uint16_t* q, int32_t H_q, const ra_kv_layer* kv,
                         const int32_t* seq_lens, int32_t B,
                         int32_t max_seq_len, const int32_t* k, int32_t k_max,
                         int32_t n_sink, int32_t window, float* out,
                         int32_t* out_idx, void* ws, size_t ws_bytes,
                         hipStream_t stream);

/*
 * ra_decode_step with two additions:
 *  out_lse:     device fp32 [B][H_q] (may be NULL): log-sum-exp of z over
 *               W u Omega, -inf when that set is empty, so that the output
 *               can be merged further by the same identity (frame "Two local
 *               softmax outputs need global weights", Eqs. (3)-(5)).
 *  flags:       0 or RA_DECODE_KEEP_SCORES.
 * Every other argument as for ra_decode_step.
 */
ra_status ra_decode_step_ex(const uint16_t* q, int32_t H_q, const ra_kv_layer* kv,
                            const int32_t* seq_lens, int32_t B,
                            int32_t max_seq_len, const int32_t* k, int32_t k_max,
                            int32_t n_sink, int32_t window, float* out,
                            float* out_lse, int32_t* out_idx, void* ws,
                            size_t ws_bytes, uint32_t flags, hipStream_t stream);

/*
 * For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): ra_decode_step_ex
 * without a workspace argument. Its workspace is a device array inside the
 * library of RA_NOALLOC_WS_BYTES bytes, one per GPU it runs on, held until
 * the process ends; this call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine). Its first call on a device looks up that
 * device's copy of the array (hipGetSymbolAddress, with the device current).
 *  Returns RA_ERR_WORKSPACE when ra_decode_workspace_bytes(B, H_q,
 *  kv->H_kv, max_seq_len, k_max) exceeds RA_NOALLOC_WS_BYTES (64 MiB: one
 *  Llama-3-8B layer, 32 query heads, up to 131072 tokens), RA_ERR_HIP if the
 *  array's address cannot be found. Every other argument, the validation and
 *  the results as for ra_decode_step_ex.
 *  All calls on one GPU share its array and no initial contents are needed,
 *  but calls that overlap in time on one GPU (other streams, other host
 *  threads) race on it: order them on one stream.
 */
#define RA_NOALLOC_WS_BYTES (64u << 20)
ra_status ra_decode_step_noalloc(const uint16_t* q, int32_t H_q, const ra_kv_layer* kv,
                                 const int32_t* seq_lens, int32_t B, int32_t max_seq_len,
                                 const int32_t* k, int32_t k_max, int32_t n_sink,
                                 int32_t window, float* out, float* out_lse, int32_t* out_idx,
                                 uint32_t flags, hipStream_t stream);

/*
 * ra_kv_append followed by ra_decode_step_ex, in one call and one launch
 * fewer: the new token's rows (k_new, v_new: device bf16 [B][H_kv][128],
 * 16-byte aligned; pos: device int32 [B], as for ra_kv_append) are written
 * by the step's second kernel, after the sampled bound's kernel (which may
 * then read the slot's previous contents: that only bounds the candidates)
 * and before every kernel whose reads decide the result. seq_lens must
 * count the new token, as after ra_kv_append. Results equal those of the
 * two separate calls. Validation and errors as for both.
 */
ra_status ra_append_decode_step(const uint16_t* k_new, const uint16_t* v_new,
                                const int32_t* pos, const uint16_t* q, int32_t H_q,
                                const ra_kv_layer* kv, const int32_t* seq_lens, int32_t B,
                                int32_t max_seq_len, const int32_t* k, int32_t k_max,
                                int32_t n_sink, int32_t window, float* out, float* out_lse,
                                int32_t* out_idx, void* ws, size_t ws_bytes, uint32_t flags,
                                hipStream_t stream);

/*
 * The kernels of one decode step, in launch order. ra_decode_step runs
 * stages RA_STAGE_SAMPLE .. RA_STAGE_MERGE; ra_decode_stages runs a contiguous
 * sub-range of them with the same arguments, so each kernel can be timed or
 * inspected on its own. State passes between stages through `ws`, so a range
 * must start where the previous range on the same workspace ended, and the
 * inputs (q, the pools, lengths and budgets) must not change between the
 * calls of one step: the scan takes the sampled pages' scores from the
 * sample stage.
 * When a range holds both RA_STAGE_THRESHOLD and RA_STAGE_SCAN and the batch
 * has at most one query head per scan block (one block per compute unit, at
 * most one per 4096 positions of capacity per KV head), the scan computes
 * the thresholds itself and RA_STAGE_THRESHOLD launches nothing; a scan run
 * without the threshold stage before it computes any that are missing. The
 * results are the same bit for bit either way.
 */
typedef enum ra_stage {
  RA_STAGE_SAMPLE = 0, /* score one page in S (S <= 64) of every sequence;
                          reset of the per-call state */
  RA_STAGE_THRESHOLD = 1, /* per head: candidate threshold from the sample */
  RA_STAGE_SCAN = 2,   /* all scores; keep W and the candidates above it */
  RA_STAGE_SELECT = 3, /* exact top-k threshold over the candidates, ties to
                          the lower position; heads with fewer candidates
                          than k are rescanned with every member of M as a
                          candidate and selected again (no work otherwise) */
  RA_STAGE_GATHER = 4, /* take the retrieved members per tile, split-K
                          softmax-V partials */
  RA_STAGE_MERGE = 5,  /* log-sum-exp merge into out / out_lse; out_idx with
                          -1 padding */
  RA_STAGE_COUNT = 6
} ra_stage;

ra_status ra_decode_stages(const uint16_t* q, int32_t H_q,
                           const ra_kv_layer* kv, const int32_t* seq_lens,
                           int32_t B, int32_t max_seq_len, const int32_t* k,
                           int32_t k_max, int32_t n_sink, int32_t window,
                           float* out, float* out_lse, int32_t* out_idx,
                           void* ws, size_t ws_bytes, uint32_t flags,
                           int32_t first_stage, int32_t last_stage,
                           hipStream_t stream);

/*
 * Where the fp32 score rows live inside a workspace sized for these
 * capacities: z for (b, h, n) is the float at byte offset
 * returned + 4 * ((b * H_q + h) * (*row_stride) + n). After RA_STAGE_GATHER
 * it holds the scores of the positions of W, and of the retrieved set if the
 * call passed RA_DECODE_KEEP_SCORES; other entries are unspecified. Returns
 * (size_t)-1 if the arguments are invalid.
 */
size_t ra_workspace_scores_offset(int32_t B, int32_t H_q, int32_t H_kv,
                                  int32_t max_seq_len, int32_t k_max,
                                  int64_t* row_stride);

/*
 * Where a uint32 counter lives inside a workspace sized for these
 * capacities (byte offset, 4-byte aligned): after RA_STAGE_SELECT of a call
 * it holds the number of query heads whose candidates fell short of k_eff,
 * which that stage then decided by the full rescan (0 in the common case). A diagnostic; the caller reads it from device memory itself.
 * In a library built with -DRA_DEBUG (libra_debug.so), the next uint32
 * holds the bounds checks of the decode kernels that failed in the call,
 * one bit per check site (their accesses were skipped); 0 when all held.
 * Returns (size_t)-1 if the arguments are invalid.
 */
size_t ra_workspace_rescan_count_offset(int32_t B, int32_t H_q, int32_t H_kv,
                                        int32_t max_seq_len, int32_t k_max);

/* ------------------------------------------------------------------ */
/* Prefill: exact top-k keys of a block of prefill queries.             */
/* ------------------------------------------------------------------ */

#define RA_PREFILL_MAX_K 256

/*
 * Bytes of workspace ra_prefill_topk needs for T query rows of H_q heads
 * against N keys with budget k. Returns 0 if the arguments are invalid.
 */
size_t ra_prefill_workspace_bytes(int32_t T, int32_t H_q, int32_t N, int32_t k);

/*
 * For every prefill query row t and query head h: the exact top-k keys of
 * one sequence by z = q . k / sqrt(128), over M = [n_sink, N - window) as in
 * the decode step, ties to the lower position. Keys are ranked by q . k in
 * fp32 (bf16 products, fp32 MFMA accumulation): the positive factor does
 * not change the order. This is the first step of the
 * slides' index frame ("Prefill queries teach the key graph what matters":
 * prefill queries find their exact top-k keys on the GPU, and each query is
 * linked to those keys). No causal cut is applied: every row is linked to
 * the best keys of the whole domain.
 *  q:       device bf16 [T][H_q][128], 16-byte aligned.
 *  kv:      the paged layer; seq selects the block-table row of the
 *           sequence (trusted, like device contents), N its key count
 *           (1 <= N <= 64 * max_pages).
 *  k:       host budget, 0 <= k <= RA_PREFILL_MAX_K; k_eff = min(k, |M|).
 *  out_idx: device int32 [T][H_q][k]: each row's k_eff positions ascending,
 *           then -1.
 *  ws, ws_bytes: device workspace of at least ra_prefill_workspace_bytes
 *           bytes, 256-byte aligned, no initial contents required.
 * The scores run on MFMA: page maxima over one page in 8, a per-row bound
 * from them, then a filter over every key at that bound. A row whose filter
 * kept at least k_eff keys, all of them stored, has its exact top-k among
 * them (every key below the bound ranks below every key kept); any other
 * row is flagged and recomputed, with the row blocks holding it, by the
 * exact pass (page maxima of every page, whose k_eff-th largest provably
 * keeps the whole top-k). The score matrix is never stored.
 * Validation and ownership as for ra_decode_step.
 */
ra_status ra_prefill_topk(const uint16_t* q, int32_t T, int32_t H_q,
                          const ra_kv_layer* kv, int32_t seq, int32_t N,
                          int32_t k, int32_t n_sink, int32_t window,
                          int32_t* out_idx, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/*
 * The kernels of ra_prefill_topk, in launch order; ra_prefill_stages runs a
 * contiguous sub-range with the same arguments (as ra_decode_stages does).
 * A stage reads what the stages before it left in the workspace, so the
 * ranges must be run in order on the same workspace. first_stage >
 * last_stage, or either outside [0, RA_PF_STAGE_COUNT), returns
 * RA_ERR_INVALID_ARGUMENT.
 */
typedef enum ra_prefill_stage {
  RA_PF_STAGE_SAMPLE = 0,        /* contraction over one page in 8: sampled page maxima */
  RA_PF_STAGE_BOUND = 1,         /* per row: the sampled bound (R-th largest sampled pair) */
  RA_PF_STAGE_FILTER = 2,        /* contraction: keys at or above the bound */
  RA_PF_STAGE_SELECT = 3,        /* per row: exact top-k, or the row is flagged */
  RA_PF_STAGE_EXACT_MAXIMA = 4,  /* flagged row blocks: page maxima of every page */
  RA_PF_STAGE_EXACT_THRESHOLD = 5, /* the k-th largest (page max, page) */
  RA_PF_STAGE_EXACT_FILTER = 6,  /* keys at or above it */
  RA_PF_STAGE_EXACT_SELECT = 7,  /* exact top-k of the flagged rows */
  RA_PF_STAGE_COUNT = 8
} ra_prefill_stage;

/*
 * Byte offset in the workspace of the per-row flags the last call left:
 * uint32 [T * H_q], 1 for a row whose sampled bound fell short (it was then
 * computed by the exact stages). For tests and diagnostics. Returns 0 if
 * the arguments are invalid (the flags never start at offset 0).
 */
size_t ra_prefill_workspace_fail_offset(int32_t T, int32_t H_q, int32_t N, int32_t k);

ra_status ra_prefill_stages(const uint16_t* q, int32_t T, int32_t H_q,
                            const ra_kv_layer* kv, int32_t seq, int32_t N,
                            int32_t k, int32_t n_sink, int32_t window,
                            int32_t* out_idx, void* ws, size_t ws_bytes,
                            int32_t first_stage, int32_t last_stage,
                            hipStream_t stream);

/* ------------------------------------------------------------------ */
/* Per-layer retrieval budgets.                                         */
/* ------------------------------------------------------------------ */

/*
 * A pyramid-shaped schedule of per-layer budgets with the total of a uniform
 * budget k_mean per layer (slides, frame "Extra experiments show where
 * budget matters": a PyramidKV-style layer budget, more keys for the lower
 * layers): k_l = k_mean (1 + s (L - 1 - 2 l) / (L - 1)) for layers
 * l = 0 .. L - 1 with slope s = slope_permille / 1000 in [0, 1], rounded to
 * integers that sum to L k_mean exactly (each layer gets the floor; the
 * L k_mean - sum of floors layers with the largest fractional parts get one
 * more, ties to the lower layer). s = 0 is the uniform budget. Host
 * arithmetic only: each layer's decode step then takes its k_l (the
 * kernels are unchanged).
 *  n_layers: 1 .. 4096; k_mean >= 0; slope_permille in [0, 1000].
 *  k_out:    host int32 [n_layers].
 * Returns RA_ERR_INVALID_ARGUMENT for arguments outside these ranges or a
 * null k_out.
 */
ra_status ra_layer_budgets(int32_t n_layers, int32_t k_mean, int32_t slope_permille,
                           int32_t* k_out);

/* ------------------------------------------------------------------ */
/* Query-aware key graph (slides, frame "Prefill queries teach the key  */
/* graph what matters": prefill queries' exact top-k keys, links to      */
/* those keys, projected into a key-only graph, searched per decode      */
/* query).                                                               */
/* ------------------------------------------------------------------ */

#define RA_GRAPH_MAX_DEGREE 64
#define RA_GRAPH_MAX_EF 256
#define RA_GRAPH_MAX_N (1 << 20) /* keys a graph spans (the visited set is in LDS) */
#define RA_GRAPH_BATCH 16        /* keys a search expands per round */

/*
 * Build one query head's key graph on the host from its prefill queries'
 * links (steps 2 and 3 of the frame): for query t = 0, 1, ... its best key
 * hubs[t] (-1: none) and its top keys lists[t][0 .. K) (-1 padded, any
 * order) are linked: for each other key b of the list, in ascending
 * position, hub -> b and b -> hub. Each key keeps its first D distinct
 * neighbours. *entry = the key that is the hub of the most queries (ties to
 * the lower position), -1 if no query has a hub.
 *  hubs:  host int32 [T]; lists: host int32 [T][K]; values in [-1, N).
 *  nbr:   host int32 [N][D], written in full (-1 padded).
 *  1 <= D <= RA_GRAPH_MAX_DEGREE, K >= 1, T >= 0, N >= 1.
 * Returns RA_ERR_INVALID_ARGUMENT for other arguments or values.
 */
ra_status ra_graph_build(const int32_t* hubs, const int32_t* lists, int32_t T, int32_t K,
                         int32_t N, int32_t D, int32_t* nbr, int32_t* entry);

/*
 * Step 4 of the frame: each query head h searches its key graph (nbr[h],
 * entry[h], over keys [0, N) of sequence seq, KV head h / G) best-first: a
 * result list of the ef best keys visited so far by (score, lower
 * position); each round expands the RA_GRAPH_BATCH best keys of the list
 * not yet expanded (each neighbour not visited before is visited, scored
 * and offered to the list) until every key in the list has been expanded. A score is q . k in fp32:
 * the bf16 products added dimension by dimension, 0 to 127, each sum
 * rounded (an fma chain).
 *  q:           device bf16 [H_q][128], 16-byte aligned.
 *  nbr:         device int32 [H_q][N][D] (neighbours outside [0, N) are
 *               skipped); entry: device int32 [H_q] (outside [0, N): no
 *               search, no keys).
 *  1 <= D <= RA_GRAPH_MAX_DEGREE, 1 <= k <= ef <= RA_GRAPH_MAX_EF,
 *  1 <= N <= RA_GRAPH_MAX_N.
 *  out_idx:     device int32 [H_q][k]: the best min(k, list size) keys in
 *               ascending position, then -1.
 *  out_visited: device int32 [H_q]: keys visited (scored) by the search.
 * One block of RA_GRAPH_BATCH waves per query head, no workspace; async on
 * `stream`; validation as for ra_decode_step.
 */
ra_status ra_graph_search(const uint16_t* q, int32_t H_q, const ra_kv_layer* kv, int32_t seq,
                          int32_t N, const int32_t* nbr, int32_t D, const int32_t* entry,
                          int32_t ef, int32_t k, int32_t* out_idx, int32_t* out_visited,
                          hipStream_t stream);

/* ------------------------------------------------------------------ */
/* Two KV tiers: attention over listed positions, and the merge of two   */
/* partial outputs (slides, frames "The GPU keeps 640 fixed positions":  */
/* W attended from GPU memory, the retrieved set from CPU memory, and    */
/* "Two local softmax outputs need global weights", Eqs. (3)-(5)).       */
/* ------------------------------------------------------------------ */

#define RA_SPARSE_MAX_K 4096

/*
 * For each query head h: softmax of z = q . k / sqrt(128) over the positions
 * idx[h][0 .. k) of sequence seq (entries outside [0, N) are skipped), times
 * V: out[h] and out_lse[h] = m + ln sum e^(z - m). No listed position gives
 * out = 0, lse = -inf. The pools of kv may be GPU memory or pinned host
 * memory mapped for the device (see ra_host_device_pointer): the kernel
 * reads host-resident rows over the host link directly.
 *  q: device bf16 [H_q][128], 16-byte aligned; idx: device int32 [H_q][k];
 *  out: device fp32 [H_q][128]; out_lse: device fp32 [H_q].
 *  1 <= k <= RA_SPARSE_MAX_K. Validation as for ra_decode_step.
 */
ra_status ra_sparse_attend(const uint16_t* q, int32_t H_q, const ra_kv_layer* kv, int32_t seq,
                           int32_t N, const int32_t* idx, int32_t k, float* out, float* out_lse,
                           hipStream_t stream);

/*
 * Merge two partial outputs per head (Eqs. (3)-(5)): with m = max(lse_a,
 * lse_b), out = (e^(lse_a - m) out_a + e^(lse_b - m) out_b) / (e^(lse_a - m)
 * + e^(lse_b - m)) and lse = m + ln of the denominator; a partial with
 * lse = -inf weighs 0, and two give out = 0, lse = -inf. All buffers device
 * fp32 ([H][128] and [H]); out/lse may alias out_a/lse_a.
 */
ra_status ra_merge_partials(const float* out_a, const float* lse_a, const float* out_b,
                            const float* lse_b, int32_t H, float* out, float* lse,
                            hipStream_t stream);

/*
 * The device address of pinned host memory (allocated with hipHostMalloc,
 * or torch's pin_memory), through hipHostGetDevicePointer: what the pools
 * of a host-resident ra_kv_layer must hold. RA_ERR_HIP if the memory is not
 * mapped for the current device.
 */
ra_status ra_host_device_pointer(const void* host, void** dev);

#ifdef __cplusplus
}
#endif

#endif /* RA_H */
