"""GPU parity of the prefill exact top-k (ra_prefill_topk, through the C ABI)
against the fp64 oracle's prefill_topk, row by row: indices must equal the
oracle's outside the tie band of reading 12 (|z - z_(k)| <= 1e-3 |z_(k)| +
the fp32 dot-product bound), be unique, ascending, inside M and padded with
-1. Shapes span several 128-row blocks and 64-key pages with ragged tails,
G = 1, 2, 4, 8, shuffled pages and a second sequence's block-table row."""

import numpy as np
import pytest
import torch

import oracle
import synth
import top_sparse_attention_gqa_amd as ra
from tests.parity import check_indices, gamma, say, score_bound

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


def gpu_prefill(L, Q, seq, N, k, ns, win, flags=False):
    T, H_q = Q.shape[0], Q.shape[1]
    kv = ra.KVLayer(L.k_pool, L.v_pool, L.block_table)
    out = torch.full((T, H_q, max(k, 1)), -7, dtype=torch.int32, device=DEV)
    ws = ra.alloc_prefill_workspace(T, H_q, N, k, device=DEV)
    ws.fill_(0xA5)  # no initial contents are required
    ra.prefill_topk(Q, kv, seq, N, k, ns, win, out if k else None, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()[:, :, :k]
    if not flags:
        return got
    return got, ra.prefill_fail_flags(ws, T, H_q, N, k).cpu().numpy()


def compare_rows(L, Q, seq, N, k, ns, win, got, rows=None) -> int:
    """Every (row, head) of `rows` (default all) against the oracle; returns
    the number of tie-band differences."""
    Qb = synth.bf16_bits(Q)
    Kb = synth.depage(L.k_pool, L.block_table, seq, N)
    M = oracle.selection_domain(N, ns, win)
    diffs = 0
    for t in (range(Qb.shape[0]) if rows is None else rows):
        z = oracle.scores(Qb[t], Kb)
        res = {"z": z, "M": M, "idx": [oracle.topk(z[h], M, k) for h in range(Qb.shape[1])]}
        eps = gamma(130) * score_bound(Qb[t], Kb).max(axis=1)
        for h in range(Qb.shape[1]):
            diffs += check_indices(got[t, h], res, h, k, eps[h])
    return diffs


CASES = [
    # name, H_q, H_kv, lens, seq, T, k, n_sink, window, shuffle
    ("c1_shape", 4, 1, [4096], 0, 64, 64, 16, 64, False),
    ("llama_ragged", 32, 8, [8192 + 37], 0, 33, 100, 128, 512, False),
    ("g1", 2, 2, [3000], 0, 70, 10, 0, 0, False),
    ("g8_kmax", 8, 1, [5000], 0, 17, 256, 4, 4, False),
    ("k_gt_M", 4, 2, [300], 0, 40, 100, 100, 150, False),
    ("k_one", 8, 2, [2049], 0, 50, 1, 8, 8, False),
    ("second_sequence_shuffled", 8, 2, [1500, 6000 + 5], 1, 45, 32, 16, 64, True),
    ("one_page", 4, 1, [63], 0, 5, 16, 0, 0, False),
    # k = 256 with a sampled bound below the sampled pages present (the
    # smaller cases above keep every member of M as a candidate)
    ("kmax_sampled_bound", 8, 2, [60000 + 17], 0, 24, 256, 64, 256, True),
]


@pytest.mark.parametrize("name,H_q,H_kv,lens,seq,T,k,ns,win,shuffle", CASES,
                         ids=[c[0] for c in CASES])
def test_prefill_topk_parity(name, H_q, H_kv, lens, seq, T, k, ns, win, shuffle):
    say(f"case prefill {name}: H_q={H_q} H_kv={H_kv} N={lens[seq]} T={T} k={k}")
    L = synth.make_layer(H_q, H_kv, lens, [min(k, 8)] * len(lens), ns, win, 2, 11, DEV,
                         shuffle_pages=shuffle)
    Q = synth.make_prefill_queries(T, H_q, L.u, 12, DEV)
    got = gpu_prefill(L, Q, seq, lens[seq], k, ns, win)
    d = compare_rows(L, Q, seq, lens[seq], k, ns, win, got)
    say(f"  band differences: {d}")


def test_prefill_constant_keys_take_the_lowest_positions():
    say("case prefill constant keys: N=3000, k=40")
    L = synth.make_layer(8, 2, [3000], [8], 16, 64, 2, 3, DEV)
    L.k_pool.fill_(0.125)
    Q = synth.make_prefill_queries(20, 8, L.u, 4, DEV)
    got, fail = gpu_prefill(L, Q, 0, 3000, 40, 16, 64, flags=True)
    assert np.array_equal(got, np.broadcast_to(np.arange(16, 56), got.shape))
    # every key ties: the sampled bound admits all 2920 members of M, more
    # than a row's lists hold, so every row is decided by the exact pass
    assert fail.all()


def test_prefill_integer_scores_resolve_ties_exactly():
    say("case prefill ternary: integer dot products, N=4000, k=50")
    L = synth.make_layer(8, 2, [4000], [8], 8, 8, 2, 5, DEV)
    g = torch.Generator(device=DEV).manual_seed(9)
    L.k_pool.copy_(torch.randint(-1, 2, L.k_pool.shape, generator=g, device=DEV).to(torch.bfloat16))
    Q = torch.randint(-1, 2, (24, 8, 128), generator=g, device=DEV).to(torch.bfloat16)
    got = gpu_prefill(L, Q, 0, 4000, 50, 8, 8)
    want = oracle.prefill_topk(synth.bf16_bits(Q), synth.depage(L.k_pool, L.block_table, 0, 4000),
                               50, 8, 8)
    assert np.array_equal(got, want)


def test_prefill_planted_keys_are_found_per_row():
    # row t of head 3 is aligned with key 1000 + 7 t: every row finds its own
    say("case prefill planted: N=9000, T=40")
    L = synth.make_layer(4, 1, [9000], [8], 0, 0, 2, 6, DEV)
    Q = synth.make_prefill_queries(40, 4, L.u, 7, DEV)
    for t in range(40):
        n = 1000 + 7 * t
        pg = int(L.block_table[0, n // 64])
        L.k_pool[pg, 0, n % 64] = (Q[t, 3].float() * 0.5).to(torch.bfloat16)
    got = gpu_prefill(L, Q, 0, 9000, 8, 0, 0)
    for t in range(40):
        assert 1000 + 7 * t in got[t, 3]


def test_prefill_k_zero_writes_nothing():
    L = synth.make_layer(4, 1, [1000], [8], 0, 0, 2, 1, DEV)
    Q = synth.make_prefill_queries(8, 4, L.u, 2, DEV)
    kv = ra.KVLayer(L.k_pool, L.v_pool, L.block_table)
    ws = ra.alloc_prefill_workspace(8, 4, 1000, 0, device=DEV)
    ra.prefill_topk(Q, kv, 0, 1000, 0, 0, 0, None, ws)
    torch.cuda.synchronize()


def test_prefill_index_build_workload_sampled_rows():
    # the benchmark's shape: T = 1024 prefill rows of a Llama-3-8B layer at
    # N = 131072, k = 100; 6 rows (all 32 heads each) checked against the oracle
    say("case prefill P1: H_q=32 H_kv=8 N=131072 T=1024 k=100 (6 rows checked)")
    L = synth.make_layer(32, 8, [131072], [2048], 128, 512, 64, 0, DEV)
    Q = synth.make_prefill_queries(1024, 32, L.u, 1, DEV)
    got, fail = gpu_prefill(L, Q, 0, 131072, 100, 128, 512, flags=True)
    d = compare_rows(L, Q, 0, 131072, 100, 128, 512, got, rows=[0, 1, 127, 128, 511, 1023])
    say(f"  band differences: {d}; rows left to the exact pass: {int(fail.sum())}")
    # the sampled bound decides (nearly) every row here
    assert fail.sum() <= fail.size // 100


def test_prefill_exact_pass_on_flagged_rows():
    # The sampled half runs, then chosen rows are flagged (their output
    # poisoned) and the exact half recomputes them: rows in several row
    # blocks of each KV head, one row block with no flagged row.
    T, H_q, H_kv, N, k, ns, win = 300, 8, 2, 20000 + 11, 48, 32, 96
    say(f"case prefill forced exact pass: H_q={H_q} H_kv={H_kv} N={N} T={T} k={k}")
    L = synth.make_layer(H_q, H_kv, [N], [8], ns, win, 2, 21, DEV)
    Q = synth.make_prefill_queries(T, H_q, L.u, 22, DEV)
    kv = ra.KVLayer(L.k_pool, L.v_pool, L.block_table)
    out = torch.full((T, H_q, k), -7, dtype=torch.int32, device=DEV)
    ws = ra.alloc_prefill_workspace(T, H_q, N, k, device=DEV)
    ws.fill_(0xA5)
    ra.prefill_stages(Q, kv, 0, N, k, ns, win, out, ws, ra.PF_STAGE_SAMPLE, ra.PF_STAGE_SELECT)
    torch.cuda.synchronize()
    fail = ra.prefill_fail_flags(ws, T, H_q, N, k)
    natural = fail.cpu().numpy().copy()
    forced = [(5, 0), (5, 3), (150, 6), (151, 1), (299, 7)]  # local rows 20, 23, 602, 605, 1199
    for t, h in forced:
        fail[t, h] = 1
        out[t, h] = -7
    ra.prefill_stages(Q, kv, 0, N, k, ns, win, out, ws, ra.PF_STAGE_EXACT_MAXIMA,
                      ra.PF_STAGE_EXACT_SELECT)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert (got != -7).all()
    rows = sorted({t for t, _ in forced} | {0, 100, 200} | set(np.nonzero(natural)[0][:4].tolist()))
    d = compare_rows(L, Q, 0, N, k, ns, win, got, rows=rows)
    say(f"  natural exact-pass rows: {int(natural.sum())}; band differences: {d}")


def test_prefill_ignores_nan_in_unused_page_slots():
    say("case prefill NaN tail: N=1000+3, unused slots of the last page hold NaN")
    L = synth.make_layer(4, 1, [1003], [8], 0, 0, 2, 8, DEV, tail_fill=float("nan"))
    Q = synth.make_prefill_queries(30, 4, L.u, 9, DEV)
    got = gpu_prefill(L, Q, 0, 1003, 20, 0, 0)
    compare_rows(L, Q, 0, 1003, 20, 0, 0, got)
