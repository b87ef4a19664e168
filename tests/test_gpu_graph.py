"""GPU parity of the query-aware key graph search (ra_graph_search, through
the C ABI) against the oracle's graph_search (slides, frame "Prefill
queries teach the key graph what matters"). The oracle builds its own graph
(oracle.graph_build) from the same links; the GPU side uses the library's
build. The search's decisions follow from fp32 scores both sides compute in
the same order, so the retrieved keys and the number of keys visited must
be equal exactly. Each round of the search expands the GRAPH_BATCH best
unexpanded keys; the oracle is run with the same batch. That batch and the
fp32 order are readings of this build, pinned on the CPU by rounds worked
by hand; one case here also checks the GPU against a search scored in plain
float64, on keys no two of which score within the fp32 bound."""

import numpy as np
import pytest
import torch

import oracle
import synth
import top_sparse_attention_gqa_amd as ra
from tests.parity import say

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


def gpu_search(L, q, seq, N, graphs, ef, k):
    """graphs: per query head (nbr [N][D], entry)."""
    H_q = q.shape[0]
    nbr = torch.tensor(np.stack([g[0] for g in graphs]), dtype=torch.int32, device=DEV)
    entry = torch.tensor([g[1] for g in graphs], dtype=torch.int32, device=DEV)
    out = torch.full((H_q, k), -7, dtype=torch.int32, device=DEV)
    vis = torch.full((H_q,), -7, dtype=torch.int32, device=DEV)
    kv = ra.KVLayer(L.k_pool, L.v_pool, L.block_table)
    ra.graph_search(q, kv, seq, N, nbr, entry, ef, k, out, vis)
    torch.cuda.synchronize()
    return out.cpu().numpy(), vis.cpu().numpy()


def compare(L, q, seq, N, links, D, ef, k):
    """links: per query head (hubs, lists). Returns the visited counts."""
    H_q, H_kv = q.shape[0], L.H_kv
    G = H_q // H_kv
    graphs = [ra.graph_build(h, l, N, D) for h, l in links]
    got, vis = gpu_search(L, q, seq, N, graphs, ef, k)
    qb = synth.bf16_bits(q)
    for h in range(H_q):
        K = synth.depage(L.k_pool, L.block_table, seq, N, heads=[h // G])[:, 0, :]
        nbr, entry = oracle.graph_build(links[h][0], links[h][1], N, D)
        want, want_vis = oracle.graph_search(qb[h], K, nbr, entry, ef, k, batch=ra.GRAPH_BATCH)
        row = got[h]
        assert np.array_equal(row[:want.size], want), (h, row[:want.size], want)
        assert (row[want.size:] == -1).all()
        assert vis[h] == want_vis, (h, vis[h], want_vis)
    return vis


def random_links(r, N, T, K):
    lists = np.stack([r.choice(N, K, replace=False) for _ in range(T)]).astype(np.int32)
    return lists[:, 0].copy(), lists


@pytest.mark.parametrize("N,D,ef,k,T,K", [
    (3000, 16, 64, 20, 400, 8),
    (5000 + 37, 32, 128, 100, 600, 16),
    (700, 64, 256, 256, 300, 32),
    # past about 800K keys the visited bitmap leaves no room for the block
    # table in LDS, and the search reads it from global memory
    (2**20 - 5, 16, 64, 20, 3000, 8),
])
def test_graph_search_parity_on_random_links(N, D, ef, k, T, K):
    say(f"case graph random links: N={N} D={D} ef={ef} k={k}")
    L = synth.make_layer(4, 2, [N], [8], 0, 0, 2, 21, DEV)
    r = np.random.default_rng(N)
    links = [random_links(r, N, T, K) for _ in range(4)]
    vis = compare(L, L.q[0], 0, N, links, D, ef, k)
    say(f"  visited: {vis.tolist()}")


def test_graph_search_on_links_from_prefill_top_k():
    # steps 1-4 of the frame end to end: prefill rows' exact top-K keys (on
    # the GPU for the library, by the oracle for the reference), their
    # links, the graphs, and a search per decode query head
    N, T, K, D, ef, k = 4096, 96, 16, 24, 96, 32
    say(f"case graph from prefill top-k: N={N} T={T} K={K}")
    L = synth.make_layer(8, 2, [N], [k], 16, 64, 2, 22, DEV)
    Q = synth.make_prefill_queries(T, 8, L.u, 23, DEV)
    kv = ra.KVLayer(L.k_pool, L.v_pool, L.block_table)
    lists = torch.empty(T, 8, K, dtype=torch.int32, device=DEV)
    hubs = torch.empty(T, 8, 1, dtype=torch.int32, device=DEV)
    ra.prefill_topk(Q, kv, 0, N, K, 16, 64, lists, ra.alloc_prefill_workspace(T, 8, N, K, device=DEV))
    ra.prefill_topk(Q, kv, 0, N, 1, 16, 64, hubs, ra.alloc_prefill_workspace(T, 8, N, 1, device=DEV))
    torch.cuda.synchronize()
    gl, gh = lists.cpu().numpy(), hubs.cpu().numpy()[:, :, 0]
    Kb = synth.depage(L.k_pool, L.block_table, 0, N)
    ol = oracle.prefill_topk(synth.bf16_bits(Q), Kb, K, 16, 64)
    oh = oracle.prefill_topk(synth.bf16_bits(Q), Kb, 1, 16, 64)[:, :, 0]
    # random scores have no ties in the band: the GPU lists are the oracle's
    assert np.array_equal(gl, ol) and np.array_equal(gh, oh)
    links = [(gh[:, h], gl[:, h, :]) for h in range(8)]
    compare(L, L.q[0], 0, N, links, D, ef, k)


def test_graph_search_on_a_complete_graph_finds_the_exact_top_k():
    N, k = 65, 10
    L = synth.make_layer(2, 1, [N], [k], 0, 0, 2, 24, DEV)
    full = np.array([[b for b in range(N) if b != a][:64] for a in range(N)], dtype=np.int32)
    nbr = torch.tensor(np.stack([full, full]), dtype=torch.int32, device=DEV)
    # entry 0's 64 neighbours are every other key
    got, vis = gpu_search(L, L.q[0], 0, N, [(full, 0), (full, 0)], 128, k)
    qb = synth.bf16_bits(L.q[0])
    K = synth.depage(L.k_pool, L.block_table, 0, N)[:, 0, :]
    for h in range(2):
        s = oracle.score_f32_ordered(qb[h], K, np.arange(N)).astype(np.float64)
        best = np.lexsort((np.arange(N), -s))[:k]
        assert got[h].tolist() == sorted(best.tolist()) and vis[h] == N


def test_graph_search_without_a_graph_returns_nothing():
    N = 500
    L = synth.make_layer(2, 1, [N], [8], 0, 0, 2, 25, DEV)
    empty = np.full((N, 4), -1, dtype=np.int32)
    got, vis = gpu_search(L, L.q[0], 0, N, [(empty, -1), (empty, 7)], 16, 8)
    assert (got[0] == -1).all() and vis[0] == 0
    assert got[1].tolist() == [7] + [-1] * 7 and vis[1] == 1


def test_graph_search_equals_an_fp64_scored_search_when_no_scores_are_close():
    # Keys whose exact scores are at least 2 fp32 dot-product bounds apart:
    # key i of head h is c_i times the unit vector of q_h's largest
    # coordinate (c_i a permutation of 0..255, exact in bf16) plus a 0.01
    # noise. Then the fp32 sum in any order ranks the keys as the exact dot
    # product does, and the GPU search must equal the oracle's search scored
    # in plain float64 (the definition), not only its fp32 reading.
    N, D, ef, k = 256, 16, 64, 32
    say(f"case graph vs fp64-scored search: N={N} D={D} ef={ef} k={k}")
    L = synth.make_layer(2, 2, [N], [8], 0, 0, 2, 26, DEV)
    r = np.random.default_rng(27)
    qb = synth.bf16_bits(L.q[0])
    n = torch.arange(N, device=DEV)
    pages, slots = L.block_table[0, n // 64].long(), n % 64
    for h in range(2):
        qf = oracle.as_f64(qb[h])
        j = int(np.argmax(np.abs(qf)))
        K = 0.01 * r.standard_normal((N, 128))
        K[:, j] = r.permutation(N)
        L.k_pool[pages, h, slots] = torch.tensor(K, dtype=torch.float32, device=DEV).to(torch.bfloat16)
    torch.cuda.synchronize()
    links = [random_links(r, N, 100, 8) for _ in range(2)]
    graphs = [ra.graph_build(hh, ll, N, D) for hh, ll in links]
    got, vis = gpu_search(L, L.q[0], 0, N, graphs, ef, k)
    for h in range(2):
        Kb = synth.depage(L.k_pool, L.block_table, 0, N, heads=[h])[:, 0, :]
        exact = oracle.as_f64(Kb) @ oracle.as_f64(qb[h])
        bound = 128 * 2.0 ** -24 / (1 - 128 * 2.0 ** -24) * (
            np.abs(oracle.as_f64(Kb)) @ np.abs(oracle.as_f64(qb[h])))
        assert np.min(np.diff(np.sort(exact))) > 2 * bound.max()
        nbr, entry = oracle.graph_build(links[h][0], links[h][1], N, D)
        want, want_vis = oracle.graph_search(qb[h], Kb, nbr, entry, ef, k, batch=ra.GRAPH_BATCH,
                                             scoring="f64")
        assert got[h][:want.size].tolist() == want.tolist() and (got[h][want.size:] == -1).all()
        assert vis[h] == want_vis
