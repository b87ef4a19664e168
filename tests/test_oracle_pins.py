"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: closed
forms, brute force over all subsets, special cases that reduce to a library
routine (scipy), algebraic invariants, and Table 1's printed KV capacities.
"""

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
D = 128


def rng(seed=0):
    return np.random.default_rng(seed)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest even) and return the raw bits."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return r


# ---------------------------------------------------------------- widening

def test_bf16_widening_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x0000, 0x8000, 0x3E00], dtype=np.uint16)
    v = oracle.as_f64(bits)
    assert v[0] == 1.0 and v[1] == -2.0
    assert v[2] == 2.0 ** -133                      # smallest bf16 subnormal
    assert v[3] == (2 - 2 ** -7) * 2.0 ** 127       # largest finite bf16
    assert v[4] == 0.0 and math.copysign(1, v[5]) == -1
    assert v[6] == 0.125


# ---------------------------------------------------------------- sets

@pytest.mark.parametrize("N,ns,win,W", [
    (10, 2, 3, [0, 1, 7, 8, 9]),
    (4, 3, 3, [0, 1, 2, 3]),
    (6, 0, 0, []),
    (6, 0, 2, [4, 5]),
    (6, 2, 0, [0, 1]),
    (1, 128, 512, [0]),
    (0, 1, 1, []),
    (700, 128, 512, list(range(0, 128)) + list(range(188, 700))),
])
def test_static_set_and_domain_by_hand(N, ns, win, W):
    assert oracle.static_set(N, ns, win).tolist() == W
    assert oracle.selection_domain(N, ns, win).tolist() == [n for n in range(N) if n not in W]


# ---------------------------------------------------------------- scores

def test_scores_unit_query_reads_one_coordinate():
    r = rng(1)
    K = to_bf16_bits(r.standard_normal((50, 2, D)))
    q = np.zeros((4, D))
    for h in range(4):
        q[h, 7 * h + 3] = 1.0
    z = oracle.scores(q, K)
    Kf = oracle.as_f64(K)
    for h in range(4):
        np.testing.assert_allclose(z[h], Kf[:, h // 2, 7 * h + 3] / math.sqrt(D), rtol=4e-16, atol=0)


def test_scores_all_ones_gives_sqrt_d():
    z = oracle.scores(np.ones((1, D)), np.ones((3, 1, D), dtype=np.float64))
    np.testing.assert_allclose(z, math.sqrt(D), rtol=1e-15)


def test_scores_gqa_contiguous_groups():
    # KV head 0 holds +1 keys, KV head 1 holds -1 keys; with G = 4 query
    # heads 0..3 must read head 0 and 4..7 head 1.
    K = np.zeros((5, 2, D))
    K[:, 0] = 1.0
    K[:, 1] = -1.0
    z = oracle.scores(np.ones((8, D)), K)
    s = math.sqrt(D)
    np.testing.assert_allclose(z[:4], s)
    np.testing.assert_allclose(z[4:], -s)


def test_scores_exact_rational_dot():
    r = rng(2)
    q = to_bf16_bits(r.standard_normal((2, D)))
    K = to_bf16_bits(r.standard_normal((6, 1, D)))
    z = oracle.scores(q, K)
    qf, Kf = oracle.as_f64(q), oracle.as_f64(K)
    for h in range(2):
        for n in range(6):
            exact = sum(Fraction(a) * Fraction(b) for a, b in zip(qf[h], Kf[n, 0]))
            assert abs(z[h, n] * math.sqrt(D) - float(exact)) <= 1e-13 * (1 + abs(float(exact)))


def test_scores_tiles_agree_across_tile_boundary():
    r = rng(3)
    N = 65536 + 300
    K = r.standard_normal((N, 1, D)).astype(np.float32)
    q = r.standard_normal((2, D))
    z = oracle.scores(q, K)
    for n in (0, 65535, 65536, N - 1):
        np.testing.assert_allclose(z[:, n], q @ K[n, 0].astype(np.float64) / math.sqrt(D), rtol=1e-13)


# ---------------------------------------------------------------- top-k

def brute_topk(z, M, k):
    """The unique subset of M of size min(k,|M|) whose every member beats
    every non-member under (higher score first, then lower position)."""
    M = list(M)
    k_eff = min(k, len(M))
    hits = []
    for S in itertools.combinations(M, k_eff):
        rest = [n for n in M if n not in S]
        ok = all((z[a] > z[b]) or (z[a] == z[b] and a < b) for a in S for b in rest)
        if ok:
            hits.append(list(S))
    assert len(hits) == 1
    return hits[0]


@pytest.mark.parametrize("seed", range(12))
def test_topk_brute_force_small(seed):
    r = rng(100 + seed)
    N = int(r.integers(1, 15))
    # few distinct values, so ties are common
    z = r.integers(-3, 4, size=N).astype(np.float64) * 0.5
    ns, win = int(r.integers(0, 4)), int(r.integers(0, 4))
    M = oracle.selection_domain(N, ns, win)
    for k in range(0, len(M) + 2):
        got = oracle.topk(z, M, k).tolist()
        assert got == sorted(got)
        assert got == brute_topk(z, M, k)


def test_topk_constant_scores_take_lowest_positions():
    z = np.full(100, 0.25)
    M = oracle.selection_domain(100, 10, 20)
    assert oracle.topk(z, M, 7).tolist() == list(range(10, 17))


def test_topk_full_sort_crosscheck():
    r = rng(4)
    N = 5000
    z = np.round(r.standard_normal(N), 2)       # many ties
    M = oracle.selection_domain(N, 16, 64)
    order = np.lexsort((M, -z[M]))              # by score desc, then position asc
    for k in (1, 10, 64, 777, len(M)):
        assert oracle.topk(z, M, k).tolist() == sorted(M[order[:k]].tolist())


def test_topk_never_returns_static_positions():
    z = np.zeros(300)
    z[:16] = 100.0       # sinks score highest
    z[-64:] = 90.0       # the recent window next
    M = oracle.selection_domain(300, 16, 64)
    om = oracle.topk(z, M, 10)
    assert set(om.tolist()).isdisjoint(oracle.static_set(300, 16, 64).tolist())


def test_topk_picks_largest_not_smallest():
    z = np.arange(50, dtype=np.float64)
    assert oracle.topk(z, np.arange(50), 3).tolist() == [47, 48, 49]


# ---------------------------------------------------------------- attention

def random_case(seed, N=300, H_kv=2, G=2, scale=1.0):
    r = rng(seed)
    q = to_bf16_bits(r.standard_normal((H_kv * G, D)) * scale)
    K = to_bf16_bits(r.standard_normal((N, H_kv, D)))
    V = to_bf16_bits(r.standard_normal((N, H_kv, D)))
    return q, K, V


def test_k_at_least_M_equals_dense():
    q, K, V = random_case(5)
    res = oracle.decode(q, K, V, k=10 ** 6, n_sink=8, window=16, with_dense=True)
    np.testing.assert_allclose(res["out"], res["dense_out"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(res["mass_recovered"], 1.0, rtol=1e-12)


def test_weights_sum_to_one_via_constant_values():
    q, K, _ = random_case(6)
    V = np.ones((300, 2, D))
    res = oracle.decode(q, K, V, k=20, n_sink=4, window=8)
    np.testing.assert_allclose(res["out"], 1.0, rtol=1e-14)


def test_merge_of_any_disjoint_partition_equals_union():
    r = rng(7)
    z = r.standard_normal(400) * 3
    V = r.standard_normal((400, D))
    S = r.choice(400, 150, replace=False)
    for parts in (1, 2, 3, 5):
        cuts = np.sort(r.choice(np.arange(1, 150), parts - 1, replace=False))
        pieces = np.split(r.permutation(S), cuts)
        o, l = oracle.merge([oracle.partial(z, V, p) for p in pieces])
        o_ref, l_ref = oracle.attend(z, V, S)
        np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-14)
        assert abs(l - l_ref) < 1e-12


def test_merge_ignores_empty_partials():
    r = rng(8)
    z = r.standard_normal(20)
    V = r.standard_normal((20, D))
    o, l = oracle.merge([oracle.partial(z, V, []), oracle.partial(z, V, [3, 4])])
    o_ref, l_ref = oracle.attend(z, V, [3, 4])
    np.testing.assert_allclose(o, o_ref, rtol=1e-14)
    o, l = oracle.merge([oracle.partial(z, V, [])])
    assert np.all(o == 0) and l == -math.inf


def test_one_hot_values_read_the_softmax_weights():
    r = rng(9)
    N = 120
    z = r.standard_normal(N) * 2
    V = np.eye(N, D)          # row i is e_i
    S = np.sort(r.choice(N, 40, replace=False))
    o, l = oracle.attend(z, V, S)
    w = softmax(z[S])
    np.testing.assert_allclose(o[S], w, rtol=1e-13)
    assert np.all(o[np.setdiff1d(np.arange(D), S)] == 0)
    assert abs(l - logsumexp(z[S])) < 1e-12


def test_constant_keys_give_mean_of_values():
    r = rng(10)
    N = 200
    K = np.tile(r.standard_normal((1, 1, D)), (N, 1, 1))
    V = r.standard_normal((N, 1, D))
    q = r.standard_normal((1, D))
    res = oracle.decode(q, K, V, k=30, n_sink=5, window=7)
    S = np.union1d(res["W"], res["idx"][0])
    np.testing.assert_allclose(res["out"][0], V[S, 0].mean(0), rtol=1e-12, atol=1e-14)
    # all scores tie, so the lowest positions of M are retrieved
    assert res["idx"][0].tolist() == list(range(5, 35))


def test_single_element_set_returns_that_value_row():
    r = rng(11)
    z = r.standard_normal(10)
    V = r.standard_normal((10, D))
    o, l = oracle.attend(z, V, [6])
    np.testing.assert_array_equal(o, V[6])
    assert l == z[6]


def test_k_zero_is_static_set_attention():
    q, K, V = random_case(12)
    res = oracle.decode(q, K, V, k=0, n_sink=4, window=32)
    W = oracle.static_set(300, 4, 32)
    z = res["z"]
    Vf = oracle.as_f64(V)
    for h in range(4):
        assert res["idx"][h].size == 0
        np.testing.assert_allclose(res["out"][h], softmax(z[h, W]) @ Vf[W, h // 2], rtol=1e-12, atol=1e-14)


def test_no_static_set_is_pure_topk_attention():
    q, K, V = random_case(13)
    res = oracle.decode(q, K, V, k=17, n_sink=0, window=0)
    z = res["z"]
    Vf = oracle.as_f64(V)
    for h in range(4):
        om = res["idx"][h]
        assert om.size == 17
        np.testing.assert_allclose(res["out"][h], softmax(z[h, om]) @ Vf[om, h // 2], rtol=1e-12, atol=1e-14)
        assert abs(res["lse"][h] - logsumexp(z[h, om])) < 1e-12


def test_decode_merge_path_equals_direct_softmax():
    q, K, V = random_case(14, scale=3.0)
    res = oracle.decode(q, K, V, k=40, n_sink=8, window=24)
    np.testing.assert_allclose(res["out_merge"], res["out"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(res["lse_merge"], res["lse"], rtol=1e-13)


def test_empty_attended_set():
    q, K, V = random_case(15, N=10)
    res = oracle.decode(q, K, V, k=0, n_sink=0, window=0)
    assert np.all(res["out"] == 0) and np.all(res["lse"] == -np.inf)


def test_large_score_range_is_stable():
    # sink-like keys with very large scores must not overflow the softmax
    z = np.array([700.0, -700.0, 699.0, 0.0])
    V = np.eye(4, D)
    o, l = oracle.attend(z, V, [0, 1, 2, 3])
    np.testing.assert_allclose(o[:4], softmax(z), rtol=1e-13, atol=1e-300)
    assert abs(l - logsumexp(z)) < 1e-10


# ---------------------------------------------------------------- KV sizing

def test_table1_kv_capacity_row():
    g = json.load(open(os.path.join(GOLDEN, "table1_kv_capacity.json")))
    m = g["model"]
    per_tok = oracle.kv_bytes_per_token(m["n_layers"], m["H_kv"], m["head_dim"], m["elem_bytes"])
    assert per_tok == 128 * 1024
    for toks, printed in zip(g["prompt_tokens"], g["printed_capacity_gb"]):
        gib = toks * per_tok / 2 ** 30
        assert float(f"{gib:.3g}") == printed or round(gib, 1) == printed


# --------------------------------------------------------------------------
# Prefill exact top-k ("Prefill queries teach the key graph what matters",
# step 1): every query row's selection, pinned by plain loops.
# --------------------------------------------------------------------------

def _dyadic_bf16(rng, shape):
    """bf16 bit patterns of small dyadic values (exact in fp64 and Fraction)."""
    vals = rng.integers(-8, 9, size=shape).astype(np.float32) / 4.0
    return (vals.view(np.uint32) >> 16).astype(np.uint16)


def _brute_prefill(Q, K, k, n_sink, window):
    """Exact Fraction scores by explicit loops; each row sorts (-z, n)."""
    T, H_q, d = Q.shape
    N, H_kv, _ = K.shape
    G = H_q // H_kv
    qf = oracle.as_f64(Q)
    kf = oracle.as_f64(K)
    M = [n for n in range(N) if n >= min(n_sink, N) and n < max(N - window, min(n_sink, N))]
    out = np.full((T, H_q, k), -1, dtype=np.int64)
    for t in range(T):
        for h in range(H_q):
            g = h // G
            z = {n: sum(Fraction(float(qf[t, h, j])) * Fraction(float(kf[n, g, j])) for j in range(d))
                 for n in M}
            best = sorted(M, key=lambda n: (-z[n], n))[:k]
            out[t, h, :len(best)] = sorted(best)
    return out


@pytest.mark.parametrize("seed,T,H_q,H_kv,N,k,ns,win", [
    (0, 3, 2, 1, 12, 3, 2, 3),
    (1, 2, 4, 2, 20, 5, 0, 0),
    (2, 4, 2, 2, 9, 20, 1, 1),      # k > |M|: all of M, padded
    (3, 1, 8, 1, 16, 1, 4, 4),
])
def test_prefill_topk_matches_loops_on_dyadic_inputs(seed, T, H_q, H_kv, N, k, ns, win):
    rng = np.random.default_rng(seed)
    d = oracle.HEAD_DIM
    Q = _dyadic_bf16(rng, (T, H_q, d))
    K = _dyadic_bf16(rng, (N, H_kv, d))
    got = oracle.prefill_topk(Q, K, k, ns, win)
    assert np.array_equal(got, _brute_prefill(Q, K, k, ns, win))


def test_prefill_topk_rows_are_independent_and_planted_keys_win():
    # key 7 + t is aligned with query row t of head 1 only: each row finds its
    # own key first; head 0 has a zero query, so all its scores tie and it
    # takes the lowest position
    rng = np.random.default_rng(5)
    T, H_q, H_kv, N, d = 4, 2, 2, 40, oracle.HEAD_DIM
    Q = np.zeros((T, H_q, d), dtype=np.float32)
    K = rng.standard_normal((N, H_kv, d)).astype(np.float32) * 0.01
    for t in range(T):
        Q[t, 1, t] = 1.0
        K[7 + t, 1, t] = 4.0
    Qb = (Q.view(np.uint32) >> 16).astype(np.uint16)
    Kb = (K.view(np.uint32) >> 16).astype(np.uint16)
    got = oracle.prefill_topk(Qb, Kb, 1, 0, 0)
    for t in range(T):
        assert got[t, 1, 0] == 7 + t
        assert got[t, 0, 0] == 0


# --------------------------------------------------------------------------
# Per-layer budgets (slides, frame "Extra experiments show where budget
# matters": a PyramidKV-style layer budget). Pinned by the properties the
# reading fixes and by brute force over every rounding on small cases.
# --------------------------------------------------------------------------

BUDGET_CASES = [(1, 7, 300), (2, 5, 1000), (3, 10, 500), (4, 60, 600), (5, 3, 250),
                (7, 11, 999), (8, 0, 700), (32, 10485, 500), (32, 20971, 0), (6, 9, 1000)]


@pytest.mark.parametrize("L,k,slope", BUDGET_CASES)
def test_layer_budgets_keep_the_total_and_fall_with_depth(L, k, slope):
    ks = oracle.layer_budgets(L, k, slope)
    assert len(ks) == L and all(isinstance(x, int) and x >= 0 for x in ks)
    assert sum(ks) == L * k
    assert all(a >= b for a, b in zip(ks, ks[1:]))
    if slope == 0 or L == 1:
        assert ks == [k] * L
    # the line through k at the middle layer: layers l and L-1-l pair up
    for l in range(L):
        assert abs(ks[l] + ks[L - 1 - l] - 2 * k) <= 1


def test_layer_budgets_endpoints_of_the_steepest_schedule():
    # slope 1: the first layer gets twice the mean and the last none
    assert oracle.layer_budgets(5, 8, 1000) == [16, 12, 8, 4, 0]
    assert oracle.layer_budgets(2, 5, 1000) == [10, 0]
    assert oracle.layer_budgets(3, 6, 500) == [9, 6, 3]


@pytest.mark.parametrize("L,k,slope", [(3, 5, 333), (4, 7, 450), (5, 3, 250), (6, 4, 700),
                                       (4, 1, 999), (5, 2, 100), (4, 1, 500), (6, 3, 500)])
def test_layer_budgets_round_like_brute_force(L, k, slope):
    # among all integer vectors with the total L*k and every entry within 1 of
    # the exact line, the one closest to it (least squares), then the one
    # that gives the extra units to the lowest layers
    exact = [Fraction(k) * (1 + Fraction(slope, 1000) * Fraction(L - 1 - 2 * l, L - 1))
             for l in range(L)]
    best = None
    for v in itertools.product(*[range(math.floor(x) - 1, math.ceil(x) + 2) for x in exact]):
        if sum(v) != L * k or min(v) < 0:
            continue
        key = (sum((Fraction(a) - x) ** 2 for a, x in zip(v, exact)), [-a for a in v])
        if best is None or key < best[0]:
            best = (key, list(v))
    assert oracle.layer_budgets(L, k, slope) == best[1]


# --------------------------------------------------------------------------
# Query-aware key graph (slides, frame "Prefill queries teach the key graph
# what matters"): the fixed-order fp32 score, the projection build and the
# best-first search.
# --------------------------------------------------------------------------

def _bits(x):
    return to_bf16_bits(np.asarray(x, dtype=np.float32))


def test_ordered_score_rounds_one_dimension_after_another():
    # 2^24 + 1 is not an fp32 value: summed in order the 1 is lost, so the
    # score is 0 although the exact dot product is 1
    q = np.zeros(D, dtype=np.float32)
    q[:3] = [2.0 ** 24, 1.0, -(2.0 ** 24)]
    K = np.ones((1, D), dtype=np.float32)
    assert oracle.score_f32_ordered(_bits(q), _bits(K), [0])[0] == 0.0
    # the same terms with the small one last: exact
    q[:3] = [2.0 ** 24, -(2.0 ** 24), 1.0]
    assert oracle.score_f32_ordered(_bits(q), _bits(K), [0])[0] == 1.0


def test_ordered_score_is_exact_on_small_integers_and_within_the_rounding_bound():
    r = rng(31)
    qi = r.integers(-3, 4, D).astype(np.float32)
    Ki = r.integers(-3, 4, (40, D)).astype(np.float32)
    got = oracle.score_f32_ordered(_bits(qi), _bits(Ki), np.arange(40))
    assert np.array_equal(got.astype(np.float64), Ki.astype(np.float64) @ qi.astype(np.float64))
    q = r.standard_normal(D).astype(np.float32)
    K = r.standard_normal((60, D)).astype(np.float32)
    qb, Kb = _bits(q), _bits(K)
    qf = oracle.as_f64(qb)
    Kf = oracle.as_f64(Kb)
    exact = Kf @ qf
    bound = D * 2.0 ** -24 / (1 - D * 2.0 ** -24) * (np.abs(Kf) @ np.abs(qf))
    got = oracle.score_f32_ordered(qb, Kb, np.arange(60)).astype(np.float64)
    assert np.all(np.abs(got - exact) <= bound)
    # positions pick rows
    assert np.array_equal(oracle.score_f32_ordered(qb, Kb, [5, 2]), got[[5, 2]].astype(np.float32))


def test_graph_build_on_a_worked_example():
    # hubs 3, 3, 1; degree cap 2; links in query order, ascending in a list
    nbr, entry = oracle.graph_build([3, 3, 1], [[1, 3, 5], [3, 4, -1], [0, 1, 2]], 6, 2)
    assert nbr.tolist() == [[1, -1], [3, 0], [1, -1], [1, 5], [3, -1], [3, -1]]
    assert entry == 3


def test_graph_build_is_symmetric_below_the_cap_and_respects_it():
    r = rng(32)
    N, T, K = 200, 60, 6
    lists = np.stack([r.choice(N, K, replace=False) for _ in range(T)])
    hubs = lists[:, 0].copy()
    nbr, entry = oracle.graph_build(hubs, lists, N, 1000)
    edges = {(a, int(b)) for a in range(N) for b in nbr[a] if b >= 0}
    assert all((b, a) in edges for a, b in edges)
    expect = set()
    for t in range(T):
        for b in lists[t]:
            if b != hubs[t]:
                expect |= {(int(hubs[t]), int(b)), (int(b), int(hubs[t]))}
    assert edges == expect
    counts = np.bincount(hubs, minlength=N)
    assert entry == int(np.flatnonzero(counts == counts.max())[0])
    capped, _ = oracle.graph_build(hubs, lists, N, 3)
    assert ((capped >= 0).sum(axis=1) <= 3).all()
    for a in range(N):  # a capped list is the start of the uncapped one
        full = [int(x) for x in nbr[a] if x >= 0]
        assert [int(x) for x in capped[a] if x >= 0] == full[:3]


def _random_keys(seed, N):
    r = rng(seed)
    return _bits(r.standard_normal(D)), _bits(r.standard_normal((N, D)))


def test_graph_search_on_a_complete_graph_is_the_exact_top_k():
    q, K = _random_keys(33, 50)
    nbr = np.array([[b for b in range(50) if b != a] for a in range(50)])
    s = oracle.score_f32_ordered(q, K, np.arange(50)).astype(np.float64)
    order = np.lexsort((np.arange(50), -s))          # best score, then lower position
    for k in (1, 7, 50):
        got, visited = oracle.graph_search(q, K, nbr, 13, ef=64, k=k)
        assert visited == 50
        assert got.tolist() == sorted(order[:k].tolist())


def test_graph_search_never_leaves_the_entry_component():
    q, K = _random_keys(34, 40)
    nbr = np.full((40, 39), -1)
    for comp in (range(0, 20), range(20, 40)):
        for a in comp:
            others = [b for b in comp if b != a]
            nbr[a, :len(others)] = others
    got, visited = oracle.graph_search(q, K, nbr, 25, ef=40, k=30)
    assert visited == 20 and set(got.tolist()) <= set(range(20, 40)) and got.size == 20


def test_greedy_graph_search_stops_at_a_local_maximum_and_walks_a_chain():
    q, K = _random_keys(35, 60)
    r = rng(36)
    nbr = np.stack([r.choice(60, 4, replace=False) for _ in range(60)])
    s = oracle.score_f32_ordered(q, K, np.arange(60))
    got, _ = oracle.graph_search(q, K, nbr, 0, ef=1, k=1)
    c = int(got[0])
    for u in nbr[c]:
        assert (s[u], -u) <= (s[c], -c) or u == c
    # a chain whose scores rise along it: greedy search walks to its end
    chain = np.argsort(s)                     # lowest to highest score
    cn = np.full((60, 2), -1)
    for i in range(59):
        cn[chain[i], 0] = chain[i + 1]
        cn[chain[i + 1], 1] = chain[i]
    got, visited = oracle.graph_search(q, K, cn, int(chain[0]), ef=1, k=1)
    assert got.tolist() == [int(chain[-1])] and visited == 60


def test_batched_graph_search_on_a_complete_graph_and_a_chain():
    # a batch of b expands the b best unexpanded keys per round; on a
    # complete graph every batch visits everything and returns the exact
    # top-k, and on a rising chain it still walks to the end
    q, K = _random_keys(37, 300)
    s = oracle.score_f32_ordered(q, K, np.arange(300)).astype(np.float64)
    full = np.array([[b for b in range(300) if b != a] for a in range(300)])
    for batch in (1, 4):
        got, visited = oracle.graph_search(q, K, full, 0, ef=300, k=25, batch=batch)
        assert visited == 300
        assert got.tolist() == sorted(np.lexsort((np.arange(300), -s))[:25].tolist())
    chain = np.argsort(s)
    cn = np.full((300, 2), -1)
    for i in range(299):
        cn[chain[i], 0] = chain[i + 1]
        cn[chain[i + 1], 1] = chain[i]
    got, visited = oracle.graph_search(q, K, cn, int(chain[0]), ef=2, k=1, batch=2)
    assert got.tolist() == [int(chain[-1])] and visited == 300


# A 12-key graph searched by hand (slides, frame "Prefill queries teach the
# key graph what matters", step 4: best-first search of the key graph).
# q = e_0 and key i = S[i] e_0, so key i scores S[i] exactly in bf16 and in
# any summation order; entry 0, ef = 4, k = 3. Key 10 (score 10) is reached
# only through key 5 (score 3), which no batch keeps long enough to expand.
_HW_S = [5, 2, 9, 1, 7, 3, 11, 4, 8, 6, 10, 0]
_HW_NBR = [[1, 2, 3], [0, 4, 5], [0, 6, 7], [0, 8], [1, 9], [1, 10], [2, 11], [2], [3], [4],
           [5], [6]]
T, F = True, False
# per batch: (per round: R as (key, expanded) in rank order, visited keys),
# the result, the number of keys visited
_HW_TRACES = {
    # one key per round: 0; 2 (6, 7 join, 1 and 3 drop); 6 (11 joins and
    # drops); 7 (nothing new)
    1: ([([(2, F), (0, T), (1, F), (3, F)], [0, 1, 2, 3]),
         ([(6, F), (2, T), (0, T), (7, F)], [0, 1, 2, 3, 6, 7]),
         ([(6, T), (2, T), (0, T), (7, F)], [0, 1, 2, 3, 6, 7, 11]),
         ([(6, T), (2, T), (0, T), (7, T)], [0, 1, 2, 3, 6, 7, 11])],
        [0, 2, 6], 7),
    # two per round: 0; 2 and 1 (6, 7, 4, 5 join; 7 drops); 6 and 4 (11, 9
    # join, 11 drops, 0 drops); 9 (nothing new)
    2: ([([(2, F), (0, T), (1, F), (3, F)], [0, 1, 2, 3]),
         ([(6, F), (2, T), (4, F), (0, T)], [0, 1, 2, 3, 4, 5, 6, 7]),
         ([(6, T), (2, T), (4, T), (9, F)], [0, 1, 2, 3, 4, 5, 6, 7, 9, 11]),
         ([(6, T), (2, T), (4, T), (9, T)], [0, 1, 2, 3, 4, 5, 6, 7, 9, 11])],
        [2, 4, 6], 10),
    # four per round: 0; 2, 1 and 3 (8 joins as well); 6, 8 and 4 (11 and 9
    # join and drop); every key in R expanded
    4: ([([(2, F), (0, T), (1, F), (3, F)], [0, 1, 2, 3]),
         ([(6, F), (2, T), (8, F), (4, F)], [0, 1, 2, 3, 4, 5, 6, 7, 8]),
         ([(6, T), (2, T), (8, T), (4, T)], [0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 11])],
        [2, 6, 8], 11),
}


def _hand_graph():
    q = np.zeros(D, dtype=np.float32)
    q[0] = 1.0
    K = np.zeros((12, D), dtype=np.float32)
    K[:, 0] = _HW_S
    nbr = np.full((12, 3), -1)
    for a, row in enumerate(_HW_NBR):
        nbr[a, :len(row)] = row
    return _bits(q), _bits(K), nbr


@pytest.mark.parametrize("batch", [1, 2, 4])
def test_graph_search_rounds_on_a_graph_worked_by_hand(batch):
    q, K, nbr = _hand_graph()
    rounds, result, n_visited = _HW_TRACES[batch]
    for scoring in ("f32", "f64"):
        trace = []
        got, visited = oracle.graph_search(q, K, nbr, 0, ef=4, k=3, batch=batch,
                                           scoring=scoring, trace=trace)
        assert got.tolist() == result and visited == n_visited
        assert len(trace) == len(rounds)
        for (R, V), (R_want, V_want) in zip(trace, rounds):
            assert [(int(a), bool(b)) for a, b in R] == R_want and list(V) == V_want


def test_graph_search_in_fp32_order_equals_fp64_when_no_two_scores_are_close():
    # scores spread far apart along q (gaps of about 0.05 |q|^2, far above
    # the fp32 dot-product bound): the ordered fp32 sum ranks the keys as
    # the exact dot product does, so the searches agree round by round
    r = rng(38)
    N = 400
    qf = r.standard_normal(D).astype(np.float32)
    qh = qf / np.linalg.norm(qf)
    c = r.permutation(N) * 0.05
    Kf = (0.01 * r.standard_normal((N, D)) + np.outer(c, qh)).astype(np.float32)
    q, K = _bits(qf), _bits(Kf)
    exact = oracle.as_f64(K) @ oracle.as_f64(q)
    bound = D * 2.0 ** -24 / (1 - D * 2.0 ** -24) * (np.abs(oracle.as_f64(K)) @ np.abs(oracle.as_f64(q)))
    s = np.sort(exact)
    assert np.min(np.diff(s)) > 2 * bound.max()
    nbr = np.stack([r.choice(N, 8, replace=False) for _ in range(N)])
    for batch in (1, 16):
        t32, t64 = [], []
        a = oracle.graph_search(q, K, nbr, 0, ef=32, k=16, batch=batch, scoring="f32", trace=t32)
        b = oracle.graph_search(q, K, nbr, 0, ef=32, k=16, batch=batch, scoring="f64", trace=t64)
        assert a[0].tolist() == b[0].tolist() and a[1] == b[1] and t32 == t64


def test_graph_search_scored_in_fp64_on_a_complete_graph_is_the_exact_top_k():
    q, K = _random_keys(39, 80)
    nbr = np.array([[b for b in range(80) if b != a] for a in range(80)])
    s = oracle.as_f64(K) @ oracle.as_f64(q)
    order = np.lexsort((np.arange(80), -s))
    got, visited = oracle.graph_search(q, K, nbr, 3, ef=80, k=9, batch=16, scoring="f64")
    assert visited == 80 and got.tolist() == sorted(order[:9].tolist())
