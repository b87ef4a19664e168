"""The argument the prefill's filters rest on, checked on the CPU with the
oracle's top-k: keys compare by the pair (score, page), larger score first,
then lower page (page = position // 64). For ANY bound t, the set C of the
members of M whose pair reaches t holds the exact top k_eff of M whenever
|C| >= k_eff, ties to the lower position included: a key outside C has a
smaller score than every key in C, or an equal score on a later page. The
sampled pass of ra_prefill_topk takes t from a sample of the pages and falls
back to the exact pass when |C| < k_eff or C did not fit; the exact pass
takes t from the page maxima, where |C| >= k_eff always holds."""

import numpy as np
import pytest

import oracle

PAGE = 64


def pair_set(z, M, t_score, t_page):
    pg = M // PAGE
    s = z[M]
    return M[(s > t_score) | ((s == t_score) & (pg <= t_page))]


@pytest.mark.parametrize("seed", range(40))
def test_topk_of_a_pair_bounded_set_is_the_exact_topk(seed):
    r = np.random.default_rng(seed)
    N = int(r.integers(65, 700))
    ns, win = int(r.integers(0, 40)), int(r.integers(0, 80))
    # few distinct scores: ties inside and across pages are the common case
    z = r.integers(0, 6, N).astype(np.float64)
    M = oracle.selection_domain(N, ns, win)
    k = int(r.integers(1, 60))
    want = oracle.topk(z, M, k)
    held = 0
    kth = float(np.sort(z[M])[::-1][min(k, M.size) - 1])
    for i in range(30):
        # bounds at, between and around the scores and pages that occur; the
        # first one (the k-th score, every page) always keeps enough
        t_score = kth if i == 0 else float(r.choice(z)) + float(r.choice([0.0, 0.0, 0.5, -0.5]))
        t_page = N // PAGE if i == 0 else int(r.integers(-1, N // PAGE + 2))
        C = pair_set(z, M, t_score, t_page)
        if C.size >= min(k, M.size):
            held += 1
            assert np.array_equal(oracle.topk(z, C, k), want)
    assert held > 0


def test_page_maxima_bound_holds_the_topk_within_k_pages():
    # the exact pass: t = the k-th largest (page maximum, page) pair; its set
    # has at least k keys and lies in the k pages that reach t
    r = np.random.default_rng(7)
    for _ in range(50):
        N = int(r.integers(64 * 3, 64 * 30))
        z = r.integers(0, 8, N).astype(np.float64)
        M = oracle.selection_domain(N, 5, 17)
        pages = np.unique(M // PAGE)
        k = int(r.integers(1, pages.size + 1))
        pm = np.array([z[M[M // PAGE == p]].max() for p in pages])
        order = sorted(range(pages.size), key=lambda i: (-pm[i], pages[i]))
        t = order[k - 1]
        C = pair_set(z, M, pm[t], pages[t])
        assert k <= C.size <= PAGE * k
        assert np.unique(C // PAGE).size <= k
        assert np.array_equal(oracle.topk(z, C, k), oracle.topk(z, M, k))


def test_a_bound_that_keeps_too_few_is_not_enough():
    # the reason the sampled pass checks |C| >= k_eff: with fewer, the set
    # misses members of the top-k
    z = np.arange(200, dtype=np.float64)[::-1].copy()  # position 0 is the best
    M = oracle.selection_domain(200, 0, 0)
    C = pair_set(z, M, 195.0, 0)                       # the five best
    assert C.size == 5
    assert not np.array_equal(oracle.topk(z, C, 10), oracle.topk(z, M, 10))
