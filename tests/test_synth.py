"""The seeded generator: determinism, layout, and workload structure; and
the oracle on the tiny workload (planted needles are retrieved, the
needle-retrieval analogue of the RetrievalAttention slides' frame
"Needle retrieval works across tested positions")."""

import numpy as np
import torch

import oracle
import synth
from synth import PAGE


def c1(device="cpu", **kw):
    c = synth.config("C1")
    args = dict(H_q=c.H_q, H_kv=c.H_kv, seq_lens=list(c.seq_lens),
                ks=[c.k_for(n) for n in c.seq_lens], n_sink=c.n_sink,
                window=c.window, needles_per_head=c.needles_per_head,
                seed=c.seed, device=device)
    args.update(kw)
    return synth.make_layer(**args)


def test_same_seed_same_tensors():
    a, b = c1(), c1()
    assert torch.equal(a.q, b.q)
    assert torch.equal(a.k_pool, b.k_pool) and torch.equal(a.v_pool, b.v_pool)
    assert torch.equal(a.block_table, b.block_table)
    c = c1(seed=1)
    assert not torch.equal(a.k_pool, c.k_pool)


def test_needles_lie_in_the_selection_domain():
    L = c1()
    nd = L.needles[0]
    assert nd.shape == (8, 2)
    M = set(oracle.selection_domain(4096, 16, 64).tolist())
    assert all(int(p) in M for p in nd[:, 0])
    assert len(set(nd[:, 0].tolist())) == 8
    assert sorted(nd[:, 1].tolist()) == [0, 0, 1, 1, 2, 2, 3, 3]


def test_sink_keys_are_scaled():
    L = c1()
    K = oracle.as_f64(synth.depage(L.k_pool, L.block_table, 0, 4096))
    norms = np.linalg.norm(K[:, 0, :], axis=-1)
    assert norms[:4].min() > 3.0 * np.median(norms[4:])


def test_depage_roundtrip_with_shuffled_pages_and_ragged_lengths():
    lens = [130, 64, 1, 500]
    L = synth.make_layer(8, 2, lens, [5] * 4, 4, 8, 1, seed=3, device="cpu",
                         shuffle_pages=True, reserve_tokens=70)
    # the block table is a permutation of all pages
    used = []
    for b, n in enumerate(lens):
        p = -(-(n + 70) // PAGE)
        used += L.block_table[b, :p].tolist()
    assert sorted(used) == list(range(L.k_pool.shape[0]))
    # de-paging returns each sequence's own rows
    for b, n in enumerate(lens):
        K = synth.depage(L.k_pool, L.block_table, b, n)
        assert K.shape == (n, 2, 128)
        pg = int(L.block_table[b, 0])
        first = synth.bf16_bits(L.k_pool[pg, :, 0, :])
        np.testing.assert_array_equal(K[0], first)
        # reserved slots after the sequence start out zero
        tail = synth.depage(L.k_pool, L.block_table, b, n + 70, n, n + 70)
        assert np.all(tail == 0)


def test_lengths_drawn_in_range_and_reproducible():
    a = synth.draw_lengths(16, 32768, 131072, 0)
    assert a == synth.draw_lengths(16, 32768, 131072, 0)
    assert all(32768 <= x <= 131072 for x in a) and len(set(a)) > 8


def test_budgets_from_percentages():
    c = synth.config("C3_1")
    assert [synth.config(n).k_for(1048576) for n in ("C3_1", "C3_2", "C3_3")] == [10485, 20971, 31457]
    assert c.k_for(100) == 1
    assert synth.config("C2").k_for(131072) == 2048


def test_oracle_retrieves_every_planted_needle_on_the_tiny_workload():
    L = c1()
    q = synth.bf16_bits(L.q[0])
    K = synth.depage(L.k_pool, L.block_table, 0, 4096)
    V = synth.depage(L.v_pool, L.block_table, 0, 4096)
    res = oracle.decode(q, K, V, k=64, n_sink=16, window=64, with_dense=True)
    for pos, h in L.needles[0]:
        assert pos in res["idx"][h]
    # queries are out of distribution: the mean score is below zero
    assert res["z"][:, 4:].mean() < 0
    # exact top-k maximises the attention mass over every k-subset of M:
    # no random subset of the same size recovers more
    r = np.random.default_rng(0)
    z = res["z"]
    for h in range(4):
        full = z[h] - np.log(np.exp(z[h] - z[h].max()).sum()) - z[h].max()
        for _ in range(20):
            alt = np.union1d(res["W"], r.choice(res["M"], 64, replace=False))
            assert np.exp(full[alt]).sum() < res["mass_recovered"][h]


def test_history_takes_appended_rows_from_the_stream():
    # rows below N0 come from the pool as generated, rows past it from the
    # appended stream, whatever the pool holds there
    base = synth.make_layer(4, 2, [300], [10], 4, 8, 2, 0, "cpu", reserve_tokens=5,
                            shuffle_pages=True)
    q, k, v = synth.make_decode_stream(1, 4, 2, base.u, 5, 3, "cpu")
    # what a GPU append would have written at rows 300..304: never read
    for t in range(300, 305):
        base.k_pool[int(base.block_table[0, t // PAGE]), :, t % PAGE] = 7.0
    h = synth.history(base.k_pool, base.block_table, 0, 300, k, 303, heads=[1])
    assert h.shape == (303, 1, 128)
    assert np.array_equal(h[:300], synth.depage(base.k_pool, base.block_table, 0, 300, heads=[1]))
    assert np.array_equal(h[300:], synth.bf16_bits(k[:3, 0][:, [1]]))
    assert np.array_equal(synth.history(base.k_pool, base.block_table, 0, 300, k, 200),
                          synth.depage(base.k_pool, base.block_table, 0, 200))
