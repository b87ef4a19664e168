"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on
the same seeded inputs, element by element, with the tolerances stated in
tests/parity.py. Small cases span several tiles and a ragged tail; the
workload-sized cases run in the launch configuration the benchmark times."""

import numpy as np
import pytest
import torch

import synth
import top_sparse_attention_gqa_amd as ra
from tests.parity import compare_sequence, gpu_decode, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


def layer(H_q, H_kv, lens, ks, n_sink, window, needles=2, seed=0, **kw):
    return synth.make_layer(H_q, H_kv, list(lens), list(ks), n_sink, window, needles, seed,
                            DEV, **kw)


def cfg_layer(name, seed=None):
    c = synth.config(name)
    lens = list(c.seq_lens) if c.seq_lens else synth.draw_lengths(c.B, *c.len_range, c.seed)
    return synth.make_layer(c.H_q, c.H_kv, lens, [c.k_for(n) for n in lens], c.n_sink,
                            c.window, c.needles_per_head, c.seed if seed is None else seed,
                            DEV, shuffle_pages=c.shuffle_pages)


def test_c1_tiny_full_parity():
    say("case C1: H_q=4 H_kv=1 N=4096 k=64 n_sink=16 window=64")
    L = cfg_layer("C1")
    run = gpu_decode(L, with_scores=True)
    st = compare_sequence(L, run, 0)
    # every planted needle is retrieved by its head
    for pos, h in L.needles[0]:
        assert pos in run.idx[0, h]
    assert st["band_diffs"] == 0


def test_boundary_prototype_equals_the_extended_call():
    # ra_decode_step (the boundary's own prototype: no out_lse, no flags)
    # against ra_decode_step_ex on the same inputs: bit-identical out and
    # out_idx, both equal to the oracle
    say("case boundary: C1 through ra_decode_step and ra_decode_step_ex")
    L = cfg_layer("C1")
    n, k = L.seq_lens[0], L.ks[0]
    kv = ra.KVLayer(L.k_pool, L.v_pool, L.block_table)
    seq = torch.tensor([n], dtype=torch.int32, device=DEV)
    kt = torch.tensor([k], dtype=torch.int32, device=DEV)
    out = torch.full((1, L.H_q, 128), float("nan"), device=DEV)
    idx = torch.full((1, L.H_q, k), -7, dtype=torch.int32, device=DEV)
    ws = ra.alloc_workspace(1, L.H_q, L.H_kv, n, k, device=DEV)
    ra.decode_step(L.q, kv, seq, n, kt, k, L.n_sink, L.window, out, idx, ws)
    run = gpu_decode(L)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().astype(np.float64), run.out)
    assert np.array_equal(idx.cpu().numpy(), run.idx)
    compare_sequence(L, run, 0)


def test_kv_append_writes_the_right_slot():
    say("case kv_append: B=3 H_kv=2 shuffled pages")
    L = layer(8, 2, [100, 64, 1], [4, 4, 4], 4, 8, shuffle_pages=True, reserve_tokens=130)
    kv = ra.KVLayer(L.k_pool, L.v_pool, L.block_table)
    before_k = L.k_pool.clone()
    before_v = L.v_pool.clone()
    pos = torch.tensor([100, 64, 128], dtype=torch.int32, device=DEV)
    kn, vn = synth.make_new_tokens(3, 2, L.u, 5, DEV)
    ra.kv_append(kv, kn, vn, pos)
    torch.cuda.synchronize()
    exp_k, exp_v = before_k.clone(), before_v.clone()
    for b, p in enumerate(pos.tolist()):
        pg = int(L.block_table[b, p // 64])
        exp_k[pg, :, p % 64] = kn[b]
        exp_v[pg, :, p % 64] = vn[b]
    assert torch.equal(L.k_pool.view(torch.int16), exp_k.view(torch.int16))
    assert torch.equal(L.v_pool.view(torch.int16), exp_v.view(torch.int16))


EDGE = [
    # name, H_q, H_kv, lens, k, n_sink, window
    ("one_token", 4, 1, [1], 3, 16, 64),
    ("page_minus_one", 4, 1, [63], 5, 4, 8),
    ("one_page", 4, 1, [64], 5, 4, 8),
    ("page_plus_one", 4, 1, [65], 5, 4, 8),
    ("ragged_tail", 4, 1, [5000], 64, 16, 64),
    ("two_tiles", 4, 1, [8193], 100, 16, 64),
    ("three_tiles", 8, 2, [20000], 300, 128, 512),
    ("k_zero_streaming", 4, 1, [3000], 0, 16, 64),
    ("k_one", 4, 1, [3000], 1, 16, 64),
    ("k_all_is_dense", 4, 1, [2000], 5000, 16, 64),
    ("no_static_set", 4, 1, [3000], 50, 0, 0),
    ("window_covers_all", 4, 1, [300], 10, 0, 400),
    ("sink_covers_all", 4, 1, [300], 10, 400, 0),
    ("overlapping_static", 4, 1, [500], 10, 300, 300),
    ("gqa1", 2, 2, [7000], 70, 16, 64),
    ("gqa2", 4, 2, [7000], 70, 16, 64),
    ("gqa8", 8, 1, [7000], 70, 16, 64),
    ("gqa8_two_groups", 16, 2, [9000], 70, 16, 64),
]


@pytest.mark.parametrize("name,H_q,H_kv,lens,k,ns,win", EDGE, ids=[e[0] for e in EDGE])
def test_edge_cases(name, H_q, H_kv, lens, k, ns, win):
    say(f"case {name}: H_q={H_q} H_kv={H_kv} N={lens} k={k} n_sink={ns} window={win}")
    L = layer(H_q, H_kv, lens, [k] * len(lens), ns, win)
    run = gpu_decode(L, with_scores=True)
    for b in range(len(lens)):
        compare_sequence(L, run, b)


def test_garbage_after_the_last_token_is_ignored():
    say("case nan_tail: N=4000 with NaN in the unused page slots")
    L = layer(4, 1, [4000], [64], 16, 64, tail_fill=float("nan"))
    run = gpu_decode(L, with_scores=True)
    compare_sequence(L, run, 0)
    assert np.isfinite(run.out).all()


def test_ragged_batch_with_shuffled_pages():
    lens = [1, 700, 8192, 8250, 19000]
    say(f"case ragged: B=5 lens={lens} shuffled")
    L = layer(8, 2, lens, [0, 20, 100, 170, 380], 16, 64, shuffle_pages=True)
    run = gpu_decode(L, max_seq_len=20000, k_max=400, with_scores=True)
    for b in range(len(lens)):
        compare_sequence(L, run, b)


def test_large_ragged_batches():
    # 64 and 70 short sequences of random lengths (many with an empty or
    # tiny M) and budgets, shuffled pages, every sequence against the oracle
    import random
    rnd = random.Random(11)
    for B in (64, 70):
        lens = [rnd.randint(1, 5000) for _ in range(B)]
        ks = [rnd.randint(0, 60) for _ in range(B)]
        say(f"case batch_{B}: H_q=4 H_kv=1 ragged lengths up to 5000, shuffled")
        L = layer(4, 1, lens, ks, 16, 64, seed=B, shuffle_pages=True)
        run = gpu_decode(L, with_scores=True)
        for b in range(B):
            compare_sequence(L, run, b)


def test_constant_keys_tie_to_the_lowest_positions():
    say("case ties_cand: constant keys, N=6000 (bucket fits the candidate list)")
    L = layer(4, 1, [6000], [333], 16, 64)
    L.k_pool.fill_(0.5)
    run = gpu_decode(L)
    compare_sequence(L, run, 0)
    for h in range(4):
        assert run.idx[0, h].tolist() == list(range(16, 16 + 333))


def test_constant_keys_rescan_path():
    # every score ties, so the threshold bucket (|M| = 39360) exceeds the
    # 32768-entry candidate list and the head's row is re-read
    say("case ties_rescan: constant keys, N=40000")
    L = layer(4, 1, [40000], [5000], 16, 64)
    L.k_pool.fill_(-0.25)
    run = gpu_decode(L)
    compare_sequence(L, run, 0)
    for h in range(4):
        assert run.idx[0, h].tolist() == list(range(16, 16 + 5000))


def sample_stride(P):
    """One page in S is sampled (page j with j % S == S / 2): S is the
    largest power of two up to 64 that leaves at least 16 sampled pages."""
    s = 0
    while s < 6 and (P >> (s + 1)) >= 16:
        s += 1
    return 1 << s


def plant_on_sampled_pages(L, b, g, boost=3.0):
    """Keys aligned with the group's queries on exactly the sampled pages of
    (b, g): the sample then sees only high scores, its threshold leaves fewer
    than k candidates, and the group takes the full rescan."""
    G = L.H_q // L.H_kv
    P = (L.seq_lens[b] + 63) // 64
    S = sample_stride(P)
    qdir = L.q[b, g * G:(g + 1) * G].float().sum(0)
    qdir = qdir / qdir.norm()
    for j in range(S // 2, P, S):
        pg = int(L.block_table[b, j])
        L.k_pool[pg, g] = (L.k_pool[pg, g].float() + boost * qdir).to(torch.bfloat16)


def test_misleading_sample_takes_the_dense_path():
    say("case sample_misled: N=32768, high keys on the sampled pages only, k=9000")
    L = layer(4, 1, [32768], [9000], 16, 64)
    plant_on_sampled_pages(L, 0, 0)
    run = gpu_decode(L, with_scores=True)
    assert run.rescanned > 0
    compare_sequence(L, run, 0)


def test_dense_path_in_some_groups_of_a_batch():
    # two of four (sequence, KV head) groups are rescanned, by blocks that
    # also scan units of the other groups; the rest keep their candidates
    say("case sample_misled_batch: B=2 H_kv=2, groups (0,0) and (1,1) misled")
    L = layer(8, 2, [32768, 24576 + 37], [9000, 6000], 16, 64, seed=3)
    plant_on_sampled_pages(L, 0, 0)
    plant_on_sampled_pages(L, 1, 1)
    run = gpu_decode(L, with_scores=True)
    assert run.rescanned > 0
    compare_sequence(L, run, 0)
    compare_sequence(L, run, 1)


def test_rescan_in_a_batch_with_more_heads_than_cus():
    # 70 sequences x 4 query heads with budgets up to 6000: the select runs
    # two blocks per CU, and the rescan in a launch of its own; one group's
    # sample is misled, so its heads take the rescan there
    import random
    rnd = random.Random(12)
    lens = [rnd.randint(1000, 4000) for _ in range(69)] + [32768]
    ks = [rnd.randint(0, 50) for _ in range(69)] + [6000]
    say("case narrow_select_rescan: B=70 H_q=4 H_kv=1, the last sequence misled, k=6000")
    L = layer(4, 1, lens, ks, 16, 64, seed=13, shuffle_pages=True)
    plant_on_sampled_pages(L, 69, 0)
    run = gpu_decode(L, with_scores=True)
    assert run.rescanned > 0
    for b in (0, 1, 35, 68, 69):
        compare_sequence(L, run, b)


def test_integer_scores_with_many_ties():
    say("case ternary: integer-valued dot products, N=12000")
    L = layer(8, 2, [12000], [700], 16, 64)
    g = torch.Generator(device=DEV).manual_seed(7)
    L.k_pool.copy_(torch.randint(-1, 2, L.k_pool.shape, generator=g, device=DEV).to(torch.bfloat16))
    L.q.copy_(torch.randint(-1, 2, L.q.shape, generator=g, device=DEV).to(torch.bfloat16))
    run = gpu_decode(L, with_scores=True)
    st = compare_sequence(L, run, 0)
    # integer dot products are exact in fp32, so ties resolve identically
    assert st["band_diffs"] == 0


def test_bitwise_deterministic():
    say("case determinism: C1 twice")
    L = cfg_layer("C1")
    a = gpu_decode(L)
    b = gpu_decode(L)
    assert np.array_equal(a.out, b.out) and np.array_equal(a.idx, b.idx)
    assert np.array_equal(a.lse, b.lse)


def test_c2_llama_layer_128k_full_parity():
    say("case C2: H_q=32 H_kv=8 N=131072 k=2048")
    L = cfg_layer("C2")
    run = gpu_decode(L, with_scores=True)
    assert run.rescanned == 0  # the sample's margin holds on this workload
    st = compare_sequence(L, run, 0)
    say(f"  band differences: {st['band_diffs']}")
    for pos, h in L.needles[0]:
        assert pos in run.idx[0, h]


def test_c4_ragged_batch_of_16():
    c = synth.config("C4")
    say("case C4: B=16 lengths in [32768, 131072], shuffled pages, k=2%")
    L = cfg_layer("C4")
    run = gpu_decode(L, max_seq_len=max(L.seq_lens))
    assert run.rescanned == 0
    for b in range(L.B):
        compare_sequence(L, run, b)
    assert c.B == L.B
