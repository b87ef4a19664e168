"""GPU parity of the two-tier decode pieces (slides, frames "The GPU keeps
640 fixed positions" and "Two local softmax outputs need global weights"):
attention over listed positions from GPU pools and from pinned host pools
read over the host link (ra_sparse_attend), the LSE merge of two partials
(ra_merge_partials), and a whole step whose keys and values live in host
memory: the key graph retrieves Omega reading host-resident keys, Omega is
attended from host memory, W from an HBM pool holding only its pages, and
the two partials are merged. Outputs are compared with the fp64 oracle at
the decode tests' tolerance (2e-3 absolute + 1e-2 relative)."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
import top_sparse_attention_gqa_amd as ra
from tests.parity import check_out, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


def host_kv(L):
    """The layer's pools copied to pinned host memory (block table on the GPU)."""
    kp = L.k_pool.cpu().pin_memory()
    vp = L.v_pool.cpu().pin_memory()
    return ra.KVLayer(kp, vp, L.block_table), (kp, vp)


def oracle_attend(L, b, N, q_bits, sets):
    """(out, lse) per head over the given position sets, by the oracle."""
    H_q = q_bits.shape[0]
    G = H_q // L.H_kv
    K = synth.depage(L.k_pool, L.block_table, b, N)
    V = synth.depage(L.v_pool, L.block_table, b, N)
    z = oracle.scores(q_bits, K)
    res = []
    for h in range(H_q):
        res.append(oracle.attend(z[h], V[:, h // G, :], sets[h]))
    return res, z, V


def run_sparse(L, kv, N, q, sets, k):
    H_q = q.shape[0]
    idx = np.full((H_q, k), -1, dtype=np.int32)
    for h, S in enumerate(sets):
        idx[h, :len(S)] = S
    idx_t = torch.tensor(idx, device=DEV)
    out = torch.full((H_q, 128), float("nan"), device=DEV)
    lse = torch.full((H_q,), float("nan"), device=DEV)
    ra.sparse_attend(q, kv, 0, N, idx_t, out, lse)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("where", ["gpu", "host"])
def test_sparse_attend_parity(where):
    N = 6000 + 11
    say(f"case sparse attend from {where} pools: H_q=8 H_kv=2 N={N}")
    L = synth.make_layer(8, 2, [N], [8], 0, 0, 2, 31, DEV, shuffle_pages=True)
    r = np.random.default_rng(32)
    sizes = [1, 7, 100, 640, 2000, 4096, 0, 33]
    sets = [np.sort(r.choice(N, s, replace=False)) for s in sizes]
    kv = ra.KVLayer(L.k_pool, L.v_pool, L.block_table) if where == "gpu" else host_kv(L)[0]
    out, lse = run_sparse(L, kv, N, L.q[0], sets, 4096)
    want, _, _ = oracle_attend(L, 0, N, synth.bf16_bits(L.q[0]), sets)
    for h in range(8):
        if sizes[h] == 0:
            assert (out[h] == 0).all() and lse[h] == -math.inf
            continue
        check_out(out[h], want[h][0], f"out[h={h}]")
        check_out(np.array([lse[h]]), np.array([want[h][1]]), f"lse[h={h}]")


def test_merge_partials_parity():
    H = 6
    r = np.random.default_rng(33)
    oa, ob = r.standard_normal((H, 128)), r.standard_normal((H, 128))
    la = np.array([0.5, -3.0, 40.0, -math.inf, 2.0, -math.inf])
    lb = np.array([1.5, 20.0, -10.0, 1.0, -math.inf, -math.inf])
    t = lambda a: torch.tensor(a, dtype=torch.float32, device=DEV).contiguous()
    out, lse = torch.empty(H, 128, device=DEV), torch.empty(H, device=DEV)
    ra.merge_partials(t(oa), t(la), t(ob), t(lb), out, lse)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    f32 = lambda x: np.float64(np.float32(x))
    for h in range(H):
        parts = []
        for o, l in ((oa[h], la[h]), (ob[h], lb[h])):
            o32 = np.asarray(o, dtype=np.float32).astype(np.float64)
            parts.append((f32(l), 1.0, o32) if l != -math.inf else (-math.inf, 0.0, o32))
        wo, wl = oracle.merge(parts)
        if wl == -math.inf:
            assert (out[h] == 0).all() and lse[h] == -math.inf
        else:
            check_out(out[h], wo, f"merged out[h={h}]")
            check_out(np.array([lse[h]]), np.array([wl]), f"merged lse[h={h}]")


def test_two_tier_step_with_the_key_graph():
    # keys and values of M in pinned host memory, W's pages in HBM; the key
    # graph retrieves Omega reading host-resident keys
    N, H_q, H_kv, ns, win, k, ef, D = 8192 + 40, 8, 2, 64, 128, 64, 128, 24
    say(f"case two-tier step: N={N} W={ns}+{win} k={k}")
    L = synth.make_layer(H_q, H_kv, [N], [k], ns, win, 2, 34, DEV)
    kv_host, keep = host_kv(L)
    W = np.r_[0:ns, N - win:N].astype(np.int32)
    kd, td = synth.copy_pages(L.k_pool, L.block_table, 0, W, DEV)
    vd, _ = synth.copy_pages(L.v_pool, L.block_table, 0, W, DEV)
    kv_w = ra.KVLayer(kd, vd, td)
    # a graph per head from random links among the positions of M
    r = np.random.default_rng(35)
    M = np.arange(ns, N - win)
    links = []
    for _ in range(H_q):
        lists = np.stack([r.choice(M, 12, replace=False) for _ in range(900)]).astype(np.int32)
        links.append((lists[:, 0].copy(), lists))
    graphs = [ra.graph_build(hb, ls, N, D) for hb, ls in links]
    nbr = torch.tensor(np.stack([g[0] for g in graphs]), dtype=torch.int32, device=DEV)
    entry = torch.tensor([g[1] for g in graphs], dtype=torch.int32, device=DEV)
    q = L.q[0]
    omega = torch.empty(H_q, k, dtype=torch.int32, device=DEV)
    vis = torch.empty(H_q, dtype=torch.int32, device=DEV)
    ra.graph_search(q, kv_host, 0, N, nbr, entry, ef, k, omega, vis)
    o_om, l_om = torch.empty(H_q, 128, device=DEV), torch.empty(H_q, device=DEV)
    ra.sparse_attend(q, kv_host, 0, N, omega, o_om, l_om)
    widx = torch.tensor(np.tile(W, (H_q, 1)), device=DEV)
    o_w, l_w = torch.empty(H_q, 128, device=DEV), torch.empty(H_q, device=DEV)
    ra.sparse_attend(q, kv_w, 0, N, widx, o_w, l_w)
    out, lse = torch.empty(H_q, 128, device=DEV), torch.empty(H_q, device=DEV)
    ra.merge_partials(o_w, l_w, o_om, l_om, out, lse)
    torch.cuda.synchronize()
    got_om = omega.cpu().numpy()
    out, lse = out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    qb = synth.bf16_bits(q)
    G = H_q // H_kv
    K = synth.depage(L.k_pool, L.block_table, 0, N)
    V = synth.depage(L.v_pool, L.block_table, 0, N)
    z = oracle.scores(qb, K)
    for h in range(H_q):
        nb_o, en_o = oracle.graph_build(*links[h], N, D)
        om, _ = oracle.graph_search(qb[h], K[:, h // G, :], nb_o, en_o, ef, k, batch=ra.GRAPH_BATCH)
        assert np.array_equal(got_om[h][:om.size], om)
        wo, wl = oracle.merge([oracle.partial(z[h], V[:, h // G, :], W),
                               oracle.partial(z[h], V[:, h // G, :], om)])
        check_out(out[h], wo, f"two-tier out[h={h}]")
        check_out(np.array([lse[h]]), np.array([wl]), f"two-tier lse[h={h}]")
    del keep
