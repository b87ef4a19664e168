"""The debug build (libra_debug.so, compiled with -DRA_DEBUG) on the cases
that reach every guarded access: each decode kernel checks its computed
global indices against their buffers and records a failed check in a word
of the workspace instead of making the access. On every case the word must
read 0, and the outputs must equal the release build's bit for bit (the
checks change no arithmetic) and the oracle within the parity tolerances."""

import dataclasses
import os

import numpy as np
import pytest
import torch

import synth
import top_sparse_attention_gqa_amd as ra
from top_sparse_attention_gqa_amd import _lib
from tests.parity import compare_sequence, say

pytestmark = pytest.mark.gpu

DEV = "cuda"
DEBUG_LIB = os.path.join(os.path.dirname(ra.__file__), "libra_debug.so")


@pytest.fixture(scope="module")
def debug_lib():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    assert os.path.exists(DEBUG_LIB), "build libra_debug.so with the package's build.py"
    return _lib.load_build(DEBUG_LIB)


def run(L, lib=None, max_seq_len=None, k_max=None, append=None):
    """One decode step through the given build; returns host outputs and the
    failed-check word."""
    B, H_q = L.q.shape[0], L.q.shape[1]
    max_seq_len = max_seq_len or max(L.seq_lens)
    k_max = max(L.ks) if k_max is None else k_max
    kv = ra.KVLayer(L.k_pool, L.v_pool, L.block_table)
    seq = torch.tensor(L.seq_lens, dtype=torch.int32, device=DEV)
    kt = torch.tensor(L.ks, dtype=torch.int32, device=DEV)
    out = torch.full((B, H_q, 128), float("nan"), device=DEV)
    lse = torch.full((B, H_q), float("nan"), device=DEV)
    idx = torch.full((B, H_q, max(k_max, 1)), -7, dtype=torch.int32, device=DEV)
    ws = ra.alloc_workspace(B, H_q, L.H_kv, max_seq_len, k_max, device=DEV)
    ws.fill_(0xA5)
    ctx = _lib.with_build(lib) if lib is not None else _nullctx()
    with ctx:
        if append is None:
            ra.decode_step_ex(L.q, kv, seq, max_seq_len, kt, k_max, L.n_sink, L.window, out, lse,
                              idx if k_max else None, ws, keep_scores=True)
        else:
            kn, vn, pos = append
            ra.append_decode_step(kn, vn, pos, L.q, kv, seq, max_seq_len, kt, k_max, L.n_sink,
                                  L.window, out, lse, idx if k_max else None, ws)
        off = ra.workspace_rescan_count_offset(B, H_q, L.H_kv, max_seq_len, k_max)
    torch.cuda.synchronize()
    word = int(ws[off + 4:off + 8].view(torch.int32).item())
    rescanned = int(ws[off:off + 4].view(torch.int32).item())
    return (out.cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy()[:, :, :k_max], word,
            rescanned)


class _nullctx:
    def __enter__(self):
        return None

    def __exit__(self, *a):
        return False


def check(L, debug_lib, oracle=True, **kw):
    rel = run(L, **kw)
    dbg = run(L, debug_lib, **kw)
    assert dbg[3] == 0, f"debug build: failed bounds checks, bits {dbg[3]:#x}"
    assert dbg[4] == rel[4]
    for a, b, what in zip(rel[:3], dbg[:3], ("out", "lse", "idx")):
        assert np.array_equal(a.view(np.uint32) if a.dtype != np.int32 else a,
                              b.view(np.uint32) if b.dtype != np.int32 else b), what
    if oracle:
        from tests.parity import Run
        r = Run(dbg[0].astype(np.float64), dbg[1].astype(np.float64), dbg[2], None, dbg[4])
        for b in range(L.B):
            compare_sequence(L, r, b)
    return dbg


def layer(H_q, H_kv, lens, ks, n_sink, window, seed=0, **kw):
    return synth.make_layer(H_q, H_kv, list(lens), list(ks), n_sink, window, 2, seed, DEV, **kw)


def cfg_layer(name):
    c = synth.config(name)
    lens = list(c.seq_lens) if c.seq_lens else synth.draw_lengths(c.B, *c.len_range, c.seed)
    return synth.make_layer(c.H_q, c.H_kv, lens, [c.k_for(n) for n in lens], c.n_sink,
                            c.window, c.needles_per_head, c.seed, DEV,
                            shuffle_pages=c.shuffle_pages)


SMALL = [
    # name, H_q, H_kv, lens, k, n_sink, window
    ("one_token", 4, 1, [1], [3], 16, 64),
    ("ragged_tail", 4, 1, [5000], [64], 16, 64),
    ("three_tiles", 8, 2, [20000], [300], 128, 512),
    ("k_zero", 4, 1, [3000], [0], 16, 64),
    ("k_all_is_dense", 4, 1, [2000], [5000], 16, 64),
    ("gqa8_two_groups", 16, 2, [9000], [70], 16, 64),
    ("ragged_batch", 8, 2, [1, 700, 8192, 8250, 19000], [0, 20, 100, 170, 380], 16, 64),
]


@pytest.mark.parametrize("name,H_q,H_kv,lens,ks,ns,win", SMALL, ids=[c[0] for c in SMALL])
def test_debug_build_small(debug_lib, name, H_q, H_kv, lens, ks, ns, win):
    say(f"case debug {name}: H_q={H_q} H_kv={H_kv} N={lens} k={ks}")
    L = layer(H_q, H_kv, lens, ks, ns, win, shuffle_pages=len(lens) > 1)
    check(L, debug_lib)


def test_debug_build_c1_and_append(debug_lib):
    say("case debug C1, then the fused append + decode step")
    L = cfg_layer("C1")
    check(L, debug_lib)
    # the new token lands at position 4000; the step then attends over 4001
    L2 = dataclasses.replace(layer(4, 1, [4000], [64], 16, 64, reserve_tokens=1),
                             seq_lens=[4001])
    kn, vn = synth.make_new_tokens(1, 1, L2.u, 9, DEV)
    pos = torch.tensor([4000], dtype=torch.int32, device=DEV)
    k0, v0 = L2.k_pool.clone(), L2.v_pool.clone()
    rel = run(L2, append=(kn, vn, pos))
    L2.k_pool.copy_(k0)
    L2.v_pool.copy_(v0)
    dbg = run(L2, debug_lib, append=(kn, vn, pos))
    assert dbg[3] == 0
    assert np.array_equal(rel[2], dbg[2])
    assert np.array_equal(rel[0].view(np.uint32), dbg[0].view(np.uint32))


def test_debug_build_rescan_paths(debug_lib):
    # the sample's threshold misleads two groups (dense rescan), and constant
    # keys overflow the candidate list (row re-read): the rescan's writes
    say("case debug rescan: misled sample in a batch, constant keys N=40000")
    from tests.test_gpu_parity import plant_on_sampled_pages
    L = layer(8, 2, [32768, 24576 + 37], [9000, 6000], 16, 64, seed=3)
    plant_on_sampled_pages(L, 0, 0)
    plant_on_sampled_pages(L, 1, 1)
    assert check(L, debug_lib)[4] > 0
    L = layer(4, 1, [40000], [5000], 16, 64)
    L.k_pool.fill_(-0.25)
    check(L, debug_lib)


SPLIT = [
    # one sequence whose scan splits pages across blocks: many blocks per
    # unit; the LDS staging overflowing with every member of M a candidate
    # name, H_q, H_kv, N, max_seq_len, k
    ("split_many", 32, 8, 5000, 131072, 100),
    ("split_overflow", 4, 1, 4096 * 100 + 100, 4096 * 300, 4096 * 100 + 100 - 80),
]


@pytest.mark.parametrize("name,H_q,H_kv,N,cap,k", SPLIT, ids=[c[0] for c in SPLIT])
def test_debug_build_split_scan(debug_lib, name, H_q, H_kv, N, cap, k):
    say(f"case debug {name}: H_q={H_q} H_kv={H_kv} N={N} max_seq_len={cap} k={k}")
    L = layer(H_q, H_kv, [N], [k], 16, 64, seed=21)
    check(L, debug_lib, max_seq_len=cap)


def test_debug_build_workload_sizes(debug_lib):
    # a 128K-token sequence (its scan splits pages across blocks) and a
    # ragged batch of 16 with shuffled pages, against the release build
    for name in ("C2", "C4"):
        say(f"case debug {name}")
        L = cfg_layer(name)
        check(L, debug_lib, oracle=False)
