"""The decode step captured in a HIP graph (torch.cuda.CUDAGraph over the
calls' stream): the library launches only kernels on the caller's stream,
allocates nothing, never synchronises and records no memset, so the step is
capturable. Each test captures once, then replays several times with new
queries written into the captured input in place, with eager library calls
and synchronisations between the replays, and requires every replay to
equal the same step run eagerly, bit for bit."""

import pytest
import torch

import synth
import top_sparse_attention_gqa_amd as ra
from tests.parity import say

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


def buffers(B, H_q, k_max):
    out = torch.empty(B, H_q, 128, device=DEV)
    lse = torch.empty(B, H_q, device=DEV)
    idx = torch.empty(B, H_q, max(k_max, 1), dtype=torch.int32, device=DEV)
    return out, lse, idx


def same(a, b):
    return all(torch.equal(x.view(torch.int32) if x.dtype == torch.float32 else x,
                           y.view(torch.int32) if y.dtype == torch.float32 else y)
               for x, y in zip(a, b))


CASES = [
    # name, H_q, H_kv, lens, ks, n_sink, window, shuffle
    ("c1_shape", 4, 1, [4096], [64], 16, 64, False),
    ("ragged_batch", 8, 2, [1, 700, 8192, 8250, 19000], [0, 20, 100, 170, 380], 16, 64, True),
]


@pytest.mark.parametrize("name,H_q,H_kv,lens,ks,ns,win,shuffle", CASES, ids=[c[0] for c in CASES])
def test_captured_step_replays_equal_the_eager_step(name, H_q, H_kv, lens, ks, ns, win, shuffle):
    say(f"case graph {name}: H_q={H_q} H_kv={H_kv} N={lens} k={ks}")
    L = synth.make_layer(H_q, H_kv, lens, ks, ns, win, 2, 41, DEV, shuffle_pages=shuffle)
    B, k_max, cap = len(lens), max(ks), max(lens)
    kv = ra.KVLayer(L.k_pool, L.v_pool, L.block_table)
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    kt = torch.tensor(ks, dtype=torch.int32, device=DEV)
    q_static = L.q.clone()
    g_out = buffers(B, H_q, k_max)
    ws_g = ra.alloc_workspace(B, H_q, H_kv, cap, k_max, device=DEV)
    e_out = buffers(B, H_q, k_max)
    ws_e = ra.alloc_workspace(B, H_q, H_kv, cap, k_max, device=DEV)

    def step(q, o, ws):
        ra.decode_step_ex(q, kv, seq, cap, kt, k_max, ns, win, o[0], o[1],
                          o[2] if k_max else None, ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(q_static, g_out, ws_g)  # warm up on the capture's stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(q_static, g_out, ws_g)
    torch.cuda.synchronize()

    queries = [L.q] + [synth.make_prefill_queries(B, H_q, L.u, 500 + r, DEV) for r in range(3)]
    for r, q in enumerate(queries):
        q_static.copy_(q)
        graph.replay()
        torch.cuda.synchronize()
        step(q, e_out, ws_e)  # eager work between the replays
        torch.cuda.synchronize()
        assert same(g_out, e_out), f"replay {r} differs from the eager step"
    assert torch.isfinite(e_out[0]).all()


def test_captured_noalloc_step_replays():
    # the entry point for callers that cannot allocate, its device array set
    # up by an eager first call, then captured and replayed
    say("case graph noalloc: C1 shape")
    L = synth.make_layer(4, 1, [4096], [64], 16, 64, 2, 42, DEV)
    kv = ra.KVLayer(L.k_pool, L.v_pool, L.block_table)
    seq = torch.tensor([4096], dtype=torch.int32, device=DEV)
    kt = torch.tensor([64], dtype=torch.int32, device=DEV)
    q_static = L.q.clone()
    g_out = buffers(1, 4, 64)
    e_out = buffers(1, 4, 64)
    ws_e = ra.alloc_workspace(1, 4, 1, 4096, 64, device=DEV)

    def noalloc(q, o):
        ra.decode_step_noalloc(q, kv, seq, 4096, kt, 64, 16, 64, o[0], o[1], o[2])

    noalloc(q_static, g_out)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        noalloc(q_static, g_out)
    torch.cuda.synchronize()
    for r in range(3):
        q = synth.make_prefill_queries(1, 4, L.u, 600 + r, DEV)
        q_static.copy_(q)
        graph.replay()
        torch.cuda.synchronize()
        ra.decode_step_ex(q, kv, seq, 4096, kt, 64, 16, 64, e_out[0], e_out[1], e_out[2], ws_e)
        torch.cuda.synchronize()
        assert same(g_out, e_out), f"replay {r} differs from the eager step"
