"""ra_decode_step_noalloc (the entry point for callers that cannot
allocate: its workspace is the library's own device array) against
ra_decode_step_ex with a caller workspace, on two calls in a row on the
same GPU, the second with a smaller input (the array keeps the first
call's contents, and no initial contents may be needed); then a size past
the array's maximum is rejected before anything runs."""

import numpy as np
import pytest
import torch

import synth
import top_sparse_attention_gqa_amd as ra
from tests.parity import check_out, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


def run_both(H_q, H_kv, lens, ks, n_sink, window, seed, max_seq_len):
    L = synth.make_layer(H_q, H_kv, lens, ks, n_sink, window, 2, seed, DEV, shuffle_pages=True)
    B, k_max = len(lens), max(ks)
    kv = ra.KVLayer(L.k_pool, L.v_pool, L.block_table)
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    kt = torch.tensor(ks, dtype=torch.int32, device=DEV)
    res = []
    for noalloc in (False, True):
        out = torch.full((B, H_q, 128), float("nan"), device=DEV)
        lse = torch.full((B, H_q), float("nan"), device=DEV)
        idx = torch.full((B, H_q, k_max), -7, dtype=torch.int32, device=DEV)
        if noalloc:
            ra.decode_step_noalloc(L.q, kv, seq, max_seq_len, kt, k_max, n_sink, window, out, lse, idx)
        else:
            ws = ra.alloc_workspace(B, H_q, H_kv, max_seq_len, k_max, device=DEV)
            ra.decode_step_ex(L.q, kv, seq, max_seq_len, kt, k_max, n_sink, window, out, lse, idx, ws)
        torch.cuda.synchronize()
        res.append((out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
                    idx.cpu().numpy()))
    (o_ref, l_ref, i_ref), (o, l, i) = res
    assert np.array_equal(i, i_ref), "retrieved indices differ"
    check_out(o, o_ref)
    check_out(l, l_ref, "lse")
    return o, o_ref


def test_noalloc_matches_the_workspace_call_twice_then_smaller():
    a = dict(H_q=32, H_kv=8, lens=[40000, 30013], ks=[800, 600], n_sink=128, window=512,
             seed=31, max_seq_len=40000)
    size = ra.decode_workspace_bytes(2, 32, 8, 40000, 800)
    say(f"case noalloc call 1: B=2 H_q=32 H_kv=8 lens={a['lens']} ws={size} bytes")
    assert size <= ra._lib.NOALLOC_WS_BYTES
    run_both(**a)
    say("case noalloc call 2: B=1 H_q=4 H_kv=1 N=4096 k=64 (smaller)")
    o, o_ref = run_both(4, 1, [4096], [64], 16, 64, 32, 4096)
    assert np.array_equal(o, o_ref)  # same kernels, same inputs: bit-identical


def test_noalloc_rejects_sizes_past_its_array():
    # one Llama-3-8B layer at 2^20 tokens needs about 388 MiB of workspace
    need = ra.decode_workspace_bytes(1, 32, 8, 1 << 20, 10485)
    say(f"case noalloc too large: needs {need} bytes, the array holds {ra._lib.NOALLOC_WS_BYTES}")
    assert need > ra._lib.NOALLOC_WS_BYTES
    L = synth.make_layer(4, 1, [4096], [64], 16, 64, 2, 33, DEV)
    kv = ra.KVLayer(L.k_pool, L.v_pool, L.block_table)
    q = torch.zeros(1, 32, 128, dtype=torch.bfloat16, device=DEV)
    kv8 = ra.KVLayer(torch.zeros(1, 8, 64, 128, dtype=torch.bfloat16, device=DEV),
                     torch.zeros(1, 8, 64, 128, dtype=torch.bfloat16, device=DEV),
                     torch.zeros(1, 1, dtype=torch.int32, device=DEV))
    seq = torch.ones(1, dtype=torch.int32, device=DEV)
    out = torch.empty(1, 32, 128, device=DEV)
    idx = torch.empty(1, 32, 10485, dtype=torch.int32, device=DEV)
    with pytest.raises(ra.RAError) as e:
        ra.decode_step_noalloc(q, kv8, seq, 1 << 20, seq, 10485, 128, 512, out, None, idx)
    assert e.value.status == ra.RA_ERR_WORKSPACE
    del kv
