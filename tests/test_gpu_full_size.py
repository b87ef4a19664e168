"""Parity at the workloads' full sizes, in the launch configuration that
bench.py times.

* One Llama-3-8B layer (H_q=32, H_kv=8) at N = 1,048,576 with k = 1, 2 and
  3 % of N: the whole step runs on the GPU; the oracle checks all eight KV
  groups (all 32 query heads) element by element, and every planted needle
  of every head must be retrieved.
* The 32-layer workload: layers 0, 15 and 31 (seeds 0, 15, 31) run the same
  1002 token steps as the benchmark (2 warm-up steps, then 1000), each one
  call of ra_append_decode_step (the new token's rows written inside the
  step, as the benchmark times it), with the same capacity; the oracle
  checks all 32 heads of each of them after the first, a middle and the
  last step.

Layers are independent, so the sampled layers see exactly what they see in
the 32-layer run.
"""

import dataclasses

import numpy as np
import pytest
import torch

import synth
import top_sparse_attention_gqa_amd as ra
from tests.parity import Run, compare_sequence, gpu_decode, say

pytestmark = pytest.mark.gpu

DEV = "cuda"
ALL_GROUPS = [list(range(4 * g, 4 * g + 4)) for g in range(8)]


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


@pytest.mark.parametrize("name", ["C3_1", "C3_2", "C3_3"])
def test_one_layer_at_a_million_tokens(name):
    c = synth.config(name)
    n = c.seq_lens[0]
    say(f"case {name}: H_q=32 H_kv=8 N={n} k={c.k_for(n)} (all 32 heads checked)")
    L = synth.make_layer(c.H_q, c.H_kv, [n], [c.k_for(n)], c.n_sink, c.window,
                         c.needles_per_head, c.seed, DEV)
    run = gpu_decode(L, with_scores=True)
    assert run.rescanned == 0  # the sample's margin holds on this workload
    for heads in ALL_GROUPS:
        st = compare_sequence(L, run, 0, heads=heads)
        say(f"  heads {heads[0]}..{heads[-1]}: band differences {st['band_diffs']}")
    missed = [(pos, h) for pos, h in L.needles[0] if pos not in run.idx[0, h]]
    assert not missed, f"{len(missed)} needles not retrieved, e.g. {missed[:4]}"


def test_32_layer_workload_sampled_layers_over_1000_steps():
    c = synth.config("C5")
    N0 = c.seq_lens[0]
    warmup, steps = 2, c.extra["steps"]
    total = warmup + steps
    checks = {0, warmup + steps // 2, total - 1}
    sampled = (0, 15, 31)
    say(f"case C5: layers {sampled} of 32, N0={N0}, {total} append+decode steps, "
        f"checks after steps {sorted(checks)}")
    H_q, H_kv = c.H_q, c.H_kv
    layers = {l: synth.make_layer(H_q, H_kv, [N0], [c.k_for(N0)], c.n_sink, c.window,
                                  c.needles_per_head, c.seed + l, DEV, reserve_tokens=total)
              for l in sampled}
    streams = {l: synth.make_decode_stream(1, H_q, H_kv, layers[l].u, total, 10_000 + l, DEV)
               for l in sampled}
    lens = [N0 + s + 1 for s in range(total)]
    ks = [c.k_for(n) for n in lens]
    seq_all = torch.tensor(lens, dtype=torch.int32, device=DEV).view(total, 1)
    pos_all = (seq_all - 1).contiguous()
    k_all = torch.tensor(ks, dtype=torch.int32, device=DEV).view(total, 1)
    max_seq_len = N0 + total
    k_max = max(ks)
    ws = ra.alloc_workspace(1, H_q, H_kv, max_seq_len, k_max, device=DEV)
    out = torch.empty(1, H_q, 128, device=DEV)
    lse = torch.empty(1, H_q, device=DEV)
    idx = torch.empty(1, H_q, k_max, dtype=torch.int32, device=DEV)
    kvs = {l: ra.KVLayer(layers[l].k_pool, layers[l].v_pool, layers[l].block_table)
           for l in sampled}
    for s in range(total):
        for l in sampled:
            q, kn, vn = streams[l][0][s], streams[l][1][s], streams[l][2][s]
            ra.append_decode_step(kn, vn, pos_all[s], q, kvs[l], seq_all[s], max_seq_len,
                                  k_all[s], k_max, c.n_sink, c.window, out, lse, idx, ws)
            if s in checks:
                torch.cuda.synchronize()
                run = Run(out.cpu().numpy().astype(np.float64),
                          lse.cpu().numpy().astype(np.float64),
                          idx.cpu().numpy())
                view = dataclasses.replace(layers[l], q=q, seq_lens=[lens[s]], ks=[ks[s]])
                for heads in ALL_GROUPS:
                    # the appended rows come from the stream, not the pool
                    st = compare_sequence(view, run, 0, heads=heads, check_score_rows=False,
                                          appended=(N0, streams[l][1], streams[l][2]))
                    say(f"  step {s} layer {l} heads {heads[0]}..{heads[-1]}: "
                        f"band differences {st['band_diffs']}")


@pytest.mark.parametrize("N", [1 << 24, (1 << 24) - 37])
def test_longest_sequence_the_library_accepts(N):
    # RA_MAX_SEQ_LEN positions (and a ragged length just below it): 4096
    # units per KV head, positions at the top of the 24-bit row fields.
    # The oracle checks every head; its fp32 error floor is formed tile by
    # tile (an fp64 copy of all 2^24 keys would be 16 GB).
    import oracle
    from tests.parity import U32, check_indices, check_out

    H_q, H_kv, k, ns, win = 4, 1, 2000, 16, 64
    say(f"case longest: H_q={H_q} H_kv={H_kv} N={N} k={k}")
    L = synth.make_layer(H_q, H_kv, [N], [k], ns, win, 2, 77, DEV)
    run = gpu_decode(L, max_seq_len=1 << 24)
    assert run.rescanned == 0
    q = synth.bf16_bits(L.q[0])
    K = synth.depage(L.k_pool, L.block_table, 0, N)
    V = synth.depage(L.v_pool, L.block_table, 0, N)
    res = oracle.decode(q, K, V, k=k, n_sink=ns, window=win)
    qa = np.abs(oracle.as_f64(q))
    top = np.zeros(H_q)
    for t0 in range(0, N, 1 << 20):
        Ka = np.abs(oracle.as_f64(K[t0:t0 + (1 << 20), 0, :]))
        top = np.maximum(top, (qa @ Ka.T).max(axis=1))
    eps = 130 * U32 / (1 - 130 * U32) * top / np.sqrt(128.0)
    band = 0
    for h in range(H_q):
        band += check_indices(run.idx[0, h], res, h, k, eps[h])
        check_out(run.out[0, h], res["out"][h], f"out[h={h}]")
        check_out(np.array([run.lse[0, h]]), np.array([res["lse"][h]]), f"lse[h={h}]")
    for pos, h in L.needles[0]:
        assert pos in run.idx[0, h]
    say(f"  band differences: {band}")
