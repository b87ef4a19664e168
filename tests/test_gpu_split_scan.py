"""Parity of the scan's page split: with one sequence whose units do not
divide evenly over the persistent scan blocks, the blocks split pages
rather than units, and a unit two (or more) blocks share has its list slots
reserved with global atomics. These cases take that path on purpose:

* many blocks per unit (a short sequence under a large capacity);
* the LDS staging overflowing in split mode, with every member of M a
  candidate (k >= |M|), so the blocks take list slots directly;
* a misleading sample in split mode, so the full rescan follows;
* the fused append + decode step against append then decode, in split mode.

Each checks the geometry first (split on, and the reason), then compares
with the fp64 oracle (or bit for bit with the unfused calls)."""

import numpy as np
import pytest
import torch

import synth
import top_sparse_attention_gqa_amd as ra
from tests.parity import compare_sequence, gpu_decode, say
from tests.test_gpu_parity import plant_on_sampled_pages

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


def split_geometry(H_kv, N, max_seq_len):
    """(split, units, scan blocks) as the library launches the scan for one
    sequence: one block per CU, at most one per unit of capacity."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    units = H_kv * (((N + 63) // 64 + 63) // 64)
    nb = max(1, min(cus, H_kv * ((max_seq_len + 4095) // 4096)))
    return units % nb != 0, units, nb


def test_split_scan_many_blocks_per_unit():
    H_q, H_kv, N, cap = 32, 8, 5000, 131072
    split, T, NB = split_geometry(H_kv, N, cap)
    say(f"case split_many: H_q={H_q} H_kv={H_kv} N={N} max_seq_len={cap} units={T} blocks={NB}")
    assert split and T < NB
    L = synth.make_layer(H_q, H_kv, [N], [100], 16, 64, 2, 21, DEV)
    run = gpu_decode(L, max_seq_len=cap, with_scores=True)
    assert run.rescanned == 0
    compare_sequence(L, run, 0)


def test_split_scan_staging_overflow_every_member_a_candidate():
    H_q, H_kv, N, cap = 4, 1, 4096 * 200 + 100, 4096 * 300
    split, T, NB = split_geometry(H_kv, N, cap)
    ns, win = 16, 64
    M = N - ns - win
    say(f"case split_overflow: N={N} max_seq_len={cap} units={T} blocks={NB} k=|M|={M}")
    # about 50 pages per block: 12800 candidates of 4 heads overflow the
    # 8192-entry staging
    assert split and T * 64 / NB * 64 * H_q > 8192
    L = synth.make_layer(H_q, H_kv, [N], [M], ns, win, 2, 22, DEV)
    run = gpu_decode(L, max_seq_len=cap)
    assert run.rescanned == 0
    compare_sequence(L, run, 0)


def test_split_scan_misleading_sample_takes_the_rescan():
    H_q, H_kv, N, cap = 4, 1, 32768, 131072
    split, T, NB = split_geometry(H_kv, N, cap)
    say(f"case split_misled: N={N} max_seq_len={cap} units={T} blocks={NB} k=9000")
    assert split
    L = synth.make_layer(H_q, H_kv, [N], [9000], 16, 64, 2, 23, DEV)
    plant_on_sampled_pages(L, 0, 0)
    run = gpu_decode(L, max_seq_len=cap, with_scores=True)
    assert run.rescanned > 0
    compare_sequence(L, run, 0)


@pytest.mark.parametrize("H_q,H_kv,N0,cap,k,steps", [
    (8, 2, 5000, 65536, 40, 5),
    # the full-size length just past 2^20 that the 32-layer workload runs at
    (32, 8, (1 << 20) + 1000, (1 << 20) + 1003, 10495, 3),
])
def test_fused_append_equals_append_then_decode_in_split_mode(H_q, H_kv, N0, cap, k, steps):
    split, T, NB = split_geometry(H_kv, N0 + 1, cap)
    say(f"case split_fused: H_q={H_q} H_kv={H_kv} N0={N0} max_seq_len={cap} units={T} "
        f"blocks={NB} k={k} steps={steps}")
    assert split
    ns, win = 128, 512
    needles = 2 if N0 < 100000 else 64
    mk = lambda: synth.make_layer(H_q, H_kv, [N0], [k], ns, win, needles, 24, DEV,
                                  reserve_tokens=steps)
    A = mk()
    F = mk()
    q_s, k_s, v_s = synth.make_decode_stream(1, H_q, H_kv, A.u, steps, 25, DEV)
    kv_a = ra.KVLayer(A.k_pool, A.v_pool, A.block_table)
    kv_f = ra.KVLayer(F.k_pool, F.v_pool, F.block_table)
    kt = torch.tensor([k], dtype=torch.int32, device=DEV)
    ws_a = ra.alloc_workspace(1, H_q, H_kv, cap, k, device=DEV)
    ws_f = ra.alloc_workspace(1, H_q, H_kv, cap, k, device=DEV)
    outs = [[torch.empty(1, H_q, 128, device=DEV), torch.empty(1, H_q, device=DEV),
             torch.empty(1, H_q, k, dtype=torch.int32, device=DEV)] for _ in range(2)]
    for s in range(steps):
        pos = torch.tensor([N0 + s], dtype=torch.int32, device=DEV)
        seq = pos + 1
        ra.kv_append(kv_a, k_s[s], v_s[s], pos)
        ra.decode_step_ex(q_s[s], kv_a, seq, cap, kt, k, ns, win, *outs[0], ws_a)
        ra.append_decode_step(k_s[s], v_s[s], pos, q_s[s], kv_f, seq, cap, kt, k, ns, win,
                              *outs[1], ws_f)
        torch.cuda.synchronize()
        assert torch.equal(outs[0][2], outs[1][2]), f"indices differ at step {s}"
        assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert torch.equal(A.k_pool, F.k_pool) and torch.equal(A.v_pool, F.v_pool)
    # and the last step against the oracle (first and last KV group)
    import dataclasses
    from tests.parity import Run
    run = Run(outs[1][0].cpu().numpy().astype(np.float64),
              outs[1][1].cpu().numpy().astype(np.float64), outs[1][2].cpu().numpy())
    view = dataclasses.replace(F, q=q_s[steps - 1], seq_lens=[N0 + steps], ks=[k])
    G = H_q // H_kv
    for g in (0, H_kv - 1):
        compare_sequence(view, run, 0, heads=list(range(g * G, (g + 1) * G)),
                         check_score_rows=False, appended=(N0, k_s, v_s))
