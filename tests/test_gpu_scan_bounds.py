"""The candidate bounds computed inside the scan. When one call runs the
threshold stage and the scan, and the batch has at most one head per scan
block, the scan's blocks compute the heads' bounds themselves (a block
holds its first pages' keys in LDS until its group's bounds are out) and
the threshold launch is left out. Each case runs the step three ways on the
same inputs:

* one call (the library's choice);
* sample and threshold, then scan to merge: the threshold launch computes
  the bounds and the scan finds them published;
* sample alone, then scan to merge: the scan computes every bound, however
  many heads each block has to take;

and requires the outputs to be equal bit for bit, and the one-call step to
match the fp64 oracle. The cases cover G = 1, 2, 4, 8 (with G = 8 a block
holds 32 of a unit's 64 pages, so the unit's other half is scored after the
bounds are known), ragged batches, the scan's page split, one head per
block, batches with four and eight heads per block, and a sample too large
for one block's registers; a last case puts one sampled key far above the
rest of the sample (about 200 times the bulk's scores)."""

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


def scan_blocks(cap_units):
    """The scan's grid: one block per CU, at most one per unit of capacity."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return max(1, min(cus, cap_units))


def two_call_step(L, max_seq_len, first_end):
    """stages 0 .. first_end, then scan .. merge (first_end = threshold: the
    threshold launch computes the bounds; = sample: the scan does)."""
    B, H_q = L.q.shape[0], L.q.shape[1]
    k_max = max(L.ks)
    kv = ra.KVLayer(L.k_pool, L.v_pool, L.block_table)
    seq = torch.tensor(L.seq_lens, dtype=torch.int32, device=DEV)
    kt = torch.tensor(L.ks, dtype=torch.int32, device=DEV)
    out = torch.full((B, H_q, 128), float("nan"), device=DEV)
    lse = torch.full((B, H_q), float("nan"), device=DEV)
    idx = torch.full((B, H_q, max(k_max, 1)), -7, dtype=torch.int32, device=DEV)
    ws = ra.alloc_workspace(B, H_q, L.H_kv, max_seq_len, k_max, device=DEV)
    ws.fill_(0xA5)
    a = (L.q, kv, seq, max_seq_len, kt, k_max, L.n_sink, L.window, out, lse,
         idx if k_max else None, ws)
    ra.decode_stages(*a, ra.STAGE_SAMPLE, first_end)
    ra.decode_stages(*a, ra.STAGE_SCAN, ra.STAGE_MERGE)
    torch.cuda.synchronize()
    return (out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
            idx.cpu().numpy()[:, :, :k_max])


CASES = [
    # name, H_q, H_kv, lens, ks, n_sink, window, max_seq_len, shuffle
    ("c1_shape", 4, 1, [4096], [64], 16, 64, None, False),
    ("ragged_batch", 8, 2, [1, 700, 8192, 8250, 19000], [0, 20, 100, 170, 380], 16, 64, None, True),
    ("g8_half_unit_held", 8, 1, [3 * 4096 + 100], [300], 16, 64, None, False),
    ("g1", 2, 2, [20000], [150], 4, 32, None, False),
    ("g2", 4, 2, [9000, 12000], [100, 90], 4, 32, None, True),
    ("split_many_blocks", 32, 8, [5000], [100], 16, 64, 131072, False),
    ("one_bound_per_block", 4, 1, [4096] * 40, [50] * 40, 16, 64, 16384, False),
    ("four_bounds_per_block", 4, 1, [4096] * 40, [50] * 40, 16, 64, None, False),
    ("eight_bounds_per_block", 8, 1, [4096] * 41, [50] * 41, 16, 64, None, False),
    # a sample past the registers (18,752 keys per head): one call launches
    # the threshold stage, the scan alone streams the keys for its bound
    ("streamed_sample", 4, 1, [1_200_000], [12000], 128, 512, None, False),
]


@pytest.mark.parametrize("name,H_q,H_kv,lens,ks,ns,win,cap,shuffle", CASES, ids=[c[0] for c in CASES])
def test_bounds_in_the_scan_equal_the_threshold_launch(name, H_q, H_kv, lens, ks, ns, win, cap,
                                                       shuffle):
    cap = cap or max(lens)
    units_cap = len(lens) * H_kv * ((cap + 4095) // 4096)
    nb = scan_blocks(units_cap)
    heads = len(lens) * H_q
    say(f"case scan_bounds {name}: B={len(lens)} H_q={H_q} H_kv={H_kv} N={lens[:4]} "
        f"cap={cap} scan blocks={nb} heads per block={heads / nb:.2f}")
    L = synth.make_layer(H_q, H_kv, lens, ks, ns, win, 2, 77, DEV, shuffle_pages=shuffle)
    one = gpu_decode(L, max_seq_len=cap)
    for first_end in (ra.STAGE_THRESHOLD, ra.STAGE_SAMPLE):
        out2, lse2, idx2 = two_call_step(L, cap, first_end)
        assert np.array_equal(one.out, out2, equal_nan=True), first_end
        assert np.array_equal(one.lse, lse2, equal_nan=True), first_end
        assert np.array_equal(one.idx, idx2), first_end
    assert one.rescanned == 0
    for b in sorted({0, len(lens) // 2, len(lens) - 1}):
        compare_sequence(L, one, b)


def test_one_sampled_key_far_above_the_rest():
    # one key on a sampled page scores about 200 times the bulk: the bound
    # (the R-th largest sampled key's top bits) must not depend on how far
    # the largest sampled key is from it
    say("case scan_bounds far_top: N=32768 k=3000, one huge key on a sampled page")
    L = synth.make_layer(4, 1, [32768], [3000], 16, 64, 2, 78, DEV)
    P = 32768 // 64
    s = 0
    while s < 6 and (P >> (s + 1)) >= 16:
        s += 1
    j = (1 << s) // 2  # the first sampled page
    qdir = L.q[0, 0:4].float().sum(0)
    qdir = qdir / qdir.norm()
    pg = int(L.block_table[0, j])
    L.k_pool[pg, 0, 5] = (200.0 * qdir).to(torch.bfloat16)
    one = gpu_decode(L)
    for first_end in (ra.STAGE_THRESHOLD, ra.STAGE_SAMPLE):
        out2, lse2, idx2 = two_call_step(L, 32768, first_end)
        assert np.array_equal(one.out, out2, equal_nan=True), first_end
        assert np.array_equal(one.idx, idx2), first_end
    assert one.rescanned == 0
    compare_sequence(L, one, 0)
    assert (j * 64 + 5) in one.idx[0, 0]
