"""Parity of the scan's deferred candidate bursts: a block that owns several
units of one (sequence, KV head) keeps their candidates staged in LDS and
writes them in one burst, with an LDS slot counter per (head, staged unit).
These cases make the staging overflow inside a deferred run, so entries of
one unit go both to the burst and straight to its list:

* a batch of two sequences (no page split) with more units than scan
  blocks, so some blocks own two units of one sequence;
* the sampled pages of every group turned away from its queries, so the
  sampled bound sits far below the k-th score and almost every member of M
  is a candidate, while the deferral is sized for k = 1 % of N.

Each checks the geometry first, then compares with the fp64 oracle."""

import pytest
import torch

import synth
from tests.parity import compare_sequence, gpu_decode, say
from tests.test_gpu_parity import plant_on_sampled_pages

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


def unit_geometry(B, H_kv, lens, max_seq_len):
    """(units, scan blocks) as the library launches the scan: one block per
    CU, at most one per unit of capacity; a batch never splits pages."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    units = sum(H_kv * (((n + 63) // 64 + 63) // 64) for n in lens)
    nb = max(1, min(cus, B * H_kv * ((max_seq_len + 4095) // 4096)))
    return units, nb


@pytest.mark.parametrize("H_q,seed", [(4, 41), (8, 42)])
def test_deferred_bursts_with_staging_overflow(H_q, seed):
    H_kv, lens = 1, [4096 * 150, 4096 * 150 - 777]
    ks = [n // 100 for n in lens]
    T, NB = unit_geometry(2, H_kv, lens, max(lens))
    say(f"case deferred_overflow: B=2 H_q={H_q} H_kv={H_kv} N={lens} k={ks} units={T} blocks={NB}")
    # some blocks own two units of one sequence; a unit holds up to
    # 4096 * G candidates, past the 8192-entry staging
    assert NB < T < 2 * NB and 4096 * H_q > 8192 // 2
    L = synth.make_layer(H_q, H_kv, lens, ks, 128, 512, 4, seed, DEV)
    for b in range(2):
        plant_on_sampled_pages(L, b, 0, boost=-3.0)
    run = gpu_decode(L, with_scores=True)
    assert run.rescanned == 0  # a low bound leaves more candidates, not fewer
    for b in range(2):
        compare_sequence(L, run, b)
