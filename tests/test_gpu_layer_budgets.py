"""GPU parity of per-layer budgets from ra_layer_budgets (the slides' frame
"Extra experiments show where budget matters": a PyramidKV-style layer
budget): the layers of a small model each run their decode step with their
own k_l, and every layer matches the fp64 oracle's decode with that k_l at
the tolerances of the decode tests (indices outside the tie band, out and
lse elementwise)."""

import numpy as np
import pytest
import torch

import oracle
import synth
import top_sparse_attention_gqa_amd as ra
from tests.parity import compare_sequence, gpu_decode, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


@pytest.mark.parametrize("n_layers,H_q,H_kv,N,k_mean,slope", [
    (4, 8, 2, 5000, 60, 600),     # budgets 96, 72, 48, 24
    (6, 4, 1, 4096 + 17, 40, 1000),  # steepest: the last layer retrieves nothing
])
def test_layer_budget_schedule_parity(n_layers, H_q, H_kv, N, k_mean, slope):
    ks = ra.layer_budgets(n_layers, k_mean, slope)
    assert ks == oracle.layer_budgets(n_layers, k_mean, slope)
    say(f"case layer budgets: {n_layers} layers, N={N}, k_l={ks}")
    for l, k in enumerate(ks):
        L = synth.make_layer(H_q, H_kv, [N], [max(k, 1)], 16, 64, 2, 100 + l, DEV)
        run = gpu_decode(L, ks=[k], k_max=max(ks))
        st = compare_sequence(L, run, 0, ks=[k])
        # each head retrieved exactly k_l positions, padded with -1 after them
        got = run.idx[0]
        assert ((got >= 0).sum(axis=1) == k).all()
        assert (got[:, k:] == -1).all()
        assert st["band_diffs"] <= 2 * H_q
