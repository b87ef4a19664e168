"""Parity of the merge's out_idx copy when one tile holds far more retrieved
positions than the copy blocks read up front. The copy blocks load each of
their tiles' first positions together with the tile counts, sized from the
tile's mean share of k_max; a tile holding more takes a second round for
the rest, beside tiles of the same block that do not. Here the keys of one
tile are turned towards their group's queries, so a large share of every
head's top-k falls in it, and the positions must still come out complete
and in ascending order (compared with the fp64 oracle)."""

import pytest
import torch

import synth
from tests.parity import compare_sequence, gpu_decode, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


def turn_tile_towards_queries(L, b, g, t0, t1, boost=4.0):
    """Keys of positions [t0, t1) of group (b, g) plus boost times the unit
    direction of the group's summed queries."""
    G = L.H_q // L.H_kv
    qdir = L.q[b, g * G:(g + 1) * G].float().sum(0)
    qdir = qdir / qdir.norm()
    for j in range(t0 // 64, t1 // 64):
        pg = int(L.block_table[b, j])
        L.k_pool[pg, g] = (L.k_pool[pg, g].float() + boost * qdir).to(torch.bfloat16)


# span: the gather's tile at this size; up_front: the positions per tile a
# copy block reads with the counts (the power of two at or above 1.5 times
# a tile's mean share of k)
@pytest.mark.parametrize("H_q,H_kv,N,k,tile,span,up_front", [
    (8, 2, 65536, 1000, 3, 4096, 128),       # one-unit tiles, 16 per head
    (32, 8, 1 << 20, 12000, 37, 8192, 256),  # two-unit tiles, 128 per head
])
def test_one_tile_holds_most_of_the_top_k(H_q, H_kv, N, k, tile, span, up_front):
    say(f"case merge_copy: H_q={H_q} H_kv={H_kv} N={N} k={k}, tile {tile} turned to the queries")
    L = synth.make_layer(H_q, H_kv, [N], [k], 16, 64, 2, 91, DEV)
    for g in range(H_kv):
        turn_tile_towards_queries(L, 0, g, tile * span, (tile + 1) * span)
    run = gpu_decode(L)
    assert run.rescanned == 0
    # every head's turned tile holds far more positions than are read up front
    inside = ((run.idx[0] >= tile * span) & (run.idx[0] < (tile + 1) * span)).sum(axis=1)
    say(f"  positions in the turned tile per head: {inside.tolist()}")
    assert inside.min() > 2 * up_front
    compare_sequence(L, run, 0, check_score_rows=False)
