"""Host-side check of the score scan's lane mapping, simulated in numpy
(no GPU, no oracle): a wave reads 4 keys per 1 KiB load, 16 lanes x 8 dims
each; lane r of a row keeps query slot s for head s ^ F(r); a reduce-scatter
over partners r ^ 15, r ^ 7, r ^ 3, r ^ 1 (DPP row_mirror, row_half_mirror,
quad_perm [3,2,1,0], quad_perm [1,0,3,2]) leaves lane r with the full dot
product of head F(r); the D = 16 / G lanes sharing F(r) take turns keeping
loads, so after 16 loads every (key, head) of the page sits in exactly one
(lane, slot) at key 4 (s D + (r mod D)) + row."""

import numpy as np
import pytest

MASKS = (15, 7, 3, 1)


def head_of_lane(G, r):
    # the same formula as the kernel's head_of_lane<G>
    b1, b2, b3 = (r >> 1) & 1, (r >> 2) & 1, (r >> 3) & 1
    if G == 1:
        return 0
    if G == 2:
        return b3
    if G == 4:
        return b2 ^ (b3 * 3)
    return b1 ^ (b2 * 3) ^ (b3 * 6)


def simulate(G, seed=0):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((64, 128))       # one page of keys
    q = rng.standard_normal((G, 128))
    D = 16 // G
    kept = {}
    for i in range(16):                      # the 16 loads of a page
        # v[lane][s]: partial over the lane's 8 dims for head s ^ F(r)
        v = np.zeros((64, G))
        for lane in range(64):
            row, r = lane // 16, lane % 16
            tok = 4 * i + row
            for s in range(G):
                h = s ^ head_of_lane(G, r)
                v[lane, s] = K[tok, r * 8:r * 8 + 8] @ q[h, r * 8:r * 8 + 8]
        c = G
        for m in MASKS:
            nv = v.copy()
            for lane in range(64):
                p = (lane // 16) * 16 + ((lane % 16) ^ m)
                if c > 1:
                    for j in range(c // 2):
                        nv[lane, j] = v[lane, j] + v[p, c // 2 + j]
                else:
                    nv[lane, 0] = v[lane, 0] + v[p, 0]
            v = nv
            c = max(c // 2, 1)
        for lane in range(64):
            row, r = lane // 16, lane % 16
            h = head_of_lane(G, r)
            np.testing.assert_allclose(v[lane, 0], K[4 * i + row] @ q[h], rtol=1e-12)
            if i % D == (r & (D - 1)):
                kept[(lane, i // D)] = (4 * i + row, h, v[lane, 0])
    return K, q, kept


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_reduce_scatter_and_keep_cover_every_key_and_head_once(G):
    K, q, kept = simulate(G)
    D = 16 // G
    pairs = set()
    for (lane, s), (tok, h, val) in kept.items():
        row, r = lane // 16, lane % 16
        assert tok == 4 * (s * D + (r & (D - 1))) + row   # the kernel's store index
        np.testing.assert_allclose(val, K[tok] @ q[h], rtol=1e-12)
        pairs.add((tok, h))
    assert len(kept) == 64 * G and pairs == {(t, h) for t in range(64) for h in range(G)}


@pytest.mark.parametrize("G", [2, 4, 8])
def test_head_map_is_linear_with_the_required_step_values(G):
    F = [head_of_lane(G, r) for r in range(16)]
    for a in range(16):
        for b in range(16):
            assert F[a ^ b] == F[a] ^ F[b]
    want = {15: G // 2, 7: G // 4, 3: G // 8, 1: G // 16}
    for m, v in want.items():
        assert F[m] == v
    assert sorted(set(F)) == list(range(G))
