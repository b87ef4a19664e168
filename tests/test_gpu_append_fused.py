"""GPU check of ra_append_decode_step (the append written inside the decode
step) against ra_kv_append followed by ra_decode_step on identical copies of
the same layer, over several appended tokens: the retrieved indices, out
and lse must be bit-identical, and so must the pools afterwards (the fused
call writes the same rows). The new token is in the recent window, and,
with window = 0, inside M where the sampled bound may have read its slot
before it was written (that only bounds the candidates)."""

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


@pytest.mark.parametrize("lens,window,k,steps", [
    ([5000], 64, 40, 6),
    ([3000, 9000 + 13, 700], 0, 25, 5),
])
def test_fused_append_equals_append_then_decode(lens, window, k, steps):
    say(f"case fused append: lens={lens} window={window} k={k} steps={steps}")
    H_q, H_kv, ns = 8, 2, 16
    B = len(lens)
    mk = lambda: synth.make_layer(H_q, H_kv, lens, [k] * B, ns, window, 2, 41, DEV,
                                  reserve_tokens=steps, shuffle_pages=True)
    A, F = mk(), mk()                      # two identical copies
    q_s, k_s, v_s = synth.make_decode_stream(B, H_q, H_kv, A.u, steps, 42, DEV)
    kv_a = ra.KVLayer(A.k_pool, A.v_pool, A.block_table)
    kv_f = ra.KVLayer(F.k_pool, F.v_pool, F.block_table)
    max_len = max(lens) + steps
    kt = torch.full((B,), k, dtype=torch.int32, device=DEV)
    ws_a = ra.alloc_workspace(B, H_q, H_kv, max_len, k, device=DEV)
    ws_f = ra.alloc_workspace(B, H_q, H_kv, max_len, k, device=DEV)
    outs = [[torch.empty(B, H_q, 128, device=DEV), torch.empty(B, H_q, device=DEV),
             torch.empty(B, H_q, k, dtype=torch.int32, device=DEV)] for _ in range(2)]
    for s in range(steps):
        pos = torch.tensor([n + s for n in lens], dtype=torch.int32, device=DEV)
        seq = pos + 1
        ra.kv_append(kv_a, k_s[s], v_s[s], pos)
        ra.decode_step_ex(q_s[s], kv_a, seq, max_len, kt, k, ns, window, *outs[0], ws_a)
        ra.append_decode_step(k_s[s], v_s[s], pos, q_s[s], kv_f, seq, max_len, kt, k, ns, window,
                              *outs[1], ws_f)
        torch.cuda.synchronize()
        assert torch.equal(outs[0][2], outs[1][2]), f"indices differ at step {s}"
        assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert torch.equal(A.k_pool, F.k_pool) and torch.equal(A.v_pool, F.v_pool)
