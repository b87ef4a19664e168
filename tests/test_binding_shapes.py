"""The Python binding checks the shapes of the decode-path tensors against
B, H_q, H_kv and k_max before any call into the library, so an undersized
output or index buffer is a ValueError on the host, never an out-of-bounds
device write. CPU only: the checks run before any device address is taken."""

import pytest
import torch

import top_sparse_attention_gqa_amd as ra


def fake_kv(B=2, H_kv=2, max_pages=4, num_pages=8):
    # a KVLayer without device memory: only its shapes are looked at
    kv = object.__new__(ra.KVLayer)
    kv.k_pool = torch.empty(num_pages, H_kv, 64, 128, dtype=torch.bfloat16)
    kv.v_pool = torch.empty_like(kv.k_pool)
    kv.block_table = torch.zeros(B, max_pages, dtype=torch.int32)
    kv.struct = None
    return kv


def args(B=2, H_q=8, k_max=16, **over):
    a = dict(q=torch.empty(B, H_q, 128, dtype=torch.bfloat16),
             seq_lens=torch.zeros(B, dtype=torch.int32), k=torch.zeros(B, dtype=torch.int32),
             out=torch.empty(B, H_q, 128), out_lse=torch.empty(B, H_q),
             out_idx=torch.empty(B, H_q, k_max, dtype=torch.int32))
    a.update(over)
    return a


def run_ex(kv, k_max=16, **a):
    ra.decode_step_ex(a["q"], kv, a["seq_lens"], 256, a["k"], k_max, 4, 8, a["out"],
                      a["out_lse"], a["out_idx"], ws=None)


def run_plain(kv, k_max=16, **a):
    ra.decode_step(a["q"], kv, a["seq_lens"], 256, a["k"], k_max, 4, 8, a["out"],
                   a["out_idx"], ws=None)


@pytest.mark.parametrize("over,msg", [
    (dict(out=torch.empty(2, 8, 64)), "out must have shape"),
    (dict(out=torch.empty(1, 8, 128)), "out must have shape"),
    (dict(out_idx=torch.empty(2, 8, 15, dtype=torch.int32)), "out_idx must have shape"),
    (dict(out_idx=torch.empty(2, 7, 16, dtype=torch.int32)), "out_idx must have shape"),
    (dict(out_lse=torch.empty(2, 4)), "out_lse must have shape"),
    (dict(seq_lens=torch.zeros(1, dtype=torch.int32)), "seq_lens must hold 2"),
    (dict(k=torch.zeros(3, dtype=torch.int32)), "k must hold 2"),
    (dict(q=torch.empty(2, 8, 64, dtype=torch.bfloat16)), "q must be a"),
    (dict(q=torch.empty(2, 7, 128, dtype=torch.bfloat16)), "not a multiple of H_kv"),
])
def test_undersized_or_misshapen_tensors_are_rejected(over, msg):
    a = args(**over)
    with pytest.raises(ValueError, match=msg):
        run_ex(fake_kv(), **a)
    if "out_lse" not in over:
        with pytest.raises(ValueError, match=msg):
            run_plain(fake_kv(), **a)


def test_block_table_needs_a_row_per_sequence():
    with pytest.raises(ValueError, match="block_table has 1 rows"):
        run_ex(fake_kv(B=1), **args())


def test_well_shaped_tensors_pass_the_shape_checks():
    # the next check wants device tensors: reaching it means the shapes passed
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        run_ex(fake_kv(), **args())
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        run_plain(fake_kv(), **args())


def test_k_max_zero_needs_no_index_buffer():
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        run_ex(fake_kv(), k_max=0, **args(out_idx=None))


def test_append_shapes():
    kv = fake_kv()
    kn = torch.empty(2, 2, 128, dtype=torch.bfloat16)
    pos = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="k_new must have shape"):
        ra.kv_append(kv, torch.empty(2, 1, 128, dtype=torch.bfloat16), kn, pos)
    with pytest.raises(ValueError, match="v_new must have shape"):
        ra.kv_append(kv, kn, torch.empty(1, 2, 128, dtype=torch.bfloat16), pos)
    with pytest.raises(ValueError, match="block_table has 2 rows"):
        ra.kv_append(kv, torch.empty(3, 2, 128, dtype=torch.bfloat16),
                     torch.empty(3, 2, 128, dtype=torch.bfloat16), torch.zeros(3, dtype=torch.int32))
    a = args()
    with pytest.raises(ValueError, match="one position per sequence"):
        ra.append_decode_step(torch.empty(1, 2, 128, dtype=torch.bfloat16),
                              torch.empty(1, 2, 128, dtype=torch.bfloat16),
                              torch.zeros(1, dtype=torch.int32), a["q"], kv, a["seq_lens"], 256,
                              a["k"], 16, 4, 8, a["out"], a["out_lse"], a["out_idx"], ws=None)
