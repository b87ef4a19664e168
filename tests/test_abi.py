"""The C ABI on the CPU: the library loads, exports every function that
include/ra.h declares, and rejects bad host arguments with the documented
status before touching the GPU (validation is pure host code, so fake
device addresses are enough here)."""

import ctypes
import os
import re

import pytest

import top_sparse_attention_gqa_amd as ra
from top_sparse_attention_gqa_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "ra.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ra_[a-z_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("ra_abi_version", "ra_status_str", "ra_decode_workspace_bytes",
              "ra_kv_append", "ra_decode_step", "ra_decode_step_ex"):
        assert n in names


def test_library_exports_every_declared_function():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} not exported"
    assert sorted(_lib.EXPORTS) == declared_functions()


def test_version_and_status_strings():
    assert ra.abi_version() == 5
    assert ra.status_str(ra.RA_OK) == "RA_OK"
    assert ra.status_str(ra.RA_ERR_WORKSPACE) == "RA_ERR_WORKSPACE"
    assert ra.status_str(99) == "RA_ERR_UNKNOWN"


def test_workspace_size():
    a = ra.decode_workspace_bytes(1, 32, 8, 131072, 2048)
    b = ra.decode_workspace_bytes(1, 32, 8, 1048576, 31457)
    assert 0 < a < b
    # score rows dominate: B * H_q * N_cap * 4 bytes
    assert b >= 32 * 1048576 * 4
    assert ra.decode_workspace_bytes(0, 32, 8, 1024, 1) == 0
    assert ra.decode_workspace_bytes(1, 30, 8, 1024, 1) == 0   # H_q % H_kv
    assert ra.decode_workspace_bytes(1, 32, 8, 0, 1) == 0
    assert ra.decode_workspace_bytes(1, 32, 8, 1024, -1) == 0
    assert ra.decode_workspace_bytes(1, 32, 8, (1 << 24) + 1, 1) == 0
    assert ra.decode_workspace_bytes(1, 32, 8, 1 << 24, 1) > 0
    off, stride = ra.workspace_scores_offset(2, 4, 1, 5000, 64)
    assert off == 0 and stride % 8192 == 0 and stride >= 5000


FAKE = 0x10000  # a non-null, 256-byte aligned address that is never dereferenced


def _kv(**kw):
    d = dict(k_pool=FAKE, v_pool=FAKE, block_table=FAKE, num_pages=10, max_pages=10,
             H_kv=1, head_dim=128, page_size=64)
    d.update(kw)
    return _lib.KVLayerStruct(*d.values())


def _decode(kv=None, **kw):
    a = dict(q=FAKE, H_q=4, seq_lens=FAKE, B=1, max_seq_len=640, k=FAKE, k_max=8,
             n_sink=4, window=8, out=FAKE, lse=None, out_idx=FAKE, ws=FAKE,
             ws_bytes=1 << 40, flags=0)
    a.update(kw)
    kv = kv if kv is not None else _kv()
    return _lib.raw.ra_decode_step_ex(a["q"], a["H_q"], ctypes.byref(kv), a["seq_lens"], a["B"],
                                      a["max_seq_len"], a["k"], a["k_max"], a["n_sink"],
                                      a["window"], a["out"], a["lse"], a["out_idx"], a["ws"],
                                      a["ws_bytes"], a["flags"], None)


def _decode_plain(kv=None, **kw):
    # ra_decode_step: the boundary's own prototype (no out_lse, no flags)
    a = dict(q=FAKE, H_q=4, seq_lens=FAKE, B=1, max_seq_len=640, k=FAKE, k_max=8,
             n_sink=4, window=8, out=FAKE, out_idx=FAKE, ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    kv = kv if kv is not None else _kv()
    return _lib.raw.ra_decode_step(a["q"], a["H_q"], ctypes.byref(kv), a["seq_lens"], a["B"],
                                   a["max_seq_len"], a["k"], a["k_max"], a["n_sink"],
                                   a["window"], a["out"], a["out_idx"], a["ws"],
                                   a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), ra.RA_ERR_INVALID_ARGUMENT),
    (dict(out=None), ra.RA_ERR_INVALID_ARGUMENT),
    (dict(seq_lens=None), ra.RA_ERR_INVALID_ARGUMENT),
    (dict(k=None), ra.RA_ERR_INVALID_ARGUMENT),
    (dict(ws=None), ra.RA_ERR_INVALID_ARGUMENT),
    (dict(out_idx=None), ra.RA_ERR_INVALID_ARGUMENT),
    (dict(B=0), ra.RA_ERR_INVALID_ARGUMENT),
    (dict(H_q=0), ra.RA_ERR_INVALID_ARGUMENT),
    (dict(H_q=3, kv=None), ra.RA_ERR_UNSUPPORTED),
    (dict(max_seq_len=0), ra.RA_ERR_INVALID_ARGUMENT),
    (dict(k_max=-1), ra.RA_ERR_INVALID_ARGUMENT),
    (dict(n_sink=-1), ra.RA_ERR_INVALID_ARGUMENT),
    (dict(window=-5), ra.RA_ERR_INVALID_ARGUMENT),
    (dict(ws=FAKE + 16), ra.RA_ERR_INVALID_ARGUMENT),
    (dict(q=FAKE + 8), ra.RA_ERR_INVALID_ARGUMENT),        # q rows are read 16 B at a time
    (dict(seq_lens=FAKE + 2), ra.RA_ERR_INVALID_ARGUMENT),
    (dict(out_idx=FAKE + 1), ra.RA_ERR_INVALID_ARGUMENT),
    (dict(ws_bytes=1024), ra.RA_ERR_WORKSPACE),
    (dict(H_q=16), ra.RA_ERR_UNSUPPORTED),   # G = 16
    (dict(flags=2), ra.RA_ERR_INVALID_ARGUMENT),  # an unknown flag
    (dict(flags=1, ws_bytes=1024), ra.RA_ERR_WORKSPACE),  # KEEP_SCORES is known
])
def test_decode_validation(kw, status):
    kw = dict(kw)
    kw.pop("kv", None)
    assert _decode(**kw) == status
    if "flags" not in kw:
        # the plain prototype validates the same way
        assert _decode_plain(**kw) == status


def test_decode_validation_of_the_kv_descriptor():
    assert _decode(kv=_kv(head_dim=64)) == ra.RA_ERR_UNSUPPORTED
    assert _decode(kv=_kv(page_size=16)) == ra.RA_ERR_UNSUPPORTED
    assert _decode(kv=_kv(k_pool=None)) == ra.RA_ERR_INVALID_ARGUMENT
    assert _decode(kv=_kv(block_table=None)) == ra.RA_ERR_INVALID_ARGUMENT
    assert _decode(kv=_kv(num_pages=0)) == ra.RA_ERR_INVALID_ARGUMENT
    assert _decode(kv=_kv(k_pool=FAKE + 4)) == ra.RA_ERR_INVALID_ARGUMENT
    assert _decode(kv=_kv(block_table=FAKE + 2)) == ra.RA_ERR_INVALID_ARGUMENT
    assert _decode(kv=_kv(H_kv=3)) == ra.RA_ERR_INVALID_ARGUMENT  # 4 % 3
    assert _lib.raw.ra_decode_step_ex(FAKE, 4, None, FAKE, 1, 640, FAKE, 8, 4, 8, FAKE, None,
                                      FAKE, FAKE, 1 << 40, 0, None) == ra.RA_ERR_INVALID_ARGUMENT
    assert _lib.raw.ra_decode_step(FAKE, 4, None, FAKE, 1, 640, FAKE, 8, 4, 8, FAKE,
                                   FAKE, FAKE, 1 << 40, None) == ra.RA_ERR_INVALID_ARGUMENT
    assert _decode_plain(kv=_kv(head_dim=64)) == ra.RA_ERR_UNSUPPORTED


def test_k_max_zero_allows_null_out_idx_until_a_later_check():
    # with k_max == 0 a null out_idx is allowed; the call then fails only on
    # the (too small) workspace, which proves out_idx was accepted
    assert _decode(k_max=0, out_idx=None, ws_bytes=16) == ra.RA_ERR_WORKSPACE


def test_stage_range_validation():
    kv = _kv()
    args = [FAKE, 4, ctypes.byref(kv), FAKE, 1, 640, FAKE, 8, 4, 8, FAKE, None, FAKE, FAKE, 1 << 40, 0]
    assert _lib.raw.ra_decode_stages(*args, 3, 2, None) == ra.RA_ERR_INVALID_ARGUMENT
    assert _lib.raw.ra_decode_stages(*args, -1, 2, None) == ra.RA_ERR_INVALID_ARGUMENT
    assert _lib.raw.ra_decode_stages(*args, 0, 6, None) == ra.RA_ERR_INVALID_ARGUMENT
    assert ra.STAGE_COUNT == 6 and len(ra.STAGE_NAMES) == 6


def test_kv_append_validation():
    kv = _kv()
    f = _lib.raw.ra_kv_append
    assert f(ctypes.byref(kv), None, FAKE, FAKE, 1, None) == ra.RA_ERR_INVALID_ARGUMENT
    assert f(ctypes.byref(kv), FAKE, FAKE, None, 1, None) == ra.RA_ERR_INVALID_ARGUMENT
    assert f(ctypes.byref(kv), FAKE, FAKE, FAKE, 0, None) == ra.RA_ERR_INVALID_ARGUMENT
    assert f(ctypes.byref(kv), FAKE + 8, FAKE, FAKE, 1, None) == ra.RA_ERR_INVALID_ARGUMENT
    bad = _kv(head_dim=256)
    assert f(ctypes.byref(bad), FAKE, FAKE, FAKE, 1, None) == ra.RA_ERR_UNSUPPORTED


def test_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 4, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        _lib._ptr(q, torch.bfloat16, "q")
    with pytest.raises(TypeError):
        _lib._ptr(q.float(), torch.bfloat16, "q")


def _prefill(kv=None, **kw):
    a = dict(q=FAKE, T=16, H_q=4, seq=0, N=640, k=8, n_sink=4, window=8, out_idx=FAKE,
             ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    kv = kv if kv is not None else _kv()
    return _lib.raw.ra_prefill_topk(a["q"], a["T"], a["H_q"], ctypes.byref(kv), a["seq"], a["N"],
                                    a["k"], a["n_sink"], a["window"], a["out_idx"], a["ws"],
                                    a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), ra.RA_ERR_INVALID_ARGUMENT),
    (dict(out_idx=None), ra.RA_ERR_INVALID_ARGUMENT),
    (dict(ws=None), ra.RA_ERR_INVALID_ARGUMENT),
    (dict(T=0), ra.RA_ERR_INVALID_ARGUMENT),
    (dict(H_q=0), ra.RA_ERR_INVALID_ARGUMENT),
    (dict(seq=-1), ra.RA_ERR_INVALID_ARGUMENT),
    (dict(N=0), ra.RA_ERR_INVALID_ARGUMENT),
    (dict(N=641), ra.RA_ERR_INVALID_ARGUMENT),          # beyond 64 * max_pages
    (dict(k=-1), ra.RA_ERR_INVALID_ARGUMENT),
    (dict(k=257), ra.RA_ERR_INVALID_ARGUMENT),          # above RA_PREFILL_MAX_K
    (dict(n_sink=-1), ra.RA_ERR_INVALID_ARGUMENT),
    (dict(q=FAKE + 8), ra.RA_ERR_INVALID_ARGUMENT),
    (dict(ws=FAKE + 64), ra.RA_ERR_INVALID_ARGUMENT),
    (dict(ws_bytes=1024), ra.RA_ERR_WORKSPACE),
    (dict(H_q=16), ra.RA_ERR_UNSUPPORTED),              # G = 16
])
def test_prefill_validation(kw, status):
    assert _prefill(**kw) == status


def test_prefill_workspace_size():
    a = ra.prefill_workspace_bytes(1024, 32, 131072, 100)
    # dominated by the candidate lists: rows * 64 k entries of 8 bytes
    assert a >= 1024 * 32 * 64 * 100 * 8
    assert ra.prefill_workspace_bytes(0, 32, 1000, 10) == 0
    assert ra.prefill_workspace_bytes(4, 32, 1000, 257) == 0
    assert ra.prefill_workspace_bytes(4, 32, 0, 10) == 0
    # k = 0 needs no work but still validates; a null out_idx is allowed then
    assert _prefill(k=0, out_idx=None, ws_bytes=1 << 40) == ra.RA_OK


def test_prefill_stage_range_validation():
    kv = _kv()
    args = [FAKE, 16, 4, ctypes.byref(kv), 0, 640, 8, 4, 8, FAKE, FAKE, 1 << 40]
    assert _lib.raw.ra_prefill_stages(*args, 2, 1, None) == ra.RA_ERR_INVALID_ARGUMENT
    assert _lib.raw.ra_prefill_stages(*args, -1, 1, None) == ra.RA_ERR_INVALID_ARGUMENT
    assert _lib.raw.ra_prefill_stages(*args, 0, ra.PF_STAGE_COUNT, None) == ra.RA_ERR_INVALID_ARGUMENT
    assert ra.PF_STAGE_COUNT == 8 and len(ra.PF_STAGE_NAMES) == 8


def test_prefill_fail_flags_lie_inside_the_workspace():
    for T, H_q, N, k in [(16, 4, 640, 8), (1024, 32, 131072, 100), (3, 8, 70, 256)]:
        off = ra.prefill_workspace_fail_offset(T, H_q, N, k)
        assert off > 0 and off % 256 == 0
        assert off + 4 * T * H_q <= ra.prefill_workspace_bytes(T, H_q, N, k)
    assert ra.prefill_workspace_fail_offset(0, 4, 640, 8) == 0


def test_layer_budgets_match_the_oracle():
    # host arithmetic of the library against the oracle's exact rationals
    import oracle
    for L in (1, 2, 3, 5, 8, 31, 32, 80):
        for k in (0, 1, 7, 100, 10485, 31457):
            for slope in (0, 1, 333, 500, 999, 1000):
                assert ra.layer_budgets(L, k, slope) == oracle.layer_budgets(L, k, slope), (L, k, slope)


def test_layer_budgets_reject_bad_arguments():
    buf = (ctypes.c_int32 * 4)()
    for args in ((0, 5, 0), (4, -1, 0), (4, 5, -1), (4, 5, 1001), (5000, 5, 0)):
        assert _lib.raw.ra_layer_budgets(*args, ctypes.cast(buf, ctypes.c_void_p)) == ra.RA_ERR_INVALID_ARGUMENT
    assert _lib.raw.ra_layer_budgets(4, 5, 0, None) == ra.RA_ERR_INVALID_ARGUMENT


def test_graph_build_matches_the_oracle():
    # host build of the library against the oracle's projection
    import numpy as np

    import oracle
    r = np.random.default_rng(7)
    for N, T, K, D in ((50, 20, 5, 3), (300, 120, 8, 16), (1000, 400, 16, 64), (64, 0, 4, 8)):
        lists = np.stack([r.choice(N, K, replace=False) for _ in range(T)]).astype(np.int32) \
            if T else np.zeros((0, K), np.int32)
        if T:
            lists[r.random((T, K)) < 0.1] = -1       # some padding
        hubs = np.array([l[l >= 0][0] if (l >= 0).any() else -1 for l in lists], np.int32)
        if T:
            hubs[::7] = -1                            # some queries without a hub
        nbr, entry = ra.graph_build(hubs, lists, N, D)
        want, want_entry = oracle.graph_build(hubs, lists, N, D)
        assert np.array_equal(nbr, want) and entry == want_entry


def test_graph_arguments_are_checked():
    import numpy as np
    with pytest.raises(ra.RAError):
        ra.graph_build(np.array([5], np.int32), np.array([[1, 2]], np.int32), 4, 2)   # hub >= N
    with pytest.raises(ra.RAError):
        ra.graph_build(np.array([0], np.int32), np.array([[1, 2]], np.int32), 4, 65)  # D > 64
    # every call below fails validation, so nothing is launched
    kv = _kv()
    base = [FAKE, 4, ctypes.byref(kv), 0, 640, FAKE, 8, FAKE, 8, 4, FAKE, FAKE, None]
    bad = list(base); bad[9] = 9                  # k > ef
    assert _lib.raw.ra_graph_search(*bad) == ra.RA_ERR_INVALID_ARGUMENT
    bad = list(base); bad[8] = 257                # ef > 256
    assert _lib.raw.ra_graph_search(*bad) == ra.RA_ERR_INVALID_ARGUMENT
    bad = list(base); bad[6] = 65                 # D > 64
    assert _lib.raw.ra_graph_search(*bad) == ra.RA_ERR_INVALID_ARGUMENT
    bad = list(base); bad[4] = 641                # N beyond the table's pages
    assert _lib.raw.ra_graph_search(*bad) == ra.RA_ERR_INVALID_ARGUMENT
    bad = list(base); bad[10] = None              # no output
    assert _lib.raw.ra_graph_search(*bad) == ra.RA_ERR_INVALID_ARGUMENT


def test_tier_entry_points_check_arguments():
    # every call below fails validation, so nothing is launched
    kv = _kv()
    a = [FAKE, 4, ctypes.byref(kv), 0, 640, FAKE, 8, FAKE, FAKE, None]
    bad = list(a); bad[6] = 0                      # k = 0
    assert _lib.raw.ra_sparse_attend(*bad) == ra.RA_ERR_INVALID_ARGUMENT
    bad = list(a); bad[6] = 4097                   # k > RA_SPARSE_MAX_K
    assert _lib.raw.ra_sparse_attend(*bad) == ra.RA_ERR_INVALID_ARGUMENT
    bad = list(a); bad[4] = 641                    # N beyond the table
    assert _lib.raw.ra_sparse_attend(*bad) == ra.RA_ERR_INVALID_ARGUMENT
    bad = list(a); bad[7] = None                   # no output
    assert _lib.raw.ra_sparse_attend(*bad) == ra.RA_ERR_INVALID_ARGUMENT
    assert _lib.raw.ra_merge_partials(FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, None) == ra.RA_ERR_INVALID_ARGUMENT
    assert _lib.raw.ra_merge_partials(FAKE, None, FAKE, FAKE, 4, FAKE, FAKE, None) == ra.RA_ERR_INVALID_ARGUMENT
    dev = ctypes.c_void_p()
    assert _lib.raw.ra_host_device_pointer(None, ctypes.byref(dev)) == ra.RA_ERR_INVALID_ARGUMENT
