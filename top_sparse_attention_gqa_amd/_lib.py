"""ctypes binding of libra.so (include/ra.h): argument marshalling only.

Every step of the decode path runs in the library's HIP kernels. If the
library has not been built this module raises on import: there is no
fallback. Tensors are torch tensors on the GPU; they are passed as raw
pointers, with their dtype, contiguity and alignment checked first, and for
the decode path (kv_append, decode_step, decode_step_ex, decode_stages,
append_decode_step) their shapes against B, H_q, H_kv and k_max as well, so
that an undersized output never becomes an out-of-bounds device write.
Arguments given as raw integer addresses are passed through unchecked.
"""

from __future__ import annotations

import contextlib
import ctypes
import os
from ctypes import POINTER, c_int, c_int32, c_int64, c_size_t, c_uint32, c_void_p, c_char_p

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libra.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python top_sparse_attention_gqa_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)

RA_OK = 0
RA_ERR_INVALID_ARGUMENT = 1
RA_ERR_WORKSPACE = 2
RA_ERR_UNSUPPORTED = 3
RA_ERR_HIP = 4

(STAGE_SAMPLE, STAGE_THRESHOLD, STAGE_SCAN, STAGE_SELECT, STAGE_GATHER,
 STAGE_MERGE) = range(6)
STAGE_COUNT = 6
STAGE_NAMES = ["sample", "threshold", "scan", "select", "gather", "merge"]

HEAD_DIM = 128
PAGE_SIZE = 64
DECODE_KEEP_SCORES = 1
PREFILL_MAX_K = 256
(PF_STAGE_SAMPLE, PF_STAGE_BOUND, PF_STAGE_FILTER, PF_STAGE_SELECT,
 PF_STAGE_EXACT_MAXIMA, PF_STAGE_EXACT_THRESHOLD, PF_STAGE_EXACT_FILTER,
 PF_STAGE_EXACT_SELECT) = range(8)
PF_STAGE_COUNT = 8
PF_STAGE_NAMES = ["sample", "bound", "filter", "select",
                  "exact_maxima", "exact_threshold", "exact_filter", "exact_select"]

EXPORTS = ["ra_abi_version", "ra_status_str", "ra_decode_workspace_bytes",
           "ra_kv_append", "ra_decode_step", "ra_decode_step_ex", "ra_decode_stages",
           "ra_workspace_scores_offset", "ra_workspace_rescan_count_offset",
           "ra_prefill_workspace_bytes", "ra_prefill_topk", "ra_prefill_stages",
           "ra_prefill_workspace_fail_offset",
           "ra_layer_budgets", "ra_graph_build", "ra_graph_search", "ra_sparse_attend",
           "ra_merge_partials", "ra_host_device_pointer", "ra_append_decode_step",
           "ra_decode_step_noalloc"]


class KVLayerStruct(ctypes.Structure):
    _fields_ = [("k_pool", c_void_p), ("v_pool", c_void_p), ("block_table", c_void_p),
                ("num_pages", c_int32), ("max_pages", c_int32), ("H_kv", c_int32),
                ("head_dim", c_int32), ("page_size", c_int32)]


_DECODE_ARGS = [c_void_p, c_int32, POINTER(KVLayerStruct), c_void_p, c_int32, c_int32,
                c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                c_void_p, c_size_t]
NOALLOC_WS_BYTES = 64 << 20


def _declare(lib):
    """Set the ctypes signatures of every entry point of a loaded build."""
    lib.ra_abi_version.restype = c_int
    lib.ra_abi_version.argtypes = []
    lib.ra_status_str.restype = c_char_p
    lib.ra_status_str.argtypes = [c_int]
    lib.ra_decode_workspace_bytes.restype = c_size_t
    lib.ra_decode_workspace_bytes.argtypes = [c_int32] * 5
    lib.ra_workspace_scores_offset.restype = c_size_t
    lib.ra_workspace_scores_offset.argtypes = [c_int32] * 5 + [POINTER(c_int64)]
    lib.ra_prefill_workspace_bytes.restype = c_size_t
    lib.ra_prefill_workspace_bytes.argtypes = [c_int32] * 4
    lib.ra_prefill_workspace_fail_offset.restype = c_size_t
    lib.ra_prefill_workspace_fail_offset.argtypes = [c_int32] * 4
    lib.ra_prefill_topk.restype = c_int
    lib.ra_prefill_topk.argtypes = [c_void_p, c_int32, c_int32, POINTER(KVLayerStruct), c_int32,
                                    c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p,
                                    c_size_t, c_void_p]
    lib.ra_graph_build.restype = c_int
    lib.ra_graph_build.argtypes = [c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32,
                                   c_void_p, c_void_p]
    lib.ra_graph_search.restype = c_int
    lib.ra_graph_search.argtypes = [c_void_p, c_int32, c_void_p, c_int32, c_int32, c_void_p,
                                    c_int32, c_void_p, c_int32, c_int32, c_void_p, c_void_p,
                                    c_void_p]
    lib.ra_sparse_attend.restype = c_int
    lib.ra_sparse_attend.argtypes = [c_void_p, c_int32, c_void_p, c_int32, c_int32, c_void_p, c_int32,
                                     c_void_p, c_void_p, c_void_p]
    lib.ra_merge_partials.restype = c_int
    lib.ra_merge_partials.argtypes = [c_void_p] * 4 + [c_int32, c_void_p, c_void_p, c_void_p]
    lib.ra_host_device_pointer.restype = c_int
    lib.ra_host_device_pointer.argtypes = [c_void_p, POINTER(c_void_p)]
    lib.ra_layer_budgets.restype = c_int
    lib.ra_layer_budgets.argtypes = [c_int32, c_int32, c_int32, c_void_p]
    lib.ra_prefill_stages.restype = c_int
    lib.ra_prefill_stages.argtypes = lib.ra_prefill_topk.argtypes[:-1] + [c_int32, c_int32, c_void_p]
    lib.ra_workspace_rescan_count_offset.restype = c_size_t
    lib.ra_workspace_rescan_count_offset.argtypes = [c_int32] * 5
    lib.ra_kv_append.restype = c_int
    lib.ra_kv_append.argtypes = [POINTER(KVLayerStruct), c_void_p, c_void_p, c_void_p, c_int32, c_void_p]
    lib.ra_decode_step.restype = c_int
    lib.ra_decode_step.argtypes = [c_void_p, c_int32, POINTER(KVLayerStruct), c_void_p, c_int32,
                                   c_int32, c_void_p, c_int32, c_int32, c_int32, c_void_p,
                                   c_void_p, c_void_p, c_size_t, c_void_p]
    lib.ra_decode_step_ex.restype = c_int
    lib.ra_decode_step_ex.argtypes = _DECODE_ARGS + [c_uint32, c_void_p]
    lib.ra_decode_stages.restype = c_int
    lib.ra_decode_stages.argtypes = _DECODE_ARGS + [c_uint32, c_int32, c_int32, c_void_p]
    lib.ra_decode_step_noalloc.restype = c_int
    lib.ra_decode_step_noalloc.argtypes = [c_void_p, c_int32, POINTER(KVLayerStruct), c_void_p, c_int32,
                                           c_int32, c_void_p, c_int32, c_int32, c_int32, c_void_p,
                                           c_void_p, c_void_p, c_uint32, c_void_p]
    lib.ra_append_decode_step.restype = c_int
    lib.ra_append_decode_step.argtypes = [c_void_p, c_void_p, c_void_p] + _DECODE_ARGS + [c_uint32, c_void_p]
    return lib


_declare(_lib)


def load_build(path: str):
    """Load another build of the library (libra_debug.so, say) with the same
    signatures; with_build() routes the binding's calls through it."""
    return _declare(ctypes.CDLL(path))


@contextlib.contextmanager
def with_build(lib):
    """Within the block, every call of this binding goes to lib (a handle
    from load_build); the default build is restored on exit."""
    global _lib
    saved, _lib = _lib, lib
    try:
        yield lib
    finally:
        _lib = saved


class RAError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_str(status)}")


def abi_version() -> int:
    return _lib.ra_abi_version()


def status_str(status: int) -> str:
    return _lib.ra_status_str(status).decode()


def decode_workspace_bytes(B: int, H_q: int, H_kv: int, max_seq_len: int, k_max: int) -> int:
    return int(_lib.ra_decode_workspace_bytes(B, H_q, H_kv, max_seq_len, k_max))


def workspace_scores_offset(B, H_q, H_kv, max_seq_len, k_max):
    """(byte offset, row stride in floats) of the score rows inside a workspace."""
    stride = c_int64(0)
    off = _lib.ra_workspace_scores_offset(B, H_q, H_kv, max_seq_len, k_max, ctypes.byref(stride))
    if off == ctypes.c_size_t(-1).value:
        raise ValueError("invalid capacities")
    return int(off), int(stride.value)


def workspace_rescan_count_offset(B, H_q, H_kv, max_seq_len, k_max):
    """Byte offset of the uint32 count of heads decided by the full rescan."""
    off = _lib.ra_workspace_rescan_count_offset(B, H_q, H_kv, max_seq_len, k_max)
    if off == ctypes.c_size_t(-1).value:
        raise ValueError("invalid capacities")
    return int(off)


def _ptr(t, dtype, name, nullable=False, align=4):
    if t is None:
        if nullable:
            return None
        raise ValueError(f"{name} is required")
    if isinstance(t, int):  # raw device address
        return t
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if t.data_ptr() % align:
        raise ValueError(f"{name} must be {align}-byte aligned")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def host_device_pointer(t) -> int:
    """ra_host_device_pointer: the device address of a pinned host tensor."""
    if t.device.type != "cpu" or not t.is_pinned():
        raise ValueError("a host-resident pool must be a pinned CPU tensor")
    dev = c_void_p()
    st = _lib.ra_host_device_pointer(t.data_ptr(), ctypes.byref(dev))
    if st != RA_OK:
        raise RAError(st, "ra_host_device_pointer")
    return int(dev.value)


def _pool_ptr(t, name):
    # GPU pools by address; pinned host pools by their device mapping
    if t.device.type == "cpu":
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 tensor")
        p = host_device_pointer(t)
        if p % 16:
            raise ValueError(f"{name} must be 16-byte aligned")
        return p
    return _ptr(t, torch.bfloat16, name, align=16)


class KVLayer:
    """One layer's paged KV cache: bf16 pools [num_pages][H_kv][64][128] and
    an int32 block table [B][max_pages] (on the GPU). The pools may be GPU
    tensors or pinned host tensors, which the kernels then read over the
    host link (a host-resident tier)."""

    def __init__(self, k_pool, v_pool, block_table):
        for t, n in ((k_pool, "k_pool"), (v_pool, "v_pool")):
            if t.dim() != 4 or t.shape[2] != PAGE_SIZE or t.shape[3] != HEAD_DIM:
                raise ValueError(f"{n} must be [num_pages][H_kv][64][128]")
        if k_pool.shape != v_pool.shape:
            raise ValueError("k_pool and v_pool shapes differ")
        if block_table.dim() != 2:
            raise ValueError("block_table must be [B][max_pages]")
        self.k_pool, self.v_pool, self.block_table = k_pool, v_pool, block_table
        self.struct = KVLayerStruct(
            _pool_ptr(k_pool, "k_pool"), _pool_ptr(v_pool, "v_pool"),
            _ptr(block_table, torch.int32, "block_table"), k_pool.shape[0],
            block_table.shape[1], k_pool.shape[1], HEAD_DIM, PAGE_SIZE)

    @property
    def H_kv(self) -> int:
        return self.k_pool.shape[1]


def alloc_workspace(B, H_q, H_kv, max_seq_len, k_max, device="cuda") -> torch.Tensor:
    n = decode_workspace_bytes(B, H_q, H_kv, max_seq_len, k_max)
    if n == 0:
        raise ValueError("invalid capacities")
    return torch.empty(n, dtype=torch.uint8, device=device)


def _shape(t, want, name):
    """Raise ValueError unless tensor t has shape `want` (raw addresses pass)."""
    if t is None or isinstance(t, int):
        return
    if tuple(t.shape) != tuple(want):
        raise ValueError(f"{name} must have shape {tuple(want)}, got {tuple(t.shape)}")


def _numel(t, n, name):
    if t is None or isinstance(t, int):
        return
    if t.numel() != n:
        raise ValueError(f"{name} must hold {n} elements, got {t.numel()}")


def _check_batch(kv: KVLayer, B: int):
    if B <= 0:
        raise ValueError("the batch must hold at least one sequence")
    if kv.block_table.shape[0] < B:
        raise ValueError(f"block_table has {kv.block_table.shape[0]} rows for a batch of {B}")


def _check_decode(q, kv: KVLayer, seq_lens, k, k_max, out, out_lse, out_idx):
    """Shapes of the decode-step tensors; returns (B, H_q)."""
    if isinstance(q, int) or q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be a [B][H_q][128] tensor")
    B, H_q = int(q.shape[0]), int(q.shape[1])
    if H_q % kv.H_kv != 0:
        raise ValueError(f"H_q={H_q} is not a multiple of H_kv={kv.H_kv}")
    if k_max < 0:
        raise ValueError("k_max must be >= 0")
    _check_batch(kv, B)
    _numel(seq_lens, B, "seq_lens")
    _numel(k, B, "k")
    _shape(out, (B, H_q, HEAD_DIM), "out")
    _shape(out_lse, (B, H_q), "out_lse")
    if k_max > 0:
        _shape(out_idx, (B, H_q, k_max), "out_idx")
    return B, H_q


def _check_append(kv: KVLayer, k_new, v_new, pos):
    if isinstance(pos, int):
        raise ValueError("pos must be a tensor (its length is the batch)")
    B = int(pos.numel())
    _check_batch(kv, B)
    _shape(k_new, (B, kv.H_kv, HEAD_DIM), "k_new")
    _shape(v_new, (B, kv.H_kv, HEAD_DIM), "v_new")
    return B


def _flags(keep_scores):
    return DECODE_KEEP_SCORES if keep_scores else 0


def _ws_numel(ws):
    return ws.numel() if not isinstance(ws, int) else 0


def kv_append(kv: KVLayer, k_new, v_new, pos, stream=None) -> None:
    """ra_kv_append: write one token's K/V rows ([B][H_kv][128] bf16) at
    positions pos ([B] int32)."""
    B = _check_append(kv, k_new, v_new, pos)
    st = _lib.ra_kv_append(ctypes.byref(kv.struct), _ptr(k_new, torch.bfloat16, "k_new", align=16),
                           _ptr(v_new, torch.bfloat16, "v_new", align=16), _ptr(pos, torch.int32, "pos"),
                           B, _stream(stream))
    if st != RA_OK:
        raise RAError(st, "ra_kv_append")


def decode_stages(q, kv: KVLayer, seq_lens, max_seq_len, k, k_max, n_sink, window,
                  out, out_lse, out_idx, ws, first=0, last=None,
                  stream=None, keep_scores=False) -> None:
    """ra_decode_stages (the whole step when first..last covers every stage).
    keep_scores: also leave the retrieved set's scores in the score rows."""
    B, H_q = _check_decode(q, kv, seq_lens, k, k_max, out, out_lse, out_idx)
    last = STAGE_COUNT - 1 if last is None else last
    st = _lib.ra_decode_stages(
        _ptr(q, torch.bfloat16, "q", align=16), H_q, ctypes.byref(kv.struct),
        _ptr(seq_lens, torch.int32, "seq_lens"), B, max_seq_len, _ptr(k, torch.int32, "k"),
        k_max, n_sink, window, _ptr(out, torch.float32, "out"),
        _ptr(out_lse, torch.float32, "out_lse", nullable=True),
        _ptr(out_idx, torch.int32, "out_idx", nullable=(k_max == 0)),
        _ptr(ws, torch.uint8, "ws", align=256), _ws_numel(ws),
        _flags(keep_scores), first, last, _stream(stream))
    if st != RA_OK:
        raise RAError(st, "ra_decode_stages")


def decode_step(q, kv: KVLayer, seq_lens, max_seq_len, k, k_max, n_sink, window,
                out, out_idx, ws, stream=None) -> None:
    """ra_decode_step: one exact top-k sparse GQA decode step.
    q bf16 [B][H_q][128]; seq_lens, k int32 [B]; out fp32 [B][H_q][128];
    out_idx int32 [B][H_q][k_max]; ws from alloc_workspace."""
    B, H_q = _check_decode(q, kv, seq_lens, k, k_max, out, None, out_idx)
    st = _lib.ra_decode_step(
        _ptr(q, torch.bfloat16, "q", align=16), H_q, ctypes.byref(kv.struct),
        _ptr(seq_lens, torch.int32, "seq_lens"), B, max_seq_len, _ptr(k, torch.int32, "k"),
        k_max, n_sink, window, _ptr(out, torch.float32, "out"),
        _ptr(out_idx, torch.int32, "out_idx", nullable=(k_max == 0)),
        _ptr(ws, torch.uint8, "ws", align=256), _ws_numel(ws), _stream(stream))
    if st != RA_OK:
        raise RAError(st, "ra_decode_step")


def decode_step_ex(q, kv: KVLayer, seq_lens, max_seq_len, k, k_max, n_sink, window,
                   out, out_lse, out_idx, ws, stream=None, keep_scores=False) -> None:
    """ra_decode_step_ex: decode_step plus the per-head log-sum-exp
    (out_lse fp32 [B][H_q], or None) and the flags.
    keep_scores: also leave the retrieved set's scores in the score rows."""
    B, H_q = _check_decode(q, kv, seq_lens, k, k_max, out, out_lse, out_idx)
    st = _lib.ra_decode_step_ex(
        _ptr(q, torch.bfloat16, "q", align=16), H_q, ctypes.byref(kv.struct),
        _ptr(seq_lens, torch.int32, "seq_lens"), B, max_seq_len, _ptr(k, torch.int32, "k"),
        k_max, n_sink, window, _ptr(out, torch.float32, "out"),
        _ptr(out_lse, torch.float32, "out_lse", nullable=True),
        _ptr(out_idx, torch.int32, "out_idx", nullable=(k_max == 0)),
        _ptr(ws, torch.uint8, "ws", align=256), _ws_numel(ws),
        _flags(keep_scores), _stream(stream))
    if st != RA_OK:
        raise RAError(st, "ra_decode_step_ex")


def decode_step_noalloc(q, kv: KVLayer, seq_lens, max_seq_len, k, k_max, n_sink, window,
                        out, out_lse, out_idx, stream=None, keep_scores=False) -> None:
    """ra_decode_step_noalloc: decode_step_ex with the library's own device
    workspace (NOALLOC_WS_BYTES per GPU); allocates nothing."""
    B, H_q = _check_decode(q, kv, seq_lens, k, k_max, out, out_lse, out_idx)
    st = _lib.ra_decode_step_noalloc(
        _ptr(q, torch.bfloat16, "q", align=16), H_q, ctypes.byref(kv.struct),
        _ptr(seq_lens, torch.int32, "seq_lens"), B, max_seq_len, _ptr(k, torch.int32, "k"),
        k_max, n_sink, window, _ptr(out, torch.float32, "out"),
        _ptr(out_lse, torch.float32, "out_lse", nullable=True),
        _ptr(out_idx, torch.int32, "out_idx", nullable=(k_max == 0)),
        _flags(keep_scores), _stream(stream))
    if st != RA_OK:
        raise RAError(st, "ra_decode_step_noalloc")


def append_decode_step(k_new, v_new, pos, q, kv: KVLayer, seq_lens, max_seq_len, k, k_max,
                       n_sink, window, out, out_lse, out_idx, ws, stream=None,
                       keep_scores=False) -> None:
    """ra_append_decode_step: kv_append of (k_new, v_new) at pos, then the
    decode step (as decode_step_ex), with one launch fewer (the rows are
    written inside it)."""
    B, H_q = _check_decode(q, kv, seq_lens, k, k_max, out, out_lse, out_idx)
    if _check_append(kv, k_new, v_new, pos) != B:
        raise ValueError("pos must hold one position per sequence of q")
    st = _lib.ra_append_decode_step(
        _ptr(k_new, torch.bfloat16, "k_new", align=16), _ptr(v_new, torch.bfloat16, "v_new", align=16),
        _ptr(pos, torch.int32, "pos"),
        _ptr(q, torch.bfloat16, "q", align=16), H_q, ctypes.byref(kv.struct),
        _ptr(seq_lens, torch.int32, "seq_lens"), B, max_seq_len, _ptr(k, torch.int32, "k"),
        k_max, n_sink, window, _ptr(out, torch.float32, "out"),
        _ptr(out_lse, torch.float32, "out_lse", nullable=True),
        _ptr(out_idx, torch.int32, "out_idx", nullable=(k_max == 0)),
        _ptr(ws, torch.uint8, "ws", align=256), _ws_numel(ws),
        _flags(keep_scores), _stream(stream))
    if st != RA_OK:
        raise RAError(st, "ra_append_decode_step")


def scores_view(ws: torch.Tensor, B, H_q, H_kv, max_seq_len, k_max) -> torch.Tensor:
    """The fp32 score rows [B][H_q][row_stride] inside a workspace: after the
    gather stage they hold the scores of W and of the retrieved positions."""
    off, stride = workspace_scores_offset(B, H_q, H_kv, max_seq_len, k_max)
    n = B * H_q * stride
    return ws[off:off + 4 * n].view(torch.float32).view(B, H_q, stride)


def rescan_count(ws: torch.Tensor, B, H_q, H_kv, max_seq_len, k_max) -> int:
    """Heads of the last call on this workspace whose candidates fell short
    of k_eff and were decided by the full rescan (reads device memory)."""
    off = workspace_rescan_count_offset(B, H_q, H_kv, max_seq_len, k_max)
    return int(ws[off:off + 4].view(torch.int32).item())


def prefill_workspace_bytes(T: int, H_q: int, N: int, k: int) -> int:
    return int(_lib.ra_prefill_workspace_bytes(T, H_q, N, k))


def prefill_workspace_fail_offset(T: int, H_q: int, N: int, k: int) -> int:
    return int(_lib.ra_prefill_workspace_fail_offset(T, H_q, N, k))


def prefill_fail_flags(ws, T: int, H_q: int, N: int, k: int) -> torch.Tensor:
    """View of the per-row flags in a prefill workspace: int32 [T][H_q], 1 for
    a row the exact pass decided (its sampled bound fell short)."""
    off = prefill_workspace_fail_offset(T, H_q, N, k)
    return ws[off:off + 4 * T * H_q].view(torch.int32).view(T, H_q)


def alloc_prefill_workspace(T, H_q, N, k, device="cuda") -> torch.Tensor:
    n = prefill_workspace_bytes(T, H_q, N, k)
    if n == 0:
        raise ValueError("invalid capacities")
    return torch.empty(n, dtype=torch.uint8, device=device)


def prefill_stages(q, kv: KVLayer, seq: int, N: int, k: int, n_sink: int, window: int,
                   out_idx, ws, first=PF_STAGE_SAMPLE, last=PF_STAGE_EXACT_SELECT,
                   stream=None) -> None:
    """ra_prefill_stages (ra_prefill_topk when first..last covers every stage).
    q: bf16 [T][H_q][128]; out_idx: int32 [T][H_q][k] (ascending, -1 padded)."""
    T, H_q = q.shape[0], q.shape[1]
    if k > 0 and tuple(out_idx.shape) != (T, H_q, k):
        raise ValueError("out_idx must be [T][H_q][k]")
    st = _lib.ra_prefill_stages(
        _ptr(q, torch.bfloat16, "q", align=16), T, H_q, ctypes.byref(kv.struct), seq, N, k,
        n_sink, window, _ptr(out_idx, torch.int32, "out_idx", nullable=(k == 0)),
        _ptr(ws, torch.uint8, "ws", align=256), ws.numel(), first, last, _stream(stream))
    if st != RA_OK:
        raise RAError(st, "ra_prefill_stages")


def prefill_topk(q, kv: KVLayer, seq: int, N: int, k: int, n_sink: int, window: int,
                 out_idx, ws, stream=None) -> None:
    """ra_prefill_topk: exact top-k keys of every prefill query row and head.
    q: bf16 [T][H_q][128]; out_idx: int32 [T][H_q][k] (ascending, -1 padded)."""
    T, H_q = q.shape[0], q.shape[1]
    if k > 0 and tuple(out_idx.shape) != (T, H_q, k):
        raise ValueError("out_idx must be [T][H_q][k]")
    st = _lib.ra_prefill_topk(
        _ptr(q, torch.bfloat16, "q", align=16), T, H_q, ctypes.byref(kv.struct), seq, N, k,
        n_sink, window, _ptr(out_idx, torch.int32, "out_idx", nullable=(k == 0)),
        _ptr(ws, torch.uint8, "ws", align=256), ws.numel(), _stream(stream))
    if st != RA_OK:
        raise RAError(st, "ra_prefill_topk")


raw = _lib  # the C entry points, for tests that pass raw pointers


def layer_budgets(n_layers: int, k_mean: int, slope_permille: int) -> list:
    """ra_layer_budgets: pyramid-shaped per-layer budgets with the total of
    k_mean per layer (slope 0: uniform)."""
    buf = (ctypes.c_int32 * max(n_layers, 1))()
    st = _lib.ra_layer_budgets(n_layers, k_mean, slope_permille, ctypes.cast(buf, c_void_p))
    if st != RA_OK:
        raise RAError(st, "ra_layer_budgets")
    return [int(x) for x in buf[:n_layers]]

GRAPH_MAX_DEGREE = 64
GRAPH_MAX_EF = 256
GRAPH_MAX_N = 1 << 20
GRAPH_BATCH = 16  # keys a search expands per round


def graph_build(hubs, lists, N: int, D: int):
    """ra_graph_build (host): one query head's key graph from its prefill
    queries' best keys hubs [T] and top keys lists [T][K] (int32 arrays,
    -1 padded). Returns (nbr int32 [N][D], entry)."""
    import numpy as np
    h = np.ascontiguousarray(np.asarray(hubs, dtype=np.int32))
    L = np.ascontiguousarray(np.asarray(lists, dtype=np.int32))
    T = int(h.shape[0])
    K = int(L.shape[1]) if L.ndim == 2 else 1
    if T and (L.ndim != 2 or L.shape[0] != T):
        raise ValueError("lists must be [T][K]")
    nbr = np.empty((N, D), dtype=np.int32)
    entry = ctypes.c_int32(-1)
    st = _lib.ra_graph_build(h.ctypes.data if T else None, L.ctypes.data if T else None, T, K,
                             N, D, nbr.ctypes.data, ctypes.addressof(entry))
    if st != RA_OK:
        raise RAError(st, "ra_graph_build")
    return nbr, int(entry.value)


def graph_search(q, kv: KVLayer, seq: int, N: int, nbr, entry, ef: int, k: int, out_idx,
                 out_visited, stream=None) -> None:
    """ra_graph_search: best-first search of each query head's key graph.
    q bf16 [H_q][128]; nbr int32 [H_q][N][D]; entry int32 [H_q];
    out_idx int32 [H_q][k]; out_visited int32 [H_q] (all device)."""
    H_q = q.shape[0]
    D = nbr.shape[-1]
    if tuple(nbr.shape) != (H_q, N, D) or tuple(out_idx.shape) != (H_q, k):
        raise ValueError("nbr must be [H_q][N][D] and out_idx [H_q][k]")
    st = _lib.ra_graph_search(
        _ptr(q, torch.bfloat16, "q", align=16), H_q, ctypes.byref(kv.struct), seq, N,
        _ptr(nbr, torch.int32, "nbr"), D, _ptr(entry, torch.int32, "entry"), ef, k,
        _ptr(out_idx, torch.int32, "out_idx"), _ptr(out_visited, torch.int32, "out_visited"),
        _stream(stream))
    if st != RA_OK:
        raise RAError(st, "ra_graph_search")

SPARSE_MAX_K = 4096


def sparse_attend(q, kv: KVLayer, seq: int, N: int, idx, out, out_lse, stream=None) -> None:
    """ra_sparse_attend: softmax . V over the positions idx [H_q][k] (int32,
    -1 skipped) for each query head; out fp32 [H_q][128], out_lse [H_q]."""
    H_q = q.shape[0]
    k = idx.shape[1]
    if idx.shape[0] != H_q or tuple(out.shape) != (H_q, HEAD_DIM) or tuple(out_lse.shape) != (H_q,):
        raise ValueError("idx must be [H_q][k], out [H_q][128], out_lse [H_q]")
    st = _lib.ra_sparse_attend(
        _ptr(q, torch.bfloat16, "q", align=16), H_q, ctypes.byref(kv.struct), seq, N,
        _ptr(idx, torch.int32, "idx"), k, _ptr(out, torch.float32, "out"),
        _ptr(out_lse, torch.float32, "out_lse"), _stream(stream))
    if st != RA_OK:
        raise RAError(st, "ra_sparse_attend")


def merge_partials(out_a, lse_a, out_b, lse_b, out, lse, stream=None) -> None:
    """ra_merge_partials: the LSE merge of two partial outputs per head."""
    H = lse_a.shape[0]
    st = _lib.ra_merge_partials(
        _ptr(out_a, torch.float32, "out_a"), _ptr(lse_a, torch.float32, "lse_a"),
        _ptr(out_b, torch.float32, "out_b"), _ptr(lse_b, torch.float32, "lse_b"), H,
        _ptr(out, torch.float32, "out"), _ptr(lse, torch.float32, "lse"), _stream(stream))
    if st != RA_OK:
        raise RAError(st, "ra_merge_partials")

