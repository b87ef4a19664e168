"""Exact top-k sparse GQA decode attention for MI355X (gfx950).

The decode step (exact scores over the whole KV cache, per-head top-k over
the non-static positions, softmax . V over the static and retrieved union,
log-sum-exp merge) runs in the HIP kernels of libra.so, behind the C ABI in
include/ra.h. This package is the thin Python binding: import fails loudly
if the library has not been built.
"""

from ._lib import (  # noqa: F401
    EXPORTS,
    HEAD_DIM,
    PAGE_SIZE,
    PF_STAGE_COUNT,
    PF_STAGE_FILTER,
    PF_STAGE_MAXIMA,
    PF_STAGE_NAMES,
    PF_STAGE_SELECT,
    PF_STAGE_THRESHOLD,
    PREFILL_MAX_K,
    RA_ERR_HIP,
    RA_ERR_INVALID_ARGUMENT,
    RA_ERR_UNSUPPORTED,
    RA_ERR_WORKSPACE,
    RA_OK,
    STAGE_COUNT,
    STAGE_GATHER,
    STAGE_MERGE,
    STAGE_NAMES,
    STAGE_SAMPLE,
    STAGE_SCAN,
    STAGE_SELECT,
    STAGE_THRESHOLD,
    KVLayer,
    KVLayerStruct,
    RAError,
    abi_version,
    alloc_prefill_workspace,
    alloc_workspace,
    decode_stages,
    decode_step,
    decode_workspace_bytes,
    kv_append,
    layer_budgets,
    prefill_stages,
    prefill_topk,
    prefill_workspace_bytes,
    rescan_count,
    scores_view,
    status_str,
    workspace_rescan_count_offset,
    workspace_scores_offset,
)
