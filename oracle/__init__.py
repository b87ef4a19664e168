"""CPU fp64 oracle for exact top-k sparse GQA decode attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the
HIP path and imports nothing from it.

Parity pins: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, brute force, invariants and the one worked numeric
example the pages print (Table 1's KV capacity row). No function is
"parity unpinned".
"""

from .ra_oracle import (  # noqa: F401
    HEAD_DIM,
    as_f64,
    attend,
    decode,
    decode_head,
    dense,
    graph_build,
    graph_search,
    kv_bytes_per_token,
    layer_budgets,
    merge,
    partial,
    prefill_topk,
    score_f32_ordered,
    scores,
    selection_domain,
    static_set,
    topk,
)
