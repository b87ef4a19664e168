"""Seeded synthetic inputs for the top-k sparse GQA decode step.

This package only draws random tensors and lays them out in the paged KV
format; it computes none of the method's arithmetic (no scores, no top-k, no
softmax). Both the HIP path's tests and the CPU oracle's tests take their
inputs from here, and from nowhere else.
"""

from .configs import CONFIGS, LayerConfig, config  # noqa: F401
from .gen import (  # noqa: F401
    PAGE,
    HEAD_DIM,
    LayerInputs,
    bf16_bits,
    depage,
    history,
    draw_lengths,
    make_decode_stream,
    make_layer,
    copy_pages,
    make_prefill_queries,
    make_topic_queries,
    make_new_tokens,
)
