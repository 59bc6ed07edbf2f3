"""Seeded synthetic inputs for speculative-decoding draft verification.

This package is the only code shared by the CPU oracle and the HIP path's
tests and benchmark.  It synthesises logits, draft distributions, draft token
ids and per-request Philox (seed, offset) pairs; it contains none of the
verification arithmetic (no temperature softmax, no top-k/top-p filter, no
acceptance rule, no Philox stream).  Greedy draft ids copy numpy's argmax of
the logits with a fixed probability so that draft chains get accepted.
"""
from .synth import (  # noqa: F401
    CONFIGS,
    MODE_GREEDY,
    MODE_TEMPERATURE,
    MODE_TOPK,
    MODE_TOPP,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_config,
    make_d2t,
    make_ragged_config,
    make_ragged_d2t_config,
    make_sample_config,
    fuzz_case,
)
