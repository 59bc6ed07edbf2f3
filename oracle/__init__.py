"""CPU oracle for speculative-decoding draft verification.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, float64 numpy
statement of what the verification path computes, written from the source
pages' descriptions.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import it; the library and its Python binding never do,
and this package imports nothing from them.

Parity status: every function here is pinned by tests against values other
than itself (published Philox known answers and an independent Philox build,
closed-form laws, library routines, brute force at tiny sizes).
"""
from . import philox  # noqa: F401
from .verify import (  # noqa: F401
    CDF_BAND,
    GREEDY_TEMPERATURE,
    RNG_SLOT_SPAN,
    cdf_sum_band,
    chain_reject,
    chain_reject_core,
    chain_reject_ragged,
    chain_uniforms,
    d2t_expand,
    decode_logits,
    greedy_verify,
    gumbel_band,
    gumbel_row,
    gumbel_sample,
    joint_filter_row,
    one_hot_drafts,
    ragged_pad,
    renorm_row,
    residual_draw,
    sample,
    softmax_renorm,
    temperature_softmax,
    verify_fused,
)
