"""Seeded synthetic inputs shared by the tests, the bench and the oracle's own checks.

This package draws random numbers and rounds them to the storage dtype.  It holds
none of the mapping arithmetic (no rotation, no feature assembly, no affine map,
no statistics); both the HIP library and the fp64 oracle receive what it draws.
"""

from .workloads import (  # noqa: F401
    ApplyConfig,
    FitStatsConfig,
    APPLY_CONFIGS,
    FIT_STATS_CONFIG,
    FITCHECK,
    bf16_round_bits,
    bf16_bits_to_f32,
    bf16_bits_to_f64,
    layer_sel,
    src_head,
    src_layer,
    w_layer,
    b_layer,
    fit_batch,
    fitcheck_draws,
)
