"""Oracle for the Dion3 step: a plain fp64 CPU computation written from the pages.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does, and the
oracle imports nothing from the product package.
"""

from .dion3 import (  # noqa: F401
    DEFAULT_BETA2, DEFAULT_COEFFS, DEFAULT_EPS, DEFAULT_NORMUON_EPS, DEFAULT_RESTART_AFTER,
    DEFAULT_T, MUON_QUINTIC, normuon_scale,
    apply_rows, canonical_axis, compose_poly, dion3_step, f32, frobenius_normalize,
    k_from_fraction, l1_row_norms, momentum_accumulate, muon_step, ns_gram,
    ns_gram_rounded, ns_standard, ns_standard_flops, polar_svd, round_sum, round_to,
    select_rows,
)
