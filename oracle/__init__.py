"""CPU float64 oracle for FAVOR attention -- test infrastructure only.

Only the test suite, the package smoke check and the benchmark's CPU
baseline leg may import this package.  The GPU library never imports it,
and it imports nothing from the GPU library.
"""
from .favor_oracle import (  # noqa: F401
    KINDS, default_workers, favor_attention, favor_quadratic, favor_quadratic_rows,
    favor_rows, feature_map, feature_width, gram_schmidt_rows,
    orthogonal_random_features, performer_block, softmax_attention,
)
