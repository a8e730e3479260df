"""fp64 CPU oracle for exact attention -- test infrastructure only.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package. The HIP library never imports it and shares no code
with it.
"""
from .attention import (  # noqa: F401
    MaskSpec,
    attention_backward,
    attention_decode,
    attention_forward,
    head_backward,
    head_forward,
    mask_for,
    probabilities,
)
from .philox import Dropout, keep_threshold, philox4x32  # noqa: F401
