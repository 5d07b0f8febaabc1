"""Float64 CPU oracle (test infrastructure only; never used by the product path)."""
from .attention import (  # noqa: F401
    allowed,
    backward,
    bwd_preprocess,
    forward,
    key_grads,
    key_span,
    logical_mask_bias,
    mask_matrix,
    rows_forward,
    sample_keys,
    sample_rows,
)
