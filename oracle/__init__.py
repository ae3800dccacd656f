"""fp64 CPU oracle (test infrastructure only; see falcon_oracle)."""
from .falcon_oracle import (  # noqa: F401
    FALCON_1, FALCON_2, FALCON_3, FALCON_1A, FALCON_2A, FALCON_3A,
    falcon_recurrence, falcon_masked_parallel, falcon_decode_step, is_regression,
)
