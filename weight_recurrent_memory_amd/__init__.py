"""Falcon fast-weight attention on MI355X (gfx950): HIP kernels behind a C ABI.

The compute lives in ``libfalcon.so`` (built from ``csrc/``); this package only
marshals torch tensors into its C entry points.  Importing the package does not
load the library; the first call does, and fails loudly if it is missing.
"""
from .binding import (  # noqa: F401
    FALCON_1, FALCON_2, FALCON_3, FALCON_1A, FALCON_2A, FALCON_3A,
    VARIANT_NAMES, FalconError, bwd_chunk, bwd_chunk_noalloc, decode_step, fwd_chunk,
    fwd_masked, fwd_recurrent, library_path, load_library,
)
