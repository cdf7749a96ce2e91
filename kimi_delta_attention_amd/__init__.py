"""MI355X (gfx950) Kimi Delta Attention forward operator.

The operator runs in hand-written HIP kernels behind the C ABI of
``include/kda.h`` (``libkda.so``); this package is its thin Python binding.
Importing it does not load the library; the first call does, and raises if the
library has not been built.
"""
from ._lib import (MAX_DRAFT, MAX_SEGMENTS, KdaError, decode_commit, decode_step,  # noqa: F401
                   decode_layer, decode_verify, epilogue, load, prefill_chunked,
                   prefill_chunked_noalloc, prefill_layer,
                   prefill_segmented,
                   prefill_varlen, prologue, segmented_workspace_size, segments_preferred,
                   workspace_size)

__all__ = ["prefill_chunked", "prefill_chunked_noalloc", "prefill_varlen", "prefill_segmented", "prefill_layer",
           "decode_step",
           "decode_verify", "decode_commit", "decode_layer", "prologue", "epilogue",
           "workspace_size", "segmented_workspace_size", "segments_preferred", "load", "KdaError",
           "MAX_DRAFT", "MAX_SEGMENTS"]
