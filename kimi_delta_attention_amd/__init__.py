"""MI355X (gfx950) Kimi Delta Attention forward operator.

The operator runs in hand-written HIP kernels behind the C ABI of
``include/kda.h`` (``libkda.so``); this package is its thin Python binding.
Importing it does not load the library; the first call does, and raises if the
library has not been built.
"""
from ._lib import (KdaError, decode_step, load, prefill_chunked, prefill_varlen,  # noqa: F401
                   workspace_size)

__all__ = ["prefill_chunked", "prefill_varlen", "decode_step", "workspace_size", "load",
           "KdaError"]
