"""MI355X-native forward pass of a Qwen3-0.6B-shaped decoder (prefill + greedy decode).

The work runs in libq3.so (gfx950 HIP kernels behind the C ABI in
include/q3.h).  This package is the Python binding: `Q3Model` marshals
arguments and borrows torch device memory and streams.  There is no CPU
fallback; constructing a model without the built library raises.
"""
from ._lib import (LIB_PATH, Q3_BF16, Q3_F32, Q3_MAX_BATCH, Q3Error, EXPORTS,  # noqa: F401
                   load)
from .engine import Q3Model, checkpoint_validate, make_config  # noqa: F401
