"""Seeded synthetic inputs for decode-step attention over a paged KV cache.

This package draws random numbers, builds block tables and stores values in
their storage formats (float32, bfloat16 bits, float8-e4m3fn bits).  It holds
none of the attention arithmetic, so the CPU oracle and the HIP path can both
take their inputs from it without sharing any of the method's code.
"""

from .configs import (  # noqa: F401
    DTYPES,
    PagedDecodeInputs,
    make_inputs,
    named_config,
    CONFIG_NAMES,
)
