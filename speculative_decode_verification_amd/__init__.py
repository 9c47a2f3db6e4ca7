"""Exact k-row speculative-verification kernels for AMD Instinct MI355X.

The compute path is libsdv.so (HIP kernels for gfx950 behind the C ABI in
include/sdv.h); ``ops`` marshals torch tensors into those calls and
``pipeline`` composes them into one verification step.  Importing this
package does not load the library; the first call does, and fails loudly
if it has not been built.
"""

from ._lib import (ACT_BF16, ACT_F32, MAX_ROWS, MODE_GATEUP_SWIGLU, MODE_PLAIN, ROUTE_SIGMOID,
                   ROUTE_SOFTMAX, SdvError, LIB_PATH)

__all__ = ["ACT_BF16", "ACT_F32", "MAX_ROWS", "MODE_GATEUP_SWIGLU", "MODE_PLAIN", "ROUTE_SIGMOID",
           "ROUTE_SOFTMAX", "SdvError", "LIB_PATH"]
