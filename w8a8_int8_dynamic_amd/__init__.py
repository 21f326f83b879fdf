"""W8A8 int8-dynamic linear layers on MI355X (gfx950).

The compute path is libw8a8.so (hand-written HIP kernels behind the C ABI in
include/w8a8.h). This package is its thin Python binding: ``ops`` wraps each
entry point for torch tensors, ``W8A8Linear`` is the layer and
``quantize_linear_layers`` swaps it into a model. Importing the
package loads the library and raises if it has not been built.
"""
from . import _lib
from ._lib import W8A8Error

_lib.lib()   # fail at import time when the HIP library is missing

from . import ops  # noqa: E402
from .linear import W8A8Linear, quantize_linear_layers  # noqa: E402

__all__ = ["ops", "W8A8Linear", "W8A8Error", "quantize_linear_layers"]
