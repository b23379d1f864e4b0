"""Seeded synthetic inputs for the quantized linear layer.

This module only draws random numbers and shapes them; it holds none of the
quantization arithmetic.  Both the CPU oracle's tests and the HIP path's tests
and benchmark consume these arrays, so the two sides always see the same
bytes.
"""

from .inputs import *  # noqa: F401,F403
