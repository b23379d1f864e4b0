"""Plain CPU oracle for the quantized linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only the test suite, the entry point's ``smoke()`` check
and the benchmark's CPU-baseline leg use it.  It shares no code, header,
table or constant generator with the HIP library; the two meet only in the
seeded synthetic inputs.

Each function is written from the pages' definitions (cited per function by
page title and section) as slow, direct numpy / pure-Python code:

* ``formats``  -- floating-point value tables built from the generic float
  formula, nearest-value encoders (round half to even, saturating), bf16/fp16
  rounding.
* ``intquant`` -- group-wise INT4/INT8 symmetric and asymmetric quantization,
  nibble packing, dequantization.
* ``fp8``      -- per-row FP8 E4M3 quantization (weights per output channel and
  dynamic per-token activations).
* ``mx``       -- OCP MXFP4: 32-element blocks, shared E8M0 exponent, E2M1 codes.
* ``gemm``     -- fp64 reference products of the dequantized operands, the
  relative Frobenius error metric, a pure-Python brute-force product, SiLU
  and the SwiGLU reference over the quantized gate+up concatenation.
* ``norm``     -- LayerNorm / RMSNorm followed by per-row dynamic
  quantization.
* ``smooth``   -- SmoothQuant channel statistics, smoothing factors and the
  quantization of smoothed operands.
* ``kvcache``  -- FP8 E4M3 KV-cache quantization (per token and head, or
  static per channel) into a paged cache through a slot mapping.

Every function here is pinned by a ``-m "not gpu"`` test against something
other than itself (values printed on the pages, a library routine, exact
rational arithmetic, closed forms, invariants or brute force); no function is
parity-unpinned.
"""

from . import formats, intquant, fp8, mx, gemm, norm, smooth, kvcache  # noqa: F401
